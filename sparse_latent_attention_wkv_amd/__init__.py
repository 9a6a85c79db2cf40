"""MI355X (gfx950) sparse latent-attention prefill: Python binding of libmla.so.

The functions below carry the names of the C entry points in ``include/mla.h`` and only
marshal arguments: they check dtypes, shapes, devices and contiguity of torch tensors, allocate
outputs with ``torch.empty`` on the input's device, and call the library on the current torch
stream. Every step of the computation runs in the library's HIP kernels; there is no fallback.
If ``libmla.so`` has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MLA_LIBRARY names another build of the same library (the host-sanitizer build of the checks
# uses it); by default the in-tree libmla.so.
LIB_PATH = os.environ.get("MLA_LIBRARY") or os.path.join(_PKG, "libmla.so")

HIDDEN, KV_LORA, ROPE, KV_A_OUT = 7168, 512, 64, 576
HEADS, QK_NOPE, QK_HEAD, V_HEAD = 128, 128, 192, 128
Q_LORA = 1536
KV_B_OUT = HEADS * (QK_NOPE + V_HEAD)

_lib = None

_VP, _I, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "mla_kv_latent": (_I, [_VP, _VP, _VP, _F, _VP, _I, _I, _VP, _VP, _VP, _VP]),
    "mla_kv_norm_rope": (_I, [_VP, _I, _I, _I, _VP, _F, _VP, _I, _VP, _VP, _VP]),
    "mla_rope_table": (_I, [_I, _F, _VP, _VP]),
    "mla_kv_latent_cache": (_I, [_VP, _VP, _VP, _F, _VP, _I, _I, _I, _I, _VP, _VP, _VP, _VP, _VP,
                                 _I, _I, _VP, _VP]),
    "mla_kv_norm_rope_cache": (_I, [_VP, _I, _I, _I, _VP, _F, _VP, _I, _VP, _VP, _VP, _VP, _I, _I,
                                    _VP, _VP]),
    "mla_window_kv": (_I, [_VP, _I, _I, _I, _VP, _F, _VP, _I, _I, _VP, _VP, _I, _VP, _VP]),
    "mla_q_path": (_I, [_VP, _VP, _VP, _F, _VP, _VP, _I, _I, _I, _I, _VP, _VP, _VP, _VP]),
    "mla_kv_up": (_I, [_VP, _VP, _I, _I, _VP, _VP]),
    "mla_attn_workspace_bytes": (_SZ, [_I, _I, _I]),
    "mla_selection_bitmap": (_I, [_VP, _I, _I, _I, _VP, _VP]),
    "mla_sparse_prefill_attn": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _F, _VP, _VP, _SZ, _VP]),
    "mla_attn_prepare": (_I, [_VP, _I, _I, _I, _VP, _SZ, _VP]),
    "mla_sparse_prefill_attn_prepared": (_I, [_VP, _VP, _VP, _I, _I, _F, _VP, _VP, _SZ, _VP]),
    "mla_check_topk": (_I, [_VP, _I, _I, _I, _VP, _VP]),
    "mla_sparse_prefill_attn_noalloc": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _F, _VP, _VP]),
    "mla_noalloc_scratch_bytes": (_SZ, [_I, _I]),
    "mla_selection_list_stride": (_I, [_I, _I]),
    "mla_selection_lists": (_I, [_VP, _I, _I, _I, _VP, _VP, _VP]),
    "mla_attn_latent_workspace_bytes": (_SZ, [_I, _I, _I]),
    "mla_sparse_prefill_attn_latent": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _F, _VP, _VP, _SZ, _VP]),
    "mla_attn_auto_split": (_I, [_I, _I]),
    "mla_attn_auto_workspace_bytes": (_SZ, [_I, _I, _I]),
    "mla_sparse_prefill_attn_auto": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _F, _VP, _VP, _SZ, _VP]),
    "mla_default_softmax_scale": (_F, []),
    "mla_status_string": (ctypes.c_char_p, [_I]),
    "mla_last_hip_error": (_I, []),
    "mla_build_info": (ctypes.c_char_p, []),
}


class MLAError(RuntimeError):
    pass


def lib():
    """The loaded libmla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MLAError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_latent_attention_wkv_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _check(status: int):
    if status != 0:
        msg = lib().mla_status_string(status).decode()
        if status == -6:
            msg += f" (hipError {lib().mla_last_hip_error()})"
        raise MLAError(msg)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def mla_default_softmax_scale() -> float:
    return float(lib().mla_default_softmax_scale())


def mla_attn_workspace_bytes(B: int, T: int, K: int) -> int:
    return int(lib().mla_attn_workspace_bytes(B, T, K))


def mla_rope_table(T: int, device, theta: float = 10000.0) -> torch.Tensor:
    """(cos, sin) table [T, 32, 2] fp32 for positions 0..T-1."""
    out = torch.empty((T, 32, 2), dtype=torch.float32, device=device)
    with torch.cuda.device(out.device):
        _check(lib().mla_rope_table(T, theta, _ptr(out), _stream(out.device)))
    return out


def mla_kv_latent(x, w_dkv, kv_gain, eps: float = 1e-6, rope_cs=None, out=None):
    """x [B, T, 7168] bf16 -> (kv_raw [B, T, 576], c_kv [B, T, 512], k_pe [B, T, 64]) bf16."""
    if x.dim() != 3:
        raise ValueError("x must be [B, T, 7168]")
    B, T, _ = x.shape
    _need(x, "x", torch.bfloat16, (B, T, HIDDEN))
    _need(w_dkv, "w_dkv", torch.bfloat16, (KV_A_OUT, HIDDEN))
    _need(kv_gain, "kv_gain", torch.float32, (KV_LORA,))
    if rope_cs is None:
        rope_cs = mla_rope_table(T, x.device)
    _need(rope_cs, "rope_cs", torch.float32, (T, 32, 2))
    if out is None:
        out = (torch.empty((B, T, KV_A_OUT), dtype=torch.bfloat16, device=x.device),
               torch.empty((B, T, KV_LORA), dtype=torch.bfloat16, device=x.device),
               torch.empty((B, T, ROPE), dtype=torch.bfloat16, device=x.device))
    kv_raw, c_kv, k_pe = out
    _need(kv_raw, "kv_raw", torch.bfloat16, (B, T, KV_A_OUT))
    _need(c_kv, "c_kv", torch.bfloat16, (B, T, KV_LORA))
    _need(k_pe, "k_pe", torch.bfloat16, (B, T, ROPE))
    with torch.cuda.device(x.device):
        _check(lib().mla_kv_latent(_ptr(x), _ptr(w_dkv), _ptr(kv_gain), eps, _ptr(rope_cs), B, T,
                                   _ptr(kv_raw), _ptr(c_kv), _ptr(k_pe), _stream(x.device)))
    return kv_raw, c_kv, k_pe


def mla_kv_norm_rope(kv_raw, gain, eps: float = 1e-6, rope_cs=None, T: int | None = None, out=None):
    """kv_raw [rows, 576] (latent + rotary key) or [rows, 512] (latent only) bf16 ->
    (c_kv [rows, 512], k_pe [rows, 64] or None). Row r is at position r % T for the rotary.
    `out` = (c_kv, k_pe) reuses caller buffers."""
    if kv_raw.dim() != 2:
        raise ValueError("kv_raw must be 2-D [rows, 576 or 512]")
    rows, stride = kv_raw.shape
    _need(kv_raw, "kv_raw", torch.bfloat16)
    _need(gain, "gain", torch.float32, (KV_LORA,))
    has_rope = rope_cs is not None
    if out is not None:
        c_kv, k_pe = out
        _need(c_kv, "c_kv", torch.bfloat16, (rows, KV_LORA))
    else:
        c_kv = torch.empty((rows, KV_LORA), dtype=torch.bfloat16, device=kv_raw.device)
        k_pe = None
    if has_rope:
        T = rope_cs.shape[0] if T is None else T
        _need(rope_cs, "rope_cs", torch.float32, (T, 32, 2))
        if k_pe is None:
            k_pe = torch.empty((rows, ROPE), dtype=torch.bfloat16, device=kv_raw.device)
        _need(k_pe, "k_pe", torch.bfloat16, (rows, ROPE))
    else:
        k_pe = None
    with torch.cuda.device(kv_raw.device):
        _check(lib().mla_kv_norm_rope(_ptr(kv_raw), rows, stride, int(has_rope), _ptr(gain), eps,
                                      _ptr(rope_cs), T or 1, _ptr(c_kv), _ptr(k_pe),
                                      _stream(kv_raw.device)))
    return c_kv, k_pe


def _positions_table(rope_cs, start_pos: int, n: int, device):
    if rope_cs is None:
        return mla_rope_table(start_pos + n, device)
    _need(rope_cs, "rope_cs", torch.float32)
    if rope_cs.dim() != 3 or rope_cs.shape[1:] != (32, 2) or rope_cs.shape[0] < start_pos + n:
        raise ValueError(f"rope_cs must be [>= {start_pos + n}, 32, 2] fp32")
    return rope_cs


def _cache_pair(kv_cache, pe_cache, B: int, T: int, start_pos: int):
    _need(kv_cache, "kv_cache", torch.bfloat16)
    _need(pe_cache, "pe_cache", torch.bfloat16)
    if kv_cache.dim() != 3 or kv_cache.shape[2] != KV_LORA:
        raise ValueError("kv_cache must be [cache_batch, cache_len, 512]")
    cb, cl, _ = kv_cache.shape
    if tuple(pe_cache.shape) != (cb, cl, ROPE):
        raise ValueError("pe_cache must be [cache_batch, cache_len, 64] like kv_cache")
    if cb < B or cl < start_pos + T:
        raise ValueError("caches too small for these batch rows and positions")
    return cb, cl


def mla_kv_latent_cache(x, w_dkv, kv_gain, kv_cache, pe_cache, start_pos: int = 0,
                        eps: float = 1e-6, scale_fmt: int = 0, rope_cs=None,
                        want_norm: bool = False):
    """x [B, T, 7168] bf16 at positions start_pos.. -> (kv_raw [B, T, 576], c_kv [B, T, 512]
    rounded through fp8, k_pe [B, T, 64]) bf16, plus c_norm (before the round trip) when
    ``want_norm``; rows start_pos.. of kv_cache [Bc, L, 512] / pe_cache [Bc, L, 64] are
    written in place. scale_fmt 0: fp32 block scale, 1: power-of-two block scale."""
    if x.dim() != 3:
        raise ValueError("x must be [B, T, 7168]")
    B, T, _ = x.shape
    _need(x, "x", torch.bfloat16, (B, T, HIDDEN))
    _need(w_dkv, "w_dkv", torch.bfloat16, (KV_A_OUT, HIDDEN))
    _need(kv_gain, "kv_gain", torch.float32, (KV_LORA,))
    cb, cl = _cache_pair(kv_cache, pe_cache, B, T, start_pos)
    rope_cs = _positions_table(rope_cs, start_pos, T, x.device)
    dev = x.device
    kv_raw = torch.empty((B, T, KV_A_OUT), dtype=torch.bfloat16, device=dev)
    c_kv = torch.empty((B, T, KV_LORA), dtype=torch.bfloat16, device=dev)
    k_pe = torch.empty((B, T, ROPE), dtype=torch.bfloat16, device=dev)
    c_norm = torch.empty((B, T, KV_LORA), dtype=torch.bfloat16, device=dev) if want_norm else None
    with torch.cuda.device(dev):
        _check(lib().mla_kv_latent_cache(_ptr(x), _ptr(w_dkv), _ptr(kv_gain), eps, _ptr(rope_cs),
                                         B, T, start_pos, scale_fmt, _ptr(kv_raw), _ptr(c_kv),
                                         _ptr(k_pe), _ptr(kv_cache), _ptr(pe_cache), cb, cl,
                                         _ptr(c_norm), _stream(dev)))
    return (kv_raw, c_kv, k_pe, c_norm) if want_norm else (kv_raw, c_kv, k_pe)


def mla_kv_norm_rope_cache(kv_raw, gain, kv_cache, pe_cache, start_pos: int = 0,
                           eps: float = 1e-6, scale_fmt: int = 0, rope_cs=None,
                           want_norm: bool = False, out=None):
    """The norm / rotary / fp8 round trip / cache step of mla_kv_latent_cache from
    kv_raw [B, T, 576] bf16 -> (c_kv, k_pe[, c_norm]). `out` = (c_kv, k_pe[, c_norm]) reuses
    caller buffers."""
    if kv_raw.dim() != 3:
        raise ValueError("kv_raw must be [B, T, 576]")
    B, T, _ = kv_raw.shape
    _need(kv_raw, "kv_raw", torch.bfloat16, (B, T, KV_A_OUT))
    _need(gain, "gain", torch.float32, (KV_LORA,))
    cb, cl = _cache_pair(kv_cache, pe_cache, B, T, start_pos)
    rope_cs = _positions_table(rope_cs, start_pos, T, kv_raw.device)
    dev = kv_raw.device
    if out is None:
        out = (torch.empty((B, T, KV_LORA), dtype=torch.bfloat16, device=dev),
               torch.empty((B, T, ROPE), dtype=torch.bfloat16, device=dev),
               torch.empty((B, T, KV_LORA), dtype=torch.bfloat16, device=dev) if want_norm else None)
    c_kv, k_pe = out[0], out[1]
    c_norm = out[2] if len(out) > 2 else None
    _need(c_kv, "c_kv", torch.bfloat16, (B, T, KV_LORA))
    _need(k_pe, "k_pe", torch.bfloat16, (B, T, ROPE))
    if c_norm is not None:
        _need(c_norm, "c_norm", torch.bfloat16, (B, T, KV_LORA))
    with torch.cuda.device(dev):
        _check(lib().mla_kv_norm_rope_cache(_ptr(kv_raw), B, T, start_pos, _ptr(gain), eps,
                                            _ptr(rope_cs), scale_fmt, _ptr(c_kv), _ptr(k_pe),
                                            _ptr(kv_cache), _ptr(pe_cache), cb, cl, _ptr(c_norm),
                                            _stream(dev)))
    return (c_kv, k_pe, c_norm) if c_norm is not None else (c_kv, k_pe)


def mla_window_kv(kv_raw, gain, window_cache, start_pos: int = 0, eps: float = 1e-20,
                  scale_fmt: int = 0, rope_cs=None, want_pre: bool = False, out=None):
    """V4.1 window keys/values: kv_raw [B, S, 512] bf16 -> kv [B, S, 512] (norm, rotary tail,
    fp8 round trip), plus kv_pre (before the round trip) when ``want_pre``; the last
    min(S, window) positions go to slot position % window of window_cache [Bc, window, 512]
    in place. `out` = (kv[, kv_pre]) reuses caller buffers."""
    if kv_raw.dim() != 3:
        raise ValueError("kv_raw must be [B, S, 512]")
    B, S, _ = kv_raw.shape
    _need(kv_raw, "kv_raw", torch.bfloat16, (B, S, KV_LORA))
    _need(gain, "gain", torch.float32, (KV_LORA,))
    _need(window_cache, "window_cache", torch.bfloat16)
    if window_cache.dim() != 3 or window_cache.shape[2] != KV_LORA or window_cache.shape[0] < B:
        raise ValueError("window_cache must be [cache_batch >= B, window, 512]")
    cb, W, _ = window_cache.shape
    rope_cs = _positions_table(rope_cs, start_pos, S, kv_raw.device)
    dev = kv_raw.device
    if out is None:
        out = (torch.empty((B, S, KV_LORA), dtype=torch.bfloat16, device=dev),
               torch.empty((B, S, KV_LORA), dtype=torch.bfloat16, device=dev) if want_pre else None)
    kv = out[0]
    pre = out[1] if len(out) > 1 else None
    _need(kv, "kv", torch.bfloat16, (B, S, KV_LORA))
    if pre is not None:
        _need(pre, "kv_pre", torch.bfloat16, (B, S, KV_LORA))
    with torch.cuda.device(dev):
        _check(lib().mla_window_kv(_ptr(kv_raw), B, S, start_pos, _ptr(gain), eps, _ptr(rope_cs),
                                   scale_fmt, W, _ptr(kv), _ptr(window_cache), cb, _ptr(pre),
                                   _stream(dev)))
    return (kv, pre) if pre is not None else kv


def mla_q_path(x, w_qa, q_gain, w_qb, start_pos: int = 0, eps: float = 1e-6, rope_cs=None,
               out=None):
    """x [B, T, 7168] bf16 -> (qa [B, T, 1536], qr [B, T, 1536], q [B, T, 128, 192]) bf16:
    wq_a, q_norm, wq_b and the rotary of each head's features 128..191 at positions start_pos..
    `out` = (qa, qr, q) reuses caller buffers."""
    if x.dim() != 3:
        raise ValueError("x must be [B, T, 7168]")
    B, T, _ = x.shape
    _need(x, "x", torch.bfloat16, (B, T, HIDDEN))
    _need(w_qa, "w_qa", torch.bfloat16, (Q_LORA, HIDDEN))
    _need(q_gain, "q_gain", torch.float32, (Q_LORA,))
    _need(w_qb, "w_qb", torch.bfloat16, (HEADS * QK_HEAD, Q_LORA))
    rope_cs = _positions_table(rope_cs, start_pos, T, x.device)
    dev = x.device
    if out is None:
        out = (torch.empty((B, T, Q_LORA), dtype=torch.bfloat16, device=dev),
               torch.empty((B, T, Q_LORA), dtype=torch.bfloat16, device=dev),
               torch.empty((B, T, HEADS, QK_HEAD), dtype=torch.bfloat16, device=dev))
    qa, qr, q = out
    _need(qa, "qa", torch.bfloat16, (B, T, Q_LORA))
    _need(qr, "qr", torch.bfloat16, (B, T, Q_LORA))
    _need(q, "q", torch.bfloat16, (B, T, HEADS, QK_HEAD))
    with torch.cuda.device(dev):
        _check(lib().mla_q_path(_ptr(x), _ptr(w_qa), _ptr(q_gain), eps, _ptr(w_qb), _ptr(rope_cs),
                                B, T, start_pos, Q_LORA, _ptr(qa), _ptr(qr), _ptr(q), _stream(dev)))
    return qa, qr, q


def mla_kv_up(c_kv, w_ukv, out=None):
    """c_kv [B, T, 512] bf16 -> kv [B, 128, T, 256] bf16 (per head: 128 key | 128 value)."""
    if c_kv.dim() != 3:
        raise ValueError("c_kv must be [B, T, 512]")
    B, T, _ = c_kv.shape
    _need(c_kv, "c_kv", torch.bfloat16, (B, T, KV_LORA))
    _need(w_ukv, "w_ukv", torch.bfloat16, (KV_B_OUT, KV_LORA))
    if out is None:
        out = torch.empty((B, HEADS, T, QK_NOPE + V_HEAD), dtype=torch.bfloat16, device=c_kv.device)
    _need(out, "out", torch.bfloat16, (B, HEADS, T, QK_NOPE + V_HEAD))
    with torch.cuda.device(c_kv.device):
        _check(lib().mla_kv_up(_ptr(c_kv), _ptr(w_ukv), B, T, _ptr(out), _stream(c_kv.device)))
    return out


def mla_attn_prepare(topk, workspace, stream=None):
    """Selection bitmap for mla_sparse_prefill_attn_prepared, built into `workspace` (uint8,
    at least mla_attn_workspace_bytes(B, T, K) bytes) on `stream` (default: current stream)."""
    if topk.dim() != 3:
        raise ValueError("topk must be [B, T, K]")
    B, T, K = topk.shape
    _need(topk, "topk", torch.int32)
    _need(workspace, "workspace", torch.uint8)
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(topk.device)
    with torch.cuda.device(topk.device):
        _check(lib().mla_attn_prepare(_ptr(topk), B, T, K, _ptr(workspace), workspace.numel(), s))
    return workspace


def mla_sparse_prefill_attn_prepared(q, kv, k_pe, workspace, softmax_scale: float | None = None,
                                     out=None):
    """The attention of mla_sparse_prefill_attn from a workspace mla_attn_prepare filled."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, 128, 192]")
    B, T = q.shape[0], q.shape[1]
    _need(q, "q", torch.bfloat16, (B, T, HEADS, QK_HEAD))
    _need(kv, "kv", torch.bfloat16, (B, HEADS, T, QK_NOPE + V_HEAD))
    _need(k_pe, "k_pe", torch.bfloat16, (B, T, ROPE))
    _need(workspace, "workspace", torch.uint8)
    scale = mla_default_softmax_scale() if softmax_scale is None else softmax_scale
    if out is None:
        out = torch.empty((B, T, HEADS, V_HEAD), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, T, HEADS, V_HEAD))
    with torch.cuda.device(q.device):
        _check(lib().mla_sparse_prefill_attn_prepared(_ptr(q), _ptr(kv), _ptr(k_pe), B, T, scale,
                                                      _ptr(out), _ptr(workspace), workspace.numel(),
                                                      _stream(q.device)))
    return out


def mla_selection_bitmap(topk, out=None):
    """topk [B, T, K] int32 -> bitmap [B, ceil(T/32), T] int32 (bit t%32 of word t/32 of row s).
    `out` reuses a caller buffer of that shape."""
    if topk.dim() != 3:
        raise ValueError("topk must be [B, T, K]")
    B, T, K = topk.shape
    _need(topk, "topk", torch.int32)
    if out is not None:
        bm = out
        _need(bm, "bitmap", torch.int32, (B, (T + 31) // 32, T))
    else:
        bm = torch.empty((B, (T + 31) // 32, T), dtype=torch.int32, device=topk.device)
    with torch.cuda.device(topk.device):
        _check(lib().mla_selection_bitmap(_ptr(topk), B, T, K, _ptr(bm), _stream(topk.device)))
    return bm


def mla_check_topk(topk, out=None):
    """topk [B, T, K] int32 -> dict of counts: entries outside [-1, T) ("invalid"), entries later
    than their query ("future"), repeats of an allowed entry within a row ("repeated"), rows with
    no allowed key ("empty_rows"). Reads the counts back, which waits for the call. `out` reuses
    a device int64 [4] buffer."""
    if topk.dim() != 3:
        raise ValueError("topk must be [B, T, K]")
    B, T, K = topk.shape
    _need(topk, "topk", torch.int32)
    counts = torch.empty(4, dtype=torch.int64, device=topk.device) if out is None else out
    _need(counts, "counts", torch.int64, (4,))
    with torch.cuda.device(topk.device):
        _check(lib().mla_check_topk(_ptr(topk), B, T, K, _ptr(counts), _stream(topk.device)))
    c = counts.cpu().tolist()
    return {"invalid": c[0], "future": c[1], "repeated": c[2], "empty_rows": c[3]}


def mla_sparse_prefill_attn(q, kv, k_pe, topk, softmax_scale: float | None = None,
                            workspace=None, out=None):
    """q [B, T, 128, 192], kv [B, 128, T, 256], k_pe [B, T, 64] bf16, topk [B, T, K] int32 ->
    out [B, T, 128, 128] bf16."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, 128, 192]")
    B, T = q.shape[0], q.shape[1]
    _need(q, "q", torch.bfloat16, (B, T, HEADS, QK_HEAD))
    _need(kv, "kv", torch.bfloat16, (B, HEADS, T, QK_NOPE + V_HEAD))
    _need(k_pe, "k_pe", torch.bfloat16, (B, T, ROPE))
    if topk.dim() != 3 or topk.shape[:2] != (B, T):
        raise ValueError("topk must be [B, T, K]")
    _need(topk, "topk", torch.int32)
    K = topk.shape[2]
    if softmax_scale is None:
        softmax_scale = mla_default_softmax_scale()
    need = mla_attn_workspace_bytes(B, T, K)
    if need == 0:
        raise MLAError("unsupported attention shape")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, T, HEADS, V_HEAD), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, T, HEADS, V_HEAD))
    with torch.cuda.device(q.device):
        _check(lib().mla_sparse_prefill_attn(_ptr(q), _ptr(kv), _ptr(k_pe), _ptr(topk), B, T, K,
                                             softmax_scale, _ptr(out), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(),
                                             _stream(q.device)))
    return out


NOALLOC_SCRATCH_BYTES = (32 << 20) + (128 << 10)


def mla_noalloc_scratch_bytes(B: int, T: int) -> int:
    return int(lib().mla_noalloc_scratch_bytes(B, T))


def mla_sparse_prefill_attn_noalloc(q, kv, k_pe, topk, softmax_scale: float | None = None, out=None):
    """mla_sparse_prefill_attn without a workspace: the library's fixed per-device scratch holds
    the selection bitmap (at most NOALLOC_SCRATCH_BYTES). Pass `out` to avoid any allocation here
    as well. Calls that overlap on one device race on the scratch."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, 128, 192]")
    B, T = q.shape[0], q.shape[1]
    _need(q, "q", torch.bfloat16, (B, T, HEADS, QK_HEAD))
    _need(kv, "kv", torch.bfloat16, (B, HEADS, T, QK_NOPE + V_HEAD))
    _need(k_pe, "k_pe", torch.bfloat16, (B, T, ROPE))
    if topk.dim() != 3 or topk.shape[:2] != (B, T):
        raise ValueError("topk must be [B, T, K]")
    _need(topk, "topk", torch.int32)
    K = topk.shape[2]
    if softmax_scale is None:
        softmax_scale = mla_default_softmax_scale()
    if out is None:
        out = torch.empty((B, T, HEADS, V_HEAD), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, T, HEADS, V_HEAD))
    with torch.cuda.device(q.device):
        _check(lib().mla_sparse_prefill_attn_noalloc(_ptr(q), _ptr(kv), _ptr(k_pe), _ptr(topk), B, T, K,
                                                     softmax_scale, _ptr(out), _stream(q.device)))
    return out


def mla_attn_latent_workspace_bytes(B: int, T: int, K: int) -> int:
    return int(lib().mla_attn_latent_workspace_bytes(B, T, K))


def mla_selection_lists(topk):
    """topk [B, T, K] int32 -> (lists [B, T, L] int32, counts [B, T] int32): the allowed keys of
    each row in increasing order, then zeros up to the next multiple of 64 (the rest of the row is
    left unwritten), L = mla_selection_list_stride(T, K)."""
    if topk.dim() != 3:
        raise ValueError("topk must be [B, T, K]")
    B, T, K = topk.shape
    _need(topk, "topk", torch.int32)
    L = int(lib().mla_selection_list_stride(T, K))
    if L == 0:
        raise MLAError("unsupported selection shape")
    lists = torch.empty((B, T, L), dtype=torch.int32, device=topk.device)
    counts = torch.empty((B, T), dtype=torch.int32, device=topk.device)
    with torch.cuda.device(topk.device):
        _check(lib().mla_selection_lists(_ptr(topk), B, T, K, _ptr(lists), _ptr(counts),
                                         _stream(topk.device)))
    return lists, counts


def mla_sparse_prefill_attn_latent(q, c_kv, k_pe, w_ukv, topk, softmax_scale: float | None = None,
                                   workspace=None, out=None):
    """q [B, T, 128, 192], c_kv [B, T, 512], k_pe [B, T, 64], w_ukv [32768, 512] bf16,
    topk [B, T, K] int32 -> out [B, T, 128, 128] bf16 (latent-space form of the attention)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, 128, 192]")
    B, T = q.shape[0], q.shape[1]
    _need(q, "q", torch.bfloat16, (B, T, HEADS, QK_HEAD))
    _need(c_kv, "c_kv", torch.bfloat16, (B, T, KV_LORA))
    _need(k_pe, "k_pe", torch.bfloat16, (B, T, ROPE))
    _need(w_ukv, "w_ukv", torch.bfloat16, (KV_B_OUT, KV_LORA))
    if topk.dim() != 3 or topk.shape[:2] != (B, T):
        raise ValueError("topk must be [B, T, K]")
    _need(topk, "topk", torch.int32)
    K = topk.shape[2]
    if softmax_scale is None:
        softmax_scale = mla_default_softmax_scale()
    need = mla_attn_latent_workspace_bytes(B, T, K)
    if need == 0:
        raise MLAError("unsupported attention shape")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, T, HEADS, V_HEAD), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, T, HEADS, V_HEAD))
    with torch.cuda.device(q.device):
        _check(lib().mla_sparse_prefill_attn_latent(
            _ptr(q), _ptr(c_kv), _ptr(k_pe), _ptr(w_ukv), _ptr(topk), B, T, K, softmax_scale,
            _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(q.device)))
    return out


def mla_attn_auto_split(T: int, K: int) -> int:
    return int(lib().mla_attn_auto_split(T, K))


def mla_sparse_prefill_attn_auto(q, c_kv, k_pe, w_ukv, topk, softmax_scale: float | None = None,
                                 workspace=None, out=None):
    """As mla_sparse_prefill_attn_latent, with query rows below mla_attn_auto_split(T, K) taking
    the head-major form."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, 128, 192]")
    B, T = q.shape[0], q.shape[1]
    _need(q, "q", torch.bfloat16, (B, T, HEADS, QK_HEAD))
    _need(c_kv, "c_kv", torch.bfloat16, (B, T, KV_LORA))
    _need(k_pe, "k_pe", torch.bfloat16, (B, T, ROPE))
    _need(w_ukv, "w_ukv", torch.bfloat16, (KV_B_OUT, KV_LORA))
    if topk.dim() != 3 or topk.shape[:2] != (B, T):
        raise ValueError("topk must be [B, T, K]")
    _need(topk, "topk", torch.int32)
    K = topk.shape[2]
    if softmax_scale is None:
        softmax_scale = mla_default_softmax_scale()
    need = int(lib().mla_attn_auto_workspace_bytes(B, T, K))
    if need == 0:
        raise MLAError("unsupported attention shape")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, T, HEADS, V_HEAD), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, T, HEADS, V_HEAD))
    with torch.cuda.device(q.device):
        _check(lib().mla_sparse_prefill_attn_auto(
            _ptr(q), _ptr(c_kv), _ptr(k_pe), _ptr(w_ukv), _ptr(topk), B, T, K, softmax_scale,
            _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(q.device)))
    return out
