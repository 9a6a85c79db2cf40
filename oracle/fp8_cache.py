"""Plain CPU oracle for the FP8 round trip of the latent, the key-value cache writes and the
V4.1 window-KV front end.

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or run it. It shares no code with the
GPU library and imports nothing from it.

Sources:
* "DeepSeek-V3.2-Exp · Key-value down-projection", KV-cache evidence: two per-layer buffers of
  max_seq_len positions (the normalised latent and the rotary key); each call rounds the
  latent through FP8 in blocks of ``block_size`` = 128 (quantise, then multiply the fp8 values
  by their block's scale in float and cast back), then stores both at its positions.
* "DeepSeek V4.1 · Key-value RMSNorm", window-KV excerpt: normalise (eps 1e-20), rotate the
  tail of the normalised vector in place, quantise the whole vector (rotary tail included),
  then seed a ring buffer of ``window`` positions (prefill) or write one slot (decode).

Readings where the pages are silent (each is listed in the design notes):
* The quantiser's body is not on the pages. Reading: the fp8 format is e4m3 in its finite-only
  variant (4 exponent bits, bias 7, 3 mantissa bits, largest value 448, no infinities); per
  block of 128 features the scale is s = amax / 448 in float32 (``scale_fmt`` "fp32"), or that
  value rounded up to a power of two (``scale_fmt`` "ue8m0", a scale that is a bare 8-bit
  exponent); the code is the e4m3 value nearest to x / s (float32 division), ties to the even
  code. A block of zeros keeps scale 1 and stays zero.
* The caches hold the dequantised bfloat16 values, as the excerpt stores them.
* V4.1's rotary width and pair convention are not on the pages: the last 64 features, adjacent
  pairs, as for the V3.2 shared key; positions are start_pos + i.
* V4.1's decode branch writes one token; this oracle follows both branches as written and
  requires S = 1 when start_pos > 0.

Pins: ``tests/test_oracle_fp8.py``.
"""
from __future__ import annotations

import numpy as np

from .mla_oracle import (KV_LORA_RANK, QK_ROPE_HEAD_DIM, RMS_EPS_DEFAULT, RMS_EPS_WINDOW,
                         ROPE_THETA, bf16, kv_down, rms_norm, rope_angles, rotary)

FP8_BLOCK = 128        # block_size of the KV-cache evidence (module-level constant, value 128)
SCALE_FMTS = ("fp32", "ue8m0")


def e4m3_values() -> np.ndarray:
    """All non-negative finite e4m3 values, indexed by their 7-bit code (sign bit clear),
    from the format's definition: exponent field e (4 bits, bias 7) and mantissa m (3 bits);
    e = 0 encodes m/8 * 2^-6, e > 0 encodes (1 + m/8) * 2^(e-7); the code with every bit set
    (e = 15, m = 7) is not a number. 127 values, 0 to 448."""
    vals = []
    for code in range(127):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m / 8.0 * 2.0 ** -6)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, np.float64)


_E4M3 = e4m3_values()
E4M3_MAX = float(_E4M3[-1])


def e4m3_round(y) -> np.ndarray:
    """Nearest e4m3 value to each y, ties to the even code.

    Looks the magnitude up in the table of codes: the two neighbouring codes bracket it; the
    nearer wins, and at an exact midpoint the code whose last bit is 0. Above 448 the next
    step of the format's grid (480) is the not-a-number code, so magnitudes up to the midpoint
    464 round to 448 and larger ones are refused. (x / s can exceed 448 by a rounding of the
    division when s = amax / 448.)"""
    y = np.asarray(y, np.float64)
    a = np.abs(y)
    if np.any(a > E4M3_MAX + 16.0) or not np.all(np.isfinite(y)):
        raise ValueError("e4m3_round: input outside [-464, 464]")
    hi = np.searchsorted(_E4M3, a, side="left")           # first code with value >= a
    hi = np.minimum(hi, len(_E4M3) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3[lo]
    dhi = _E4M3[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    return np.copysign(_E4M3[code], y)


def fp8_scale(amax, scale_fmt: str = "fp32") -> np.ndarray:
    """Per-block scale from the block's largest magnitude (float32 result).

    "fp32": s = amax / 448 rounded to float32 (float32 division). "ue8m0": the smallest power
    of two >= that value. amax = 0 gives 1 (the block is all zeros and stays so)."""
    if scale_fmt not in SCALE_FMTS:
        raise ValueError(f"scale_fmt must be one of {SCALE_FMTS}")
    amax = np.asarray(amax, np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    if scale_fmt == "ue8m0":
        f, e = np.frexp(s.astype(np.float64))                # s = f * 2^e, 0.5 <= f < 1
        s = np.where(f == 0.5, s.astype(np.float64), np.ldexp(1.0, e)).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def fp8_round_trip(x, scale_fmt: str = "fp32", block: int = FP8_BLOCK, return_parts=False):
    """Quantise the last axis of x (bfloat16 values) to e4m3 in blocks of ``block`` features
    and bring it back: q = e4m3(float32(x / s)), result = bf16(float32(q * s)), s the block's
    scale (KV-cache evidence: quantise with block_size, view as [-1, block_size], multiply by
    the per-block scale in float, cast back to the model dtype)."""
    x = np.asarray(x, np.float32)
    n = x.shape[-1]
    if n % block:
        raise ValueError("feature width must be a multiple of the block size")
    xb = x.reshape(-1, block)
    s = fp8_scale(np.max(np.abs(xb), axis=-1), scale_fmt)[:, None]       # [nblocks, 1]
    y = (xb / s).astype(np.float32)                                        # float32 division
    q = e4m3_round(y).astype(np.float32)                                   # exact in float32
    deq = bf16((q * s).astype(np.float32)).reshape(x.shape)
    if return_parts:
        return deq, q.reshape(x.shape), s.reshape(x.shape[:-1] + (n // block,))
    return deq


# --- f2: V3.2 front end with the FP8 round trip and the cache writes --------------------------
def kv_latent_cache(x, w_dkv, gain, kv_cache, pe_cache, start_pos: int = 0,
                    eps: float = RMS_EPS_DEFAULT, scale_fmt: str = "fp32",
                    theta: float = ROPE_THETA):
    """The latent front end for positions start_pos .. start_pos+T-1, then the FP8 round trip
    of the normalised latent and the writes of both caches (KV-cache evidence).

    x [B, T, 7168]; kv_cache [Bc, L, 512], pe_cache [Bc, L, 64] (copies are returned; Bc >= B,
    L >= start_pos + T). Returns kv_raw, c_norm (before the round trip), c_kv (after it: what
    the up-projection consumes and the cache holds), k_pe, kv_cache, pe_cache."""
    kv_raw = kv_down(x, w_dkv)
    B, T, _ = kv_raw.shape
    c, pe = kv_raw[..., :KV_LORA_RANK], kv_raw[..., KV_LORA_RANK:]
    c_norm = rms_norm(c, gain, eps)
    k_pe = rotary(pe, rope_angles(start_pos + np.arange(T), pe.shape[-1], theta))
    c_kv = fp8_round_trip(c_norm, scale_fmt)
    kv_cache, pe_cache = cache_write(c_kv, k_pe, kv_cache, pe_cache, start_pos)
    return kv_raw, c_norm, c_kv, k_pe, kv_cache, pe_cache


def cache_write(c_kv, k_pe, kv_cache, pe_cache, start_pos: int):
    """kv_cache[:B, start_pos:start_pos+T] = c_kv and pe_cache[...] = k_pe on copies."""
    kv_cache = np.array(kv_cache, np.float32, copy=True)
    pe_cache = np.array(pe_cache, np.float32, copy=True)
    B, T, _ = c_kv.shape
    if kv_cache.shape[0] < B or kv_cache.shape[1] < start_pos + T or start_pos < 0:
        raise ValueError("cache too small for these positions")
    kv_cache[:B, start_pos:start_pos + T] = c_kv
    pe_cache[:B, start_pos:start_pos + T] = k_pe
    return kv_cache, pe_cache


# --- f4: V4.1 window keys/values --------------------------------------------------------------
def window_kv(kv_raw, gain, window_cache, start_pos: int = 0, eps: float = RMS_EPS_WINDOW,
              scale_fmt: str = "fp32", rope_dim: int = QK_ROPE_HEAD_DIM,
              theta: float = ROPE_THETA):
    """V4.1 window keys/values from the 512-wide projection output kv_raw [B, S, 512]:
    RMSNorm (eps 1e-20 by default), rotary on the last ``rope_dim`` features at positions
    start_pos + i, FP8 round trip of the whole vector, then the ring-buffer writes as the
    excerpt's two branches write them. window_cache [Bc, W, 512] (a copy is returned).

    Returns (kv_pre, kv, window_cache): the vector before the round trip, after it, and the
    updated ring buffer."""
    kv_raw = np.asarray(kv_raw, np.float32)
    B, S, D = kv_raw.shape
    cache = np.asarray(window_cache, np.float32)
    if cache.shape[0] < B or cache.shape[2] != D:
        raise ValueError("window cache shape does not fit")
    y = rms_norm(kv_raw, gain, eps)
    tail = rotary(y[..., D - rope_dim:], rope_angles(start_pos + np.arange(S), rope_dim, theta))
    pre = y.copy()
    pre[..., D - rope_dim:] = tail
    kv = fp8_round_trip(pre, scale_fmt)
    return pre, kv, ring_write(kv, cache, start_pos)


def ring_write(kv, window_cache, start_pos: int):
    """The window-KV excerpt's two ring-buffer branches on a copy of window_cache [Bc, W, D]:
    prefill (start_pos 0) stores all S positions if S <= W, else the last W split at S mod W;
    decode stores its one position at slot start_pos mod W."""
    kv = np.asarray(kv, np.float32)
    cache = np.array(window_cache, np.float32, copy=True)
    B, S, _ = kv.shape
    W = cache.shape[1]
    if start_pos == 0:
        if S <= W:
            cache[:B, :S] = kv
        else:
            cutoff = S % W
            last = kv[:, -W:]
            cache[:B, cutoff:W] = last[:, :W - cutoff]
            cache[:B, :cutoff] = last[:, W - cutoff:]
    else:
        if S != 1:
            raise ValueError("the decode branch writes one position")
        cache[:B, start_pos % W] = kv[:, 0]
    return cache
