"""Seeded synthetic inputs for the sparse latent-attention prefill.

This module draws random numbers and stores them; it computes no step of the attention path.
Both the CPU oracle and the GPU library are fed from here, so the two sides see identical
bits. Everything is drawn with NumPy's PCG64 from one seed per workload; every tensor gets
its own ``SeedSequence`` child, and large tensors are filled in fixed-size chunks (each with
its own grandchild seed) so the values do not depend on how many threads fill them.

Storage formats
---------------
* bfloat16 tensors are returned as ``uint16`` bit patterns (the upper half of the IEEE
  float32 pattern, rounded to nearest-even from the float32 draw).
* The learned RMSNorm gain is returned as ``float32`` holding bfloat16-representable values.
* Top-k selections are ``int32`` key positions, ``-1`` marking an empty slot.

Distributions (the workloads' own wording: "N(0, v)" names a normal with variance v):

========  ==========================  ==============================
tensor    shape                       distribution
========  ==========================  ==============================
x         [B, T, 7168]                N(0, 1)
w_dkv     [576, 7168]  ([out, in])    N(0, 1/7168)
w_ukv     [128*256, 512]              N(0, 1/512)
q         [B, T, 128, 192]            N(0, 1)
gain      [512]                       1 + N(0, 0.1), rounded to bf16
kv_raw    [rows, 512] (decode only)   N(0, 1)
topk      [B, T, K]                   see :func:`topk_rows`
========  ==========================  ==============================
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Model dimensions of the V3.2-Exp latent attention (down-projection, keys and value-head pages).
HIDDEN = 7168
KV_LORA = 512
ROPE = 64
KV_A_OUT = KV_LORA + ROPE          # 576 rows of the joint down-projection
HEADS = 128
QK_NOPE = 128
QK_HEAD = QK_NOPE + ROPE           # 192
V_HEAD = 128
KV_B_OUT = HEADS * (QK_NOPE + V_HEAD)   # 32768

_CHUNK = 1 << 22                   # elements per independently seeded chunk

# Per-tensor child index inside a workload's SeedSequence.
_STREAM = {"x": 0, "w_dkv": 1, "w_ukv": 2, "q": 3, "gain": 4, "topk": 5, "kv_raw": 6}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    K: int | None
    seed: int
    eps: float = 1e-6
    rope: bool = True
    note: str = ""


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 16, 1001, note="tiny full prefill, top-k 16"),
    "1k": Workload("1k", 1, 1024, 256, 1002, note="single sequence, top-k 256"),
    "headline": Workload("headline", 2, 4096, 2048, 1003, note="B=2, T=4096, top-k 2048"),
    "long": Workload("long", 1, 16384, 2048, 1004, note="T=16384 (max_seq_len), top-k 2048"),
    "frontend": Workload("frontend", 8, 4096, None, 1005, note="latent front end only"),
    "decode": Workload("decode", 256, 1, None, 1006, eps=1e-20, rope=False,
                       note="window-KV decode norm: 256 rows of 512, eps 1e-20"),
}


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return uint16 patterns.

    Input preparation only (normal draws are finite, so no NaN handling is needed)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen uint16 bfloat16 patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(ss: np.random.SeedSequence, shape, std: float, mean: float = 0.0) -> np.ndarray:
    """Chunked, thread-count-independent N(mean, std^2) draws rounded to bf16 bits."""
    n = int(np.prod(shape))
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)
    children = ss.spawn(nchunks)
    out = np.empty(n, np.uint16)

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(children[i]))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if mean != 0.0:
            v += np.float32(mean)
        out[lo:hi] = f32_to_bf16_bits(v)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def topk_rows(rng: np.random.Generator, B: int, T: int, K: int) -> np.ndarray:
    """Synthetic indexer output standing in for the learned top-k selector.

    Row s of batch b holds k_s = min(K, s+1) distinct positions in [0, s], always including
    s itself: when k_s = s+1 the row is all of [0, s]; otherwise s plus k_s-1 distinct
    uniform draws from [0, s-1]. Each row is shuffled and padded to K with -1.
    """
    out = np.full((B, T, K), -1, np.int32)
    for b in range(B):
        for s in range(T):
            k = min(K, s + 1)
            if k == s + 1:
                row = rng.permutation(s + 1)
            else:
                row = np.empty(k, np.int64)
                row[0] = s
                row[1:] = rng.choice(s, k - 1, replace=False)
                rng.shuffle(row)
            out[b, s, :k] = row
    return out


def _child(w: Workload, name: str) -> np.random.SeedSequence:
    return np.random.SeedSequence(w.seed).spawn(len(_STREAM))[_STREAM[name]]


def make(w: Workload | str, parts=None) -> dict:
    """Draw the requested tensors of a workload (all of its tensors when ``parts`` is None)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if parts is None:
        if w.name == "decode":
            parts = ("kv_raw", "gain")
        elif w.K is None:
            parts = ("x", "w_dkv", "gain")
        else:
            parts = ("x", "w_dkv", "gain", "w_ukv", "q", "topk")
    out = {}
    for p in parts:
        ss = _child(w, p)
        if p == "x":
            out[p] = _normal_bf16(ss, (w.B, w.T, HIDDEN), 1.0)
        elif p == "w_dkv":
            out[p] = _normal_bf16(ss, (KV_A_OUT, HIDDEN), float(np.sqrt(1.0 / HIDDEN)))
        elif p == "w_ukv":
            out[p] = _normal_bf16(ss, (KV_B_OUT, KV_LORA), float(np.sqrt(1.0 / KV_LORA)))
        elif p == "q":
            out[p] = _normal_bf16(ss, (w.B, w.T, HEADS, QK_HEAD), 1.0)
        elif p == "gain":
            out[p] = bf16_bits_to_f32(_normal_bf16(ss, (KV_LORA,), float(np.sqrt(0.1)), 1.0))
        elif p == "kv_raw":
            out[p] = _normal_bf16(ss, (w.B * w.T, KV_LORA), 1.0)
        elif p == "topk":
            if w.K is None:
                raise ValueError(f"workload {w.name} has no selection")
            out[p] = topk_rows(np.random.Generator(np.random.PCG64(ss)), w.B, w.T, w.K)
        else:
            raise KeyError(p)
    return out


def random_bf16(seed: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """Ad-hoc seeded bf16 draws (tests use this for shapes outside the named workloads)."""
    return _normal_bf16(np.random.SeedSequence(seed), tuple(shape), std, mean)


def random_topk(seed: int, B: int, T: int, K: int) -> np.ndarray:
    """Ad-hoc seeded selection with the same recipe as :func:`topk_rows`."""
    return topk_rows(np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed))), B, T, K)
