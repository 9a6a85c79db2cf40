"""Plain CPU oracle for the DeepSeek-V3.2-Exp sparse latent-attention prefill.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import or run this module. It shares no code with the GPU library and
imports nothing from it; the GPU product path never calls it.

What it computes (sources are the five model-atlas pages: "DeepSeek V4.1 · Key-value
RMSNorm", "DeepSeek-V3.2-Exp · Key-value down-projection", "DeepSeek-V3.2-Exp · Keys",
"DeepSeek-V3.2-Exp · Scale scores" and "DeepSeek-V3.2-Exp · Split value heads"):

1. ``kv_down``      joint key-value down-projection, x -> 512 latent + 64 rotary key
                    (down-projection page: formula c = x W_DKV, and the MLA key-value code excerpt).
2. ``rms_norm``     fp32 RMSNorm with learned gain (Key-value RMSNorm page: formula and the
                    RMSNorm class excerpt).
3. ``rotary``       rotation of the shared 64-wide key, adjacent pairs as complex numbers
                    (down-projection page, code excerpt calling the rotary helper; the helper's
                    body is not on the pages, the pair convention is the workload's).
4. ``kv_up``        up-projection to 128 heads of [128 key | 128 value] features, head-major
                    (Keys page, MHA-prefill excerpt; Split value heads page: [B,T,16384] ->
                    [B,128,T,128]).
5. ``sparse_prefill_attn``  scores over [k_nope | k_pe] times m^2/sqrt(192), top-k selection
                    intersected with the causal mask, softmax over keys, value mixing
                    (Keys page, MHA-prefill excerpt; Scale scores page formula).

Precision. The pages fix fp32 only for the RMSNorm (the input is widened to float before the
mean of squares). Everything else here runs in float64 and is rounded once to bfloat16
(nearest, ties to even) wherever the pages' module stores an output in the model dtype:
the down-projection output, the normalised latent, the rotated key, the up-projection output
and the attention output. Inputs are float arrays holding bfloat16-representable values.

Readings where the pages are silent (each is listed in the design notes):
* ``topk`` is ``[B, T, K]`` int32; entries outside [0, T) (in particular -1 padding) select
  nothing; repeated entries select once (the excerpt's scatter has set semantics).
* The causal mask allows key t for query s iff t <= s (prefill from position 0).
* A query whose allowed set is empty is outside the contract: the oracle raises.
* Rotary: pair i = (2i, 2i+1) rotated by pos * 10000^(-2i/64), pos = token index; no YaRN
  frequency correction (its formula is not on the pages); q arrives already rotated.

Every function has pins in ``tests/test_oracle_*.py`` that check it against facts that do not
come from this file (printed constants, closed forms, library routines, brute force).
"""
from __future__ import annotations

import math

import numpy as np

# --- model dimensions (MLA init excerpt; Keys page shape; Split value heads page) ----------
HIDDEN = 7168
KV_LORA_RANK = 512
QK_ROPE_HEAD_DIM = 64
QK_NOPE_HEAD_DIM = 128
QK_HEAD_DIM = QK_NOPE_HEAD_DIM + QK_ROPE_HEAD_DIM   # 192
V_HEAD_DIM = 128
N_HEADS = 128

# --- model-args defaults (Keys page, model-args excerpt) ------------------------------------
MAX_SEQ_LEN = 4096 * 4
ORIGINAL_SEQ_LEN = 4096
ROPE_THETA = 10000.0
ROPE_FACTOR = 40.0
MSCALE = 1.0
RMS_EPS_DEFAULT = 1e-6      # RMSNorm class default; the V3.2 kv_norm is built without an eps
RMS_EPS_WINDOW = 1e-20      # Key-value RMSNorm page formula (V4.1 window keys/values)

_BF16_MAX = float.fromhex("0x1.fep127")   # largest finite bfloat16


def parameter_shapes() -> dict:
    """Shapes of the latent-path parameters as the MLA init excerpt builds them.

    ``wkv_a`` maps dim -> kv_lora_rank + qk_rope_head_dim and is stored [out, in] (the
    down-projection page: the module holds the weight output by input); ``kv_norm`` owns one
    gain per latent feature; ``wkv_b`` maps the latent to n_heads * (nope + value) features.
    """
    return {
        "wkv_a": (KV_LORA_RANK + QK_ROPE_HEAD_DIM, HIDDEN),
        "kv_norm": (KV_LORA_RANK,),
        "wkv_b": (N_HEADS * (QK_NOPE_HEAD_DIM + V_HEAD_DIM), KV_LORA_RANK),
    }


def softmax_scale(qk_head_dim: int = QK_HEAD_DIM, max_seq_len: int = MAX_SEQ_LEN,
                  original_seq_len: int = ORIGINAL_SEQ_LEN, rope_factor: float = ROPE_FACTOR,
                  mscale: float = MSCALE) -> float:
    """Score scale: qk_head_dim^-1/2, times m^2 with m = 1 + 0.1*mscale*ln(rope_factor) when
    the maximum length exceeds the original one (MLA init excerpt; Scale scores page formula
    S' = S * m^2 / sqrt(192), m = 1 + 0.1 ln 40)."""
    s = qk_head_dim ** -0.5
    if max_seq_len > original_seq_len:
        m = 0.1 * mscale * math.log(rope_factor) + 1.0
        s = s * m * m
    return s


def bf16(a) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even, directly from float64 (no detour
    through float32, which would round twice). Returns float32 (exact for every bfloat16).

    bfloat16 keeps 8 significant bits and float32's exponent range; below 2^-126 the spacing
    stays 2^-133 (subnormals). Magnitudes that round past the largest finite value give inf.
    """
    a = np.asarray(a, dtype=np.float64)
    out = a.copy()
    fin = np.isfinite(a)
    v = a[fin]
    _, ex = np.frexp(v)                       # v = f * 2^ex, 0.5 <= |f| < 1
    qexp = np.maximum(ex - 8, -133)           # exponent of one unit in the last place
    r = np.ldexp(np.round(np.ldexp(v, -qexp)), qexp)   # np.round: half to even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[fin] = r
    return out.astype(np.float32)


# --- 1. joint key-value down-projection --------------------------------------------------------
def kv_down(x, w_dkv) -> np.ndarray:
    """kv_raw = x W^T with W stored [out=576, in=7168] (down-projection page: formula and the
    Linear excerpt, weight [out, in], no bias). float64 products and sums, one bf16 rounding.
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w_dkv, np.float64)
    if x.shape[-1] != w.shape[1]:
        raise ValueError("x feature width does not match W_DKV's input width")
    return bf16(x @ w.T)


# --- 2. latent RMSNorm ---------------------------------------------------------------------------
def rms_norm(c, gain, eps: float = RMS_EPS_DEFAULT) -> np.ndarray:
    """y = gain * x / sqrt(mean(x^2) + eps) over the last axis, in float32, cast back to bf16
    (Key-value RMSNorm page: formula for m_2 and y, and the RMSNorm forward, which widens to
    float, takes the mean of squares, multiplies by rsqrt(var + eps), then by the gain)."""
    x = np.asarray(c, np.float32)
    g = np.asarray(gain, np.float32)
    if g.shape != x.shape[-1:]:
        raise ValueError("gain length must equal the normalised width")
    var = np.mean(np.square(x), axis=-1, keepdims=True, dtype=np.float32)
    r = np.float32(1.0) / np.sqrt(var + np.float32(eps))
    y = (x * r).astype(np.float32)
    return bf16((g * y).astype(np.float32))


# --- 3. rotary rotation of the shared key ----------------------------------------------------------
def rope_angles(positions, dim: int = QK_ROPE_HEAD_DIM, theta: float = ROPE_THETA) -> np.ndarray:
    """phi[p, i] = pos_p * theta^(-2i/dim), i < dim/2, in float64."""
    pos = np.asarray(positions, np.float64)
    i = np.arange(dim // 2, dtype=np.float64)
    return np.multiply.outer(pos, theta ** (-2.0 * i / dim))


def rotary(pe, angles) -> np.ndarray:
    """Rotate adjacent pairs (2i, 2i+1) of the last axis, read as re + j*im, by angles[..., i]
    (complex multiply by e^{j phi}); float64, one bf16 rounding. ``angles`` broadcasts against
    pe[..., ::2]."""
    pe = np.asarray(pe, np.float64)
    re, im = pe[..., 0::2], pe[..., 1::2]
    c, s = np.cos(angles), np.sin(angles)
    out = np.empty_like(pe)
    out[..., 0::2] = re * c - im * s
    out[..., 1::2] = re * s + im * c
    return bf16(out)


def kv_latent(x, w_dkv, gain, eps: float = RMS_EPS_DEFAULT, theta: float = ROPE_THETA):
    """Down-projection, split [512 | 64], latent RMSNorm, rotary on the shared key with
    pos = t (MLA key-value code excerpt on the down-projection page).

    x: [B, T, 7168]. Returns kv_raw [B, T, 576], c_kv [B, T, 512], k_pe [B, T, 64]."""
    kv_raw = kv_down(x, w_dkv)
    c, pe = kv_raw[..., :KV_LORA_RANK], kv_raw[..., KV_LORA_RANK:]
    c_kv = rms_norm(c, gain, eps)
    T = kv_raw.shape[-2]
    k_pe = rotary(pe, rope_angles(np.arange(T), pe.shape[-1], theta))
    return kv_raw, c_kv, k_pe


# --- 4. key-value up-projection --------------------------------------------------------------------
def kv_up(c_kv, w_ukv, n_heads: int = N_HEADS, rounded: bool = True) -> np.ndarray:
    """kv[b, h, t, :] = bf16(c_kv[b, t] @ W_UKV^T)[h*256:(h+1)*256]; features 0..127 of a head
    are its non-rotary key, 128..255 its value (MHA-prefill excerpt: view to
    [B, T, heads, 256] then split [128, 128]; Keys and Split value heads pages: head-major
    shapes [B, 128, T, .]). Returns [B, H, T, 256] float32 (bf16 values).

    ``rounded=False`` returns the float64 products without the bf16 rounding. The per-head
    keys and values are a stored module output only where something stores them; a
    computation that regroups the products around the latent never forms them, and its
    reference is the same arithmetic with this rounding left out (float64 result)."""
    c = np.asarray(c_kv, np.float64)
    w = np.asarray(w_ukv, np.float64)
    B, T, _ = c.shape
    per = w.shape[0] // n_heads
    out = np.empty((B, n_heads, T, per), np.float32 if rounded else np.float64)
    for b in range(B):
        y = c[b] @ w.T                             # [T, H*per]
        if rounded:
            y = bf16(y)
        out[b] = y.reshape(T, n_heads, per).transpose(1, 0, 2)
    return out


# --- 5. sparse attention over the selection -------------------------------------------------------
def selection_mask(topk, T: int) -> np.ndarray:
    """allowed[b, s, t]: key t is one of query s's top-k entries and t <= s.

    The MHA-prefill excerpt scatters 0 into a -inf [B, T, T] mask at the top-k positions and
    adds the causal mask; this is the boolean form of that sum."""
    topk = np.asarray(topk)
    B, Tq, K = topk.shape
    if Tq != T:
        raise ValueError("topk must have one row per query")
    allowed = np.zeros((B, T, T), dtype=bool)
    rows = np.repeat(np.arange(T), K)
    for b in range(B):
        cols = topk[b].reshape(-1).astype(np.int64)
        ok = (cols >= 0) & (cols < T)
        allowed[b, rows[ok], cols[ok]] = True
    allowed &= np.tril(np.ones((T, T), dtype=bool))
    return allowed


def topk_defects(topk, T: int) -> dict:
    """Counts over a selection [B, T, K] of the entries the index mask reads in a special way
    (MHA-prefill excerpt: the indexer's indices are scattered into a -inf mask, which gives
    repeated indices set semantics, and the causal mask removes later positions; -1 marks an
    empty slot in this library's reading of the index format):
    ``invalid`` entries outside [-1, T), ``future`` entries t with s < t < T, ``repeated``
    occurrences of an allowed entry after its first in the row, ``empty_rows`` queries whose
    allowed set is empty."""
    topk = np.asarray(topk).astype(np.int64)
    B, Tq, K = topk.shape
    if Tq != T:
        raise ValueError("topk must have one row per query")
    s = np.arange(T)[None, :, None]
    invalid = (topk < -1) | (topk >= T)
    future = (topk > s) & (topk < T)
    allowed_entry = (topk >= 0) & (topk <= s)
    n_allowed = int(allowed_entry.sum())
    distinct = selection_mask(topk, T).sum(axis=-1)          # [B, T]
    return {"invalid": int(invalid.sum()), "future": int(future.sum()),
            "repeated": n_allowed - int(distinct.sum()), "empty_rows": int((distinct == 0).sum())}


def _keys(kv, k_pe, b, h):
    k = np.concatenate([np.asarray(kv[b, h, :, :QK_NOPE_HEAD_DIM], np.float64),
                        np.asarray(k_pe[b], np.float64)], axis=-1)        # [T, 192]
    v = np.asarray(kv[b, h, :, QK_NOPE_HEAD_DIM:], np.float64)            # [T, 128]
    return k, v


def sparse_prefill_attn(q, kv, k_pe, topk, scale: float, heads=None, block: int = 1024,
                        return_probs: bool = False):
    """out[b, s, h] = sum_t P[b, s, h, t] v[b, h, t] with
    P = softmax_t(scale * q[b, s, h] . [k_nope[b, h, t] | k_pe[b, t]] + mask[b, s, t]),
    mask = 0 on the allowed set and -inf elsewhere (MHA-prefill excerpt: concatenated keys,
    score einsum times the softmax scale, scattered index mask plus causal mask broadcast over
    heads, softmax over keys, value einsum).

    Written as the pages write it: dense scores over all T keys, with the mask added. Each
    (b, h) and each block of query rows is evaluated on its own; a row's softmax always sees
    all T of its keys. float64 throughout, one bf16 rounding of the output.

    q: [B, T, H, 192]; kv: [B, H, T, 256]; k_pe: [B, T, 64]; topk: [B, T, K].
    ``heads`` restricts the computation to some heads (others are left zero).
    Returns out [B, T, H, 128] (and P [B, T, H, T] in float64 when ``return_probs``).
    """
    q = np.asarray(q)
    B, T, H, D = q.shape
    if D != QK_HEAD_DIM or kv.shape != (B, H, T, QK_NOPE_HEAD_DIM + V_HEAD_DIM) \
            or k_pe.shape != (B, T, QK_ROPE_HEAD_DIM):
        raise ValueError("q / kv / k_pe shapes do not agree")
    allowed = selection_mask(topk, T)
    if not allowed.any(axis=-1).all():
        raise ValueError("a query has an empty allowed set (outside the contract)")
    mask = np.where(allowed, 0.0, -np.inf)
    out = np.zeros((B, T, H, V_HEAD_DIM), np.float32)
    probs = np.zeros((B, T, H, T)) if return_probs else None
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            k, v = _keys(kv, k_pe, b, h)
            for s0 in range(0, T, block):
                s1 = min(T, s0 + block)
                qs = np.asarray(q[b, s0:s1, h], np.float64)
                scores = (qs @ k.T) * scale + mask[b, s0:s1]
                scores = scores - scores.max(axis=-1, keepdims=True)
                e = np.exp(scores)
                p = e / e.sum(axis=-1, keepdims=True)
                out[b, s0:s1, h] = bf16(p @ v)
                if return_probs:
                    probs[b, s0:s1, h] = p
    return (out, probs) if return_probs else out


def sparse_prefill_attn_rows(q, kv, k_pe, topk, scale: float, b: int, rows) -> np.ndarray:
    """The same result for selected query rows only, evaluated over each row's own allowed
    keys (no dense T-wide scores), all heads at once. Used to check large workloads on a
    sample of outputs. Returns [len(rows), H, 128] float32 (bf16 values)."""
    q = np.asarray(q)
    _, T, H, _ = q.shape
    res = np.empty((len(rows), H, V_HEAD_DIM), np.float32)
    for n, s in enumerate(rows):
        ids = np.asarray(topk[b, s]).astype(np.int64)
        ids = np.unique(ids[(ids >= 0) & (ids < T) & (ids <= s)])
        if ids.size == 0:
            raise ValueError("a query has an empty allowed set (outside the contract)")
        k_nope = np.asarray(kv[b][:, ids, :QK_NOPE_HEAD_DIM], np.float64)     # [H, n, 128]
        v = np.asarray(kv[b][:, ids, QK_NOPE_HEAD_DIM:], np.float64)          # [H, n, 128]
        pe = np.asarray(k_pe[b, ids], np.float64)                             # [n, 64]
        qs = np.asarray(q[b, s], np.float64)                                   # [H, 192]
        sc = np.einsum("hd,hnd->hn", qs[:, :QK_NOPE_HEAD_DIM], k_nope) \
            + qs[:, QK_NOPE_HEAD_DIM:] @ pe.T
        sc = sc * scale
        sc = sc - sc.max(axis=-1, keepdims=True)
        e = np.exp(sc)
        p = e / e.sum(axis=-1, keepdims=True)
        res[n] = bf16(np.einsum("hn,hnd->hd", p, v))
    return res


def mla_prefill(x, w_dkv, gain, w_ukv, q, topk, scale: float, eps: float = RMS_EPS_DEFAULT):
    """The whole path: latent front end, up-projection, sparse attention."""
    kv_raw, c_kv, k_pe = kv_latent(x, w_dkv, gain, eps)
    kv = kv_up(c_kv, w_ukv)
    out = sparse_prefill_attn(q, kv, k_pe, topk, scale)
    return {"kv_raw": kv_raw, "c_kv": c_kv, "k_pe": k_pe, "kv": kv, "out": out}
