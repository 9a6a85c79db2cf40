"""GPU parity of the latent-space attention (mla_sparse_prefill_attn_latent), of the split form
(mla_sparse_prefill_attn_auto) and of the sorted selection lists they run on, against the CPU
oracle.

The latent form regroups the pages' products (queries absorbed into the latent, values mixed in
the latent) and never forms the per-head keys and values, so it does not round them. Its
reference is the pages' arithmetic with that rounding left out: oracle.kv_up(..., rounded=False)
followed by oracle.sparse_prefill_attn, held to the attention bound (rel-L2 <= 1e-2 and max-abs
<= 2e-2). The pages' order, which rounds the values of every head before mixing them, is also
reported and held to rel-L2 <= 1e-2: by itself that rounding moves some outputs of few-key
queries by one bf16 step of 2^-5 (a CPU pin shows it on exact arithmetic), which no regrouping
can reproduce. Rows of the split form below the split take the head-major path and are held to
the bound against the pages' order. The lists are integer work: bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import assert_within_one_step, bf16_step, dev, fp32_dot_bound, say, to_dev, to_host
from _gpu import attention_close as strict_attention_close

mla = pytest.importorskip("sparse_latent_attention_wkv_amd")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]

SCALE = oracle.softmax_scale()
f32 = synth.bf16_bits_to_f32


def latent_close(got, ref_exact, ref_pages, what=""):
    """The attention bound against the unrounded form; rel-L2 against the pages' order."""
    strict_attention_close(got, ref_exact, what)
    d = np.asarray(got, np.float64) - ref_pages
    rel = np.linalg.norm(d) / max(np.linalg.norm(ref_pages), 1e-30)
    say(f"  {what} against the pages' rounded values: rel-L2 {rel:.3e}, max-abs {np.abs(d).max():.3e}")
    assert rel <= 1e-2, f"{what}: rel-L2 against the pages' order {rel}"


# ------------------------------------------------------------------------------------ lists
def _messy_topk(seed, B, T, K):
    """The workload recipe, then repeated entries, -1 holes, positions past the query and past T."""
    topk = synth.random_topk(seed, B, T, K)
    rng = np.random.default_rng(seed)
    n = topk.size
    flat = topk.reshape(-1)
    for frac, fn in ((0.05, lambda k: flat[rng.integers(0, n, k)]),   # duplicates of other entries
                     (0.05, lambda k: np.full(k, -1)),
                     (0.03, lambda k: rng.integers(T, T + 50, k)),
                     (0.03, lambda k: rng.integers(-100, -1, k))):
        k = int(frac * n)
        flat[rng.integers(0, n, k)] = fn(k)
    # entries beyond the query position (removed by the causal mask)
    s = np.arange(T)[None, :, None]
    late = rng.random(topk.shape) < 0.05
    topk[late] = np.minimum(T - 1, s + 1 + rng.integers(0, 5, topk.shape))[late]
    return topk.astype(np.int32)


@pytest.mark.parametrize("B,T,K,messy", [(1, 1, 1, False), (1, 64, 16, False), (2, 300, 40, True),
                                         (1, 1000, 1000, False), (3, 777, 100, True),
                                         (1, 4096, 2048, False), (1, 2000, 3000, True)])
def test_selection_lists(B, T, K, messy):
    say(f"lists B={B} T={T} K={K} messy={messy}")
    topk = _messy_topk(900 + T, B, T, K) if messy else synth.random_topk(900 + T, B, T, K)
    lists, counts = mla.mla_selection_lists(torch.from_numpy(topk).to(dev()))
    lists, counts = lists.cpu().numpy(), counts.cpu().numpy()
    allowed = oracle.selection_mask(topk, T)
    L = lists.shape[2]
    assert L == (min(T, K) + 63) // 64 * 64
    for b in range(B):
        for s in range(T):
            want = np.nonzero(allowed[b, s])[0]
            n = len(want)
            assert counts[b, s] == n, (b, s)
            assert np.array_equal(lists[b, s, :n], want), (b, s)
            assert not lists[b, s, n:(n + 63) // 64 * 64].any(), (b, s)


# ------------------------------------------------------------------------------------ attention
def _latent_inputs(seed, B, T, K):
    q = synth.random_bf16(seed, (B, T, 128, 192))
    c_kv = synth.random_bf16(seed + 1, (B, T, 512))
    k_pe = synth.random_bf16(seed + 2, (B, T, 64))
    w = synth.random_bf16(seed + 3, (32768, 512), std=512 ** -0.5)
    topk = synth.random_topk(seed + 4, B, T, K)
    return q, c_kv, k_pe, w, topk


def _run_latent(q, c_kv, k_pe, w, topk):
    out = mla.mla_sparse_prefill_attn_latent(to_dev(q), to_dev(c_kv), to_dev(k_pe), to_dev(w),
                                             torch.from_numpy(topk).to(dev()), SCALE)
    torch.cuda.synchronize()
    return to_host(out)


def _oracle(q, c_kv, k_pe, w, topk):
    """(rounded kv, output of the pages' order, output without the kv rounding)."""
    kv = oracle.kv_up(f32(c_kv), f32(w))
    kv_x = oracle.kv_up(f32(c_kv), f32(w), rounded=False)
    return (kv, oracle.sparse_prefill_attn(f32(q), kv, f32(k_pe), topk, SCALE),
            oracle.sparse_prefill_attn(f32(q), kv_x, f32(k_pe), topk, SCALE))


# (1, 1100, 300): tiles of 32 keys with a ragged last tile for most rows; (1, 333, 400): K > T;
# (3, 130, 7): several sequences and a top-k below one tile.
@pytest.mark.parametrize("B,T,K", [(1, 1, 1), (1, 64, 16), (2, 200, 48), (1, 333, 400), (3, 130, 7),
                                   (1, 1100, 300)])
def test_latent_attention_matches_oracle(B, T, K):
    say(f"latent attention B={B} T={T} K={K}")
    q, c_kv, k_pe, w, topk = _latent_inputs(5000 + T + K, B, T, K)
    got = _run_latent(q, c_kv, k_pe, w, topk)
    kv, ref, ref_x = _oracle(q, c_kv, k_pe, w, topk)
    latent_close(got, ref_x, ref, f"latent B{B} T{T} K{K}")
    # query 0 sees only key 0: the output is W_UV applied to that latent row, i.e. the value row
    # of the pages' form up to the fp32 summation order
    wv = f32(w).reshape(128, 256, 512)[:, 128:, :].astype(np.float64)
    bound = fp32_dot_bound(np.abs(wv) @ np.abs(f32(c_kv)[:, 0].astype(np.float64)).T, 512)   # [128, 128, B]
    assert_within_one_step(got[:, 0], kv[:, :, 0, 128:], extra=bound.transpose(2, 0, 1), what="query 0")


def test_latent_attention_full_selection_is_dense_causal():
    B, T = 1, 300
    q, c_kv, k_pe, w, _ = _latent_inputs(5100, B, T, 1)
    topk = np.tile(np.arange(T, dtype=np.int32), (B, T, 1))
    got = _run_latent(q, c_kv, k_pe, w, topk)
    _, ref, ref_x = _oracle(q, c_kv, k_pe, w, topk)
    latent_close(got, ref_x, ref, "latent full selection")


def test_latent_attention_exact_max_path():
    """A key whose scores exceed the first tile's max by far more than 2^64 in weight: the kernel
    marks those queries and recomputes them with their exact max (no overflow)."""
    B, T, K = 1, 200, 200
    q, c_kv, k_pe, w, topk = _latent_inputs(5200, B, T, K)
    kpe = f32(k_pe)
    kpe[0, 150] = 60.0                       # rotary part of key 150: scores of order +-60 per unit
    k_pe = synth.f32_to_bf16_bits(kpe)
    got = _run_latent(q, c_kv, k_pe, w, topk)
    _, ref, ref_x = _oracle(q, c_kv, k_pe, w, topk)
    latent_close(got, ref_x, ref, "latent exact-max path")


def _latent_rows_ref(q, c_kv, k_pe, w, topk, b, rows, rounded=False):
    """Oracle for sampled query rows of a large workload: each row's allowed keys alone, as a
    compact problem (the keys renumbered 0..n-1 in order, the query last). q: bf16 bits indexed
    q[b, s] (an array, or any object with that indexing). ``rounded``: the pages' order (keys and
    values rounded to bf16) instead of the unrounded form."""
    res = []
    wf = f32(w)
    for s in rows:
        ids = np.asarray(topk[b, s]).astype(np.int64)
        ids = np.unique(ids[(ids >= 0) & (ids <= s)])
        n = len(ids)
        kv_c = oracle.kv_up(f32(c_kv[b:b + 1, ids]), wf, rounded=rounded)    # [1, H, n, 256]
        q_c = np.zeros((1, n, 128, 192), np.float32)
        q_c[0, n - 1] = f32(q[b, s])
        topk_c = np.full((1, n, n), -1, np.int32)
        topk_c[0, n - 1] = np.arange(n)
        res.append(oracle.sparse_prefill_attn_rows(q_c, kv_c, f32(k_pe[b:b + 1, ids]), topk_c, SCALE, 0,
                                                   [n - 1])[0])
    return np.stack(res)


@pytest.mark.parametrize("name", ["headline", "long"])
def test_latent_workload_sampled(name):
    w = synth.WORKLOADS[name]
    say(f"workload {name}: drawing inputs")
    d = synth.make(w)
    say(f"workload {name}: front end and latent attention")
    x, wd, wu, q = to_dev(d["x"]), to_dev(d["w_dkv"]), to_dev(d["w_ukv"]), to_dev(d["q"])
    gain = torch.from_numpy(d["gain"]).to(dev())
    topk = torch.from_numpy(d["topk"]).to(dev())
    _, c_kv, k_pe = mla.mla_kv_latent(x, wd, gain, 1e-6)
    out = mla.mla_sparse_prefill_attn_latent(q, c_kv, k_pe, wu, topk, SCALE)
    out2 = mla.mla_sparse_prefill_attn_latent(q, c_kv, k_pe, wu, topk, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "latent attention is not deterministic"
    ckv_bits = c_kv.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    kpe_bits = k_pe.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    rng = np.random.default_rng(41)
    T, K = w.T, w.K
    for b in range(w.B):
        rows = sorted(set([0, 1, 31, 32, 33, K - 1, K, T - 1] + rng.integers(0, T, 4).tolist()))
        say(f"checking {len(rows)} sampled rows of batch {b}")
        ref_x = _latent_rows_ref(d["q"], ckv_bits, kpe_bits, d["w_ukv"], d["topk"], b, rows)
        ref = _latent_rows_ref(d["q"], ckv_bits, kpe_bits, d["w_ukv"], d["topk"], b, rows, rounded=True)
        latent_close(to_host(out[b, rows]), ref_x, ref, f"{name} batch {b}")


# ------------------------------------------------------------------------------------ split form
# (1, 1100, 100): split 256 (rows 0-255 head-major, 256-1099 latent); (2, 700, 64): split 256 with
# two sequences; (1, 300, 40): split 0 (all latent); (1, 200, 2048): split = T (all head-major).
@pytest.mark.parametrize("B,T,K", [(1, 1100, 100), (2, 700, 64), (1, 300, 40), (1, 200, 2048)])
def test_auto_attention_matches_oracle(B, T, K):
    split = mla.mla_attn_auto_split(T, K)
    say(f"split form B={B} T={T} K={K} split={split}")
    q, c_kv, k_pe, w, topk = _latent_inputs(5300 + T + K, B, T, K)
    out = mla.mla_sparse_prefill_attn_auto(to_dev(q), to_dev(c_kv), to_dev(k_pe), to_dev(w),
                                           torch.from_numpy(topk).to(dev()), SCALE)
    torch.cuda.synchronize()
    got = to_host(out)
    _, ref, ref_x = _oracle(q, c_kv, k_pe, w, topk)
    # rows below the split: head-major path on rounded keys and values; the rest: latent form
    if split > 0:
        strict_attention_close(got[:, :split], ref[:, :split], f"split form B{B} T{T} K{K}, head-major rows")
    if split < T:
        latent_close(got[:, split:], ref_x[:, split:], ref[:, split:], f"split form B{B} T{T} K{K}, latent rows")


def test_auto_long_workload_sampled():
    w = synth.WORKLOADS["long"]
    d = synth.make(w)
    x, wd, wu, q = to_dev(d["x"]), to_dev(d["w_dkv"]), to_dev(d["w_ukv"]), to_dev(d["q"])
    gain = torch.from_numpy(d["gain"]).to(dev())
    topk = torch.from_numpy(d["topk"]).to(dev())
    _, c_kv, k_pe = mla.mla_kv_latent(x, wd, gain, 1e-6)
    out = mla.mla_sparse_prefill_attn_auto(q, c_kv, k_pe, wu, topk, SCALE)
    torch.cuda.synchronize()
    split = mla.mla_attn_auto_split(w.T, w.K)
    assert 0 < split < w.T
    ckv_bits = c_kv.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    kpe_bits = k_pe.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    lo, hi = [0, 1, split - 256, split - 1], [split, split + 1, w.T - 1]
    say(f"split {split}: checking rows {lo + hi}")
    got = to_host(out[0, lo + hi])
    ref = _latent_rows_ref(d["q"], ckv_bits, kpe_bits, d["w_ukv"], d["topk"], 0, lo + hi, rounded=True)
    ref_x = _latent_rows_ref(d["q"], ckv_bits, kpe_bits, d["w_ukv"], d["topk"], 0, hi)
    strict_attention_close(got[:len(lo)], ref[:len(lo)], "long split form, head-major rows")
    latent_close(got[len(lo):], ref_x, ref[len(lo):], "long split form, latent rows")


class _Rows:
    """q[b, s] for a few rows copied from a device tensor (the full query does not fit the
    oracle's host memory comfortably at the longest length)."""

    def __init__(self, q_dev, rows):
        self.rows = {int(s): q_dev[0, int(s)].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                     for s in rows}

    def __getitem__(self, key):
        return self.rows[int(key[1])]


def test_longest_sequence_auto_and_head_major():
    """T = MLA_MAX_T (32768), top-k 2048: the split form (head-major rows below the split,
    latent rows above) and the head-major path alone, on sampled rows of both ranges."""
    B, T, K = 1, 32768, 2048
    say(f"longest sequence B={B} T={T} K={K}: inputs")
    topk = synth.random_topk(4700, B, T, K)
    ckv_bits = synth.random_bf16(4701, (B, T, 512))
    kpe_bits = synth.random_bf16(4702, (B, T, 64))
    w = synth.random_bf16(4703, (32768, 512), std=512 ** -0.5)
    gen = torch.Generator(device=dev()).manual_seed(4704)
    q = torch.randn((B, T, 128, 192), generator=gen, device=dev()).to(torch.bfloat16)
    c_kv, k_pe, wu = to_dev(ckv_bits), to_dev(kpe_bits), to_dev(w)
    tk = torch.from_numpy(topk).to(dev())
    split = mla.mla_attn_auto_split(T, K)
    assert 0 < split < T
    say(f"  split form (split {split})")
    out = mla.mla_sparse_prefill_attn_auto(q, c_kv, k_pe, wu, tk, SCALE)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4705)
    rows = sorted(set([0, 1, K - 1, split - 1, split, T - 2, T - 1] + rng.integers(0, T, 3).tolist()))
    qr = _Rows(q, rows)
    got = to_host(out[0, rows])
    ref = _latent_rows_ref(qr, ckv_bits, kpe_bits, w, topk, 0, rows, rounded=True)
    ref_x = _latent_rows_ref(qr, ckv_bits, kpe_bits, w, topk, 0, rows)
    below = np.asarray(rows) < split
    strict_attention_close(got[below], ref[below], "longest sequence, split form, head-major rows")
    latent_close(got[~below], ref_x[~below], ref[~below], "longest sequence, split form, latent rows")
    say("  head-major path")
    kv = mla.mla_kv_up(c_kv, wu)
    out_hm = mla.mla_sparse_prefill_attn(q, kv, k_pe, tk, SCALE)
    torch.cuda.synchronize()
    # reference from the GPU's own keys and values (the head-major criterion of the pages'
    # tolerances: rel-L2 <= 1e-2, max-abs <= 2e-2)
    ref_hm = []
    for s_ in rows:
        ids = np.asarray(topk[0, s_]).astype(np.int64)
        ids = np.unique(ids[(ids >= 0) & (ids <= s_)])
        n = len(ids)
        kv_c = to_host(kv[0][:, torch.from_numpy(ids).to(dev())])[None]        # [1, H, n, 256]
        q_c = np.zeros((1, n, 128, 192), np.float32)
        q_c[0, n - 1] = f32(qr[0, s_])
        topk_c = np.full((1, n, n), -1, np.int32)
        topk_c[0, n - 1] = np.arange(n)
        ref_hm.append(oracle.sparse_prefill_attn_rows(q_c, kv_c, f32(kpe_bits[0:1, ids]), topk_c,
                                                      SCALE, 0, [n - 1])[0])
    strict_attention_close(to_host(out_hm[0, rows]), np.stack(ref_hm), "longest sequence, head-major")
