"""GPU checks of the selection handling around the attention calls: the validity counts of
mla_check_topk against the oracle's count (integer work: exact), and queries left with no allowed
key, which every attention form writes as zeros while the other rows keep their values."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import attention_close, dev, say, to_dev, to_host

mla = pytest.importorskip("sparse_latent_attention_wkv_amd")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]

SCALE = oracle.softmax_scale()
f32 = synth.bf16_bits_to_f32


def _messy(seed, B, T, K, empty_rows=()):
    """The workload recipe, then repeated entries, -1 holes, out-of-range and later positions,
    and some rows with no allowed entry at all."""
    topk = synth.random_topk(seed, B, T, K)
    rng = np.random.default_rng(seed)
    flat = topk.reshape(-1)
    n = flat.size
    for frac, fn in ((0.05, lambda k: flat[rng.integers(0, n, k)]),
                     (0.05, lambda k: np.full(k, -1)),
                     (0.03, lambda k: rng.integers(T, T + 50, k)),
                     (0.03, lambda k: rng.integers(-100, -1, k))):
        k = int(frac * n)
        flat[rng.integers(0, n, k)] = fn(k)
    s = np.arange(T)[None, :, None]
    late = rng.random(topk.shape) < 0.05
    topk[late] = np.minimum(T - 1, s + 1 + rng.integers(0, 5, topk.shape))[late]
    for i, r in enumerate(empty_rows):
        b = i % B
        kind = i % 3
        if kind == 0:
            topk[b, r] = -1
        elif kind == 1:
            topk[b, r] = np.minimum(T - 1, r + 1 + np.arange(K))   # only later positions
            if r == T - 1:
                topk[b, r] = T + np.arange(K)
        else:
            topk[b, r] = T + 7                                     # only out-of-range entries
    return topk.astype(np.int32)


@pytest.mark.parametrize("name,B,T,K,empty", [("clean tiny", 1, 64, 16, ()),
                                              ("messy", 2, 300, 40, (0, 5, 77, 150, 299)),
                                              ("K > T", 1, 45, 300, (3,)),
                                              ("odd K", 3, 257, 37, (10, 11, 12, 256)),
                                              ("long rows", 1, 4096, 2048, (4095,))])
def test_check_topk_counts(name, B, T, K, empty):
    topk = _messy(700 + T, B, T, K, empty) if name != "clean tiny" else synth.random_topk(700, B, T, K)
    say(f"check_topk {name} B={B} T={T} K={K}")
    got = mla.mla_check_topk(torch.from_numpy(topk).to(dev()))
    want = oracle.topk_defects(topk, T)
    say(f"  counts {got}")
    assert got == want
    if empty:
        assert got["empty_rows"] >= len(empty)


def test_check_topk_clean_headline_selection():
    topk = synth.make("headline", ("topk",))["topk"]
    got = mla.mla_check_topk(torch.from_numpy(topk).to(dev()))
    assert got == {"invalid": 0, "future": 0, "repeated": 0, "empty_rows": 0}


def _self_filled(topk):
    """The same selection with every empty row given its own position (so the oracle, which
    rejects empty rows, can compute the other rows)."""
    allowed = oracle.selection_mask(topk, topk.shape[1])
    fixed = topk.copy()
    for b, s in np.argwhere(~allowed.any(-1)):
        fixed[b, s, 0] = s
    return fixed, ~allowed.any(-1)


def test_empty_rows_give_zeros_head_major_and_latent():
    B, T, K = 2, 300, 40
    topk = _messy(7300, B, T, K, (0, 1, 5, 77, 150, 255, 256, 299))
    fixed, empty = _self_filled(topk)
    assert empty.sum() >= 8
    q = synth.random_bf16(7301, (B, T, 128, 192))
    c_kv = synth.random_bf16(7302, (B, T, 512))
    k_pe = synth.random_bf16(7303, (B, T, 64))
    w = synth.random_bf16(7304, (32768, 512), std=512 ** -0.5)
    tk = torch.from_numpy(topk).to(dev())
    qd, cd, pd, wd = to_dev(q), to_dev(c_kv), to_dev(k_pe), to_dev(w)
    kv = mla.mla_kv_up(cd, wd)
    out_hm = to_host(mla.mla_sparse_prefill_attn(qd, kv, pd, tk, SCALE))
    out_lat = to_host(mla.mla_sparse_prefill_attn_latent(qd, cd, pd, wd, tk, SCALE))
    torch.cuda.synchronize()
    for name, got in (("head-major", out_hm), ("latent", out_lat)):
        assert np.isfinite(got).all(), name
        assert (got[empty] == 0).all(), f"{name}: empty rows not zero"
    # the other rows keep the values of the same selection without the empty rows
    ref = oracle.sparse_prefill_attn(f32(q), to_host(kv), f32(k_pe), fixed, SCALE)
    attention_close(out_hm[~empty], ref[~empty], "head-major, non-empty rows")
    ref_x = oracle.sparse_prefill_attn(f32(q), oracle.kv_up(f32(c_kv), f32(w), rounded=False), f32(k_pe),
                                       fixed, SCALE)
    attention_close(out_lat[~empty], ref_x[~empty], "latent, non-empty rows")


def test_empty_rows_give_zeros_split_form():
    B, T, K = 1, 1100, 100
    split = mla.mla_attn_auto_split(T, K)
    assert 0 < split < T
    topk = _messy(7400, B, T, K, (3, split - 1, split, split + 7, T - 1))
    fixed, empty = _self_filled(topk)
    q = synth.random_bf16(7401, (B, T, 128, 192))
    c_kv = synth.random_bf16(7402, (B, T, 512))
    k_pe = synth.random_bf16(7403, (B, T, 64))
    w = synth.random_bf16(7404, (32768, 512), std=512 ** -0.5)
    got = to_host(mla.mla_sparse_prefill_attn_auto(to_dev(q), to_dev(c_kv), to_dev(k_pe), to_dev(w),
                                                   torch.from_numpy(topk).to(dev()), SCALE))
    torch.cuda.synchronize()
    assert np.isfinite(got).all()
    assert (got[empty] == 0).all()
    keep = ~empty
    keep_lo, keep_hi = keep.copy(), keep.copy()
    keep_lo[:, split:] = False
    keep_hi[:, :split] = False
    ref = oracle.sparse_prefill_attn(f32(q), oracle.kv_up(f32(c_kv), f32(w)), f32(k_pe), fixed, SCALE)
    attention_close(got[keep_lo], ref[keep_lo], "split form, head-major rows")
    ref_x = oracle.sparse_prefill_attn(f32(q), oracle.kv_up(f32(c_kv), f32(w), rounded=False), f32(k_pe),
                                       fixed, SCALE)
    attention_close(got[keep_hi], ref_x[keep_hi], "split form, latent rows")


def test_kv_latent_binding_checks_caller_outputs():
    x = torch.zeros((1, 8, 7168), dtype=torch.bfloat16, device=dev())
    w = torch.zeros((576, 7168), dtype=torch.bfloat16, device=dev())
    g = torch.ones(512, dtype=torch.float32, device=dev())
    good = (torch.empty((1, 8, 576), dtype=torch.bfloat16, device=dev()),
            torch.empty((1, 8, 512), dtype=torch.bfloat16, device=dev()),
            torch.empty((1, 8, 64), dtype=torch.bfloat16, device=dev()))
    mla.mla_kv_latent(x, w, g, 1e-6, out=good)
    short = (good[0], torch.empty((1, 4, 512), dtype=torch.bfloat16, device=dev()), good[2])
    with pytest.raises(ValueError):
        mla.mla_kv_latent(x, w, g, 1e-6, out=short)
    strided = (good[0], good[1], torch.empty((1, 8, 128), dtype=torch.bfloat16, device=dev())[..., ::2])
    with pytest.raises(ValueError):
        mla.mla_kv_latent(x, w, g, 1e-6, out=strided)
    wrong_type = (good[0].float(), good[1], good[2])
    with pytest.raises(TypeError):
        mla.mla_kv_latent(x, w, g, 1e-6, out=wrong_type)
