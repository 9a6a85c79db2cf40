"""Pins for the CPU oracle: every check compares it with something that does not come from
the oracle itself (numbers the pages print, closed forms, library routines, brute force).
CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def bf(seed, shape, std=1.0):
    return synth.bf16_bits_to_f32(synth.random_bf16(seed, shape, std))


# ---------------------------------------------------------------- (a) shapes and parameter counts
def test_parameter_counts_match_printed_accounting():
    shp = oracle.parameter_shapes()
    out, inp = shp["wkv_a"]
    # the page counts the first 512 output rows (the latent) of wkv_a: 7168 x 512
    assert inp * oracle.KV_LORA_RANK == GOLD["wkv_a_latent_params_per_instance"]["value"]
    assert sorted([inp, oracle.KV_LORA_RANK]) == sorted(GOLD["wkv_a_latent_weight_dims"]["value"])
    assert inp * oracle.KV_LORA_RANK * GOLD["moe_blocks"]["value"] == \
        GOLD["wkv_a_latent_params_all_blocks"]["value"]
    assert shp["kv_norm"] == (GOLD["kv_norm_gain_per_instance"]["value"],)
    # the joint projection also emits the 64-wide shared rotary key
    assert out == oracle.KV_LORA_RANK + oracle.QK_ROPE_HEAD_DIM == 576
    # up-projection output splits into 128 heads of 128 key + 128 value features
    assert shp["wkv_b"][0] == GOLD["value_split_in"]["value"][2] * 2
    assert GOLD["value_split_out"]["value"][1] * GOLD["value_split_out"]["value"][3] == \
        GOLD["value_split_in"]["value"][2]
    assert GOLD["key_shape"]["value"][3] == oracle.QK_HEAD_DIM
    assert oracle.MAX_SEQ_LEN == GOLD["max_seq_len"]["value"]
    assert oracle.ORIGINAL_SEQ_LEN == GOLD["original_seq_len"]["value"]


def test_kv_down_rejects_wrong_width():
    with pytest.raises(ValueError):
        oracle.kv_down(np.zeros((2, 10)), np.zeros((576, 11)))


# ---------------------------------------------------------------- (b) scale constant
def test_scale_constant():
    m = 1 + 0.1 * math.log(40)
    assert abs(m - 1.3688879454113936) < 1e-15
    g = GOLD["m_squared_printed"]
    assert round(m * m, g["decimals"]) == g["value"]
    s = oracle.softmax_scale()
    assert abs(s - 0.13523) < 5e-6                       # value stated for the workload
    assert abs(s - m * m / math.sqrt(192)) < 1e-15       # Scale scores formula
    # fp32 value handed to kernels
    assert np.float32(s).view(np.uint32) == 0x3E0A7AB9
    # the correction applies only when max_seq_len exceeds the original length
    assert oracle.softmax_scale(max_seq_len=4096) == 192 ** -0.5


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_matches_torch_cast_on_float32():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),      # subnormals
        (rng.standard_normal(2000) * 1e38).astype(np.float32),       # near overflow
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.3895314e38, 3.40e38,
                  np.inf, -np.inf], np.float32),
    ])
    # exact ties: bit 15 set and bits 0..14 clear, both parities of bit 16
    ties = (rng.integers(0x3F000000, 0x40800000, 4000, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    v = np.concatenate([v, ties.view(np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.bf16(v)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_bf16_rounds_float64_once():
    # 1 + 2^-8 + 2^-30: nearest bf16 is 1 + 2^-7. Rounding to float32 first gives
    # 1 + 2^-8 (a tie) which then rounds to even = 1.0 (double rounding).
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.bf16(np.array([v]))[0] == np.float32(1.0 + 2.0 ** -7)
    assert oracle.bf16(np.array([-v]))[0] == np.float32(-(1.0 + 2.0 ** -7))
    assert oracle.bf16(np.array([float.fromhex("0x1.ff8p127")]))[0] == np.inf


# ---------------------------------------------------------------- GEMMs
def test_kv_down_orientation_with_one_hot_weight():
    rng = np.random.default_rng(1)
    x = bf(11, (2, 3, 7168))
    perm = rng.permutation(7168)[:576]
    w = np.zeros((576, 7168), np.float32)
    w[np.arange(576), perm] = 1.0
    out = oracle.kv_down(x, w)
    assert out.shape == (2, 3, 576)
    assert np.array_equal(out, x[..., perm])


def test_kv_down_brute_force_exact_rounding():
    x = bf(12, (3, 7168))
    w = bf(13, (576, 7168), 1 / math.sqrt(7168))
    out = oracle.kv_down(x, w)
    rng = np.random.default_rng(2)
    for _ in range(40):
        i, j = int(rng.integers(3)), int(rng.integers(576))
        exact = math.fsum(float(a) * float(b) for a, b in zip(x[i], w[j]))
        ref = torch.tensor(exact, dtype=torch.float64).to(torch.float32)
        # the exact sum is a double; round it to bf16 from double via float32 only when
        # float32 holds it exactly, otherwise compare against both neighbours
        lo = np.float32(exact)
        cand = {float(torch.tensor(float(lo)).to(torch.bfloat16).float())}
        cand.add(float(torch.tensor(float(np.nextafter(lo, np.float32(np.inf)))).to(torch.bfloat16).float()))
        cand.add(float(torch.tensor(float(np.nextafter(lo, np.float32(-np.inf)))).to(torch.bfloat16).float()))
        assert float(out[i, j]) in cand
        # and it is within half a bf16 step of the exact value
        ulp = 2.0 ** (math.frexp(abs(exact))[1] - 8)
        assert abs(float(out[i, j]) - exact) <= 0.5 * ulp + 1e-300
        del ref


def test_kv_up_head_major_layout_with_one_hot_weight():
    B, T, H = 2, 5, 128
    c = bf(14, (B, T, 512))
    rng = np.random.default_rng(3)
    src = rng.integers(0, 512, H * 256)
    w = np.zeros((H * 256, 512), np.float32)
    w[np.arange(H * 256), src] = 1.0
    kv = oracle.kv_up(c, w)
    assert kv.shape == (B, H, T, 256)
    for h in (0, 1, 77, 127):
        for j in (0, 127, 128, 255):
            assert np.array_equal(kv[:, h, :, j], c[:, :, src[h * 256 + j]])


def test_kv_up_matches_torch_linear():
    c = bf(15, (1, 7, 512))
    w = bf(16, (32768, 512), 1 / math.sqrt(512))
    kv = oracle.kv_up(c, w)
    ref = torch.nn.functional.linear(torch.from_numpy(c).double(), torch.from_numpy(w).double())
    ref = ref.view(1, 7, 128, 256).permute(0, 2, 1, 3).float()
    d = np.abs(kv - ref.numpy())
    # one bf16 rounding of the float64 product: within half a step of it
    assert (d <= np.abs(ref.numpy()) * 2.0 ** -8 + 1e-30).all()


# ---------------------------------------------------------------- (f) RMSNorm
def test_rms_norm_constant_row_gives_gain_times_sign():
    gain = synth.make("tiny", ("gain",))["gain"]
    for c in (0.75, -3.0, 1e-3, 12345.0):
        row = np.full((1, 512), np.float32(c))
        out = oracle.rms_norm(row, gain, 1e-20)
        assert np.array_equal(out[0], oracle.bf16(gain * np.sign(c)))


def test_rms_norm_zero_row_and_eps_placement():
    gain = np.ones(512, np.float32)
    assert np.array_equal(oracle.rms_norm(np.zeros((1, 512), np.float32), gain), np.zeros((1, 512)))
    # constant 1e-4 with eps 1e-6: y = 1e-4 / sqrt(1e-8 + 1e-6)
    row = np.full((1, 512), np.float32(1e-4))
    expect = float(np.float32(1e-4)) / math.sqrt(float(np.float32(1e-4)) ** 2 + 1e-6)
    got = oracle.rms_norm(row, gain, 1e-6)[0, 0]
    assert abs(got - expect) <= 2.0 ** -8 * expect


def test_rms_norm_power_of_two_scale_invariance():
    x = bf(17, (64, 512))
    gain = synth.make("tiny", ("gain",))["gain"]
    a = oracle.rms_norm(x, gain, 1e-20)
    b = oracle.rms_norm(x * np.float32(4.0), gain, 1e-20)
    assert np.array_equal(a, b)


def test_rms_norm_matches_torch_rms_norm():
    x = bf(18, (256, 512))
    gain = synth.make("tiny", ("gain",))["gain"]
    for eps in (1e-6, 1e-20):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (512,), torch.from_numpy(gain), eps)
        ref = ref.to(torch.bfloat16).float().numpy()
        got = oracle.rms_norm(x, gain, eps)
        step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        assert (np.abs(got - ref) <= step).all()
        assert np.mean(got == ref) > 0.99


# ---------------------------------------------------------------- rotary
def test_rotary_position_zero_is_identity():
    pe = bf(19, (5, 64))
    ang = oracle.rope_angles(np.zeros(5))
    assert np.array_equal(oracle.rotary(pe, ang), pe)


def test_rotary_closed_form_and_pair_convention():
    theta = 10000.0
    for i in (0, 1, 17, 31):
        pe = np.zeros((1, 64), np.float32)
        pe[0, 2 * i] = 1.0
        for pos in (1, 5, 4095):
            out = oracle.rotary(pe, oracle.rope_angles(np.array([pos])))
            phi = pos * theta ** (-2 * i / 64)
            assert out[0, 2 * i] == oracle.bf16(np.array([math.cos(phi)]))[0]
            assert out[0, 2 * i + 1] == oracle.bf16(np.array([math.sin(phi)]))[0]
            others = np.delete(out[0], [2 * i, 2 * i + 1])
            assert not others.any()
        pe = np.zeros((1, 64), np.float32)
        pe[0, 2 * i + 1] = 1.0      # imaginary unit goes to (-sin, cos)
        out = oracle.rotary(pe, oracle.rope_angles(np.array([3])))
        phi = 3 * theta ** (-2 * i / 64)
        assert out[0, 2 * i] == oracle.bf16(np.array([-math.sin(phi)]))[0]
        assert out[0, 2 * i + 1] == oracle.bf16(np.array([math.cos(phi)]))[0]


def test_rotary_preserves_pair_norms_and_relative_positions():
    a = bf(20, (64,))
    bvec = bf(21, (64,))
    ang = lambda p: oracle.rope_angles(np.array([p]))[0]

    def rot64(v, p):   # unrounded rotation via complex numbers (independent of oracle.rotary)
        z = v[0::2].astype(np.float64) + 1j * v[1::2].astype(np.float64)
        return z * np.exp(1j * ang(p))
    for p in (0, 1, 100, 16383):
        out = oracle.rotary(a[None], ang(p)[None])[0]
        z = rot64(a, p)
        assert np.allclose(out[0::2], z.real, rtol=2 ** -8, atol=1e-6)
        assert np.allclose(out[1::2], z.imag, rtol=2 ** -8, atol=1e-6)
        n_in = np.hypot(a[0::2].astype(np.float64), a[1::2].astype(np.float64))
        n_out = np.hypot(out[0::2].astype(np.float64), out[1::2].astype(np.float64))
        assert np.allclose(n_in, n_out, rtol=2 ** -7, atol=1e-6)
    # <R(s)a, R(t)b> = <R(s-t)a, b>, evaluated on the float64 rotation
    s, t = 37, 11
    lhs = np.real(np.vdot(rot64(bvec, t), rot64(a, s)))
    rhs = np.real(np.vdot(bvec[0::2] + 1j * bvec[1::2], rot64(a, s - t)))
    assert abs(lhs - rhs) < 1e-9
    # the oracle's rotation composes: R(p) then R(-p) returns the input up to bf16 rounding
    out = oracle.rotary(oracle.rotary(a[None], ang(9)[None]), ang(-9)[None])[0]
    assert np.allclose(out, a, rtol=2 ** -6, atol=1e-2)


def test_kv_latent_split_order():
    x = bf(22, (1, 4, 7168))
    w = bf(23, (576, 7168), 1 / math.sqrt(7168))
    gain = synth.make("tiny", ("gain",))["gain"]
    kv_raw, c_kv, k_pe = oracle.kv_latent(x, w, gain)
    assert np.array_equal(c_kv, oracle.rms_norm(kv_raw[..., :512], gain))
    assert np.array_equal(k_pe[:, 0], kv_raw[:, 0, 512:])          # position 0 unrotated
    assert np.array_equal(k_pe, oracle.rotary(kv_raw[..., 512:], oracle.rope_angles(np.arange(4))))


# ---------------------------------------------------------------- selection
def test_selection_mask_brute_force():
    T, K = 9, 6
    topk = np.array([[[0, -1, -1, 3, 3, 8],
                      [1, 0, 0, -1, 12, -7],
                      [2, 1, 1, 1, 1, 1],
                      [3, 4, 5, 6, 7, 8],
                      [4, 0, 2, -1, -1, -1],
                      [5, 5, 5, 5, 5, 5],
                      [6, 0, 1, 2, 3, 4],
                      [7, 8, 100, -1, 2, 6],
                      [8, 7, 6, 5, 4, 3]]], np.int32)
    allowed = oracle.selection_mask(topk, T)
    for s in range(T):
        want = {int(t) for t in topk[0, s] if 0 <= t <= s}
        got = set(np.nonzero(allowed[0, s])[0].tolist())
        assert got == want, s


# ---------------------------------------------------------------- attention
def _tiny_attn_inputs(seed, B, T, H=128, K=None):
    q = bf(seed, (B, T, H, 192))
    kv = bf(seed + 1, (B, H, T, 256))
    kpe = bf(seed + 2, (B, T, 64))
    topk = synth.random_topk(seed + 3, B, T, K or max(1, T // 2))
    return q, kv, kpe, topk


def test_softmax_rows_sum_to_one_and_are_zero_off_the_selection():
    q, kv, kpe, topk = _tiny_attn_inputs(30, 1, 24, H=8, K=5)
    scale = oracle.softmax_scale()
    _, P = oracle.sparse_prefill_attn(q, kv, kpe, topk, scale, return_probs=True)
    allowed = oracle.selection_mask(topk, 24)
    assert np.allclose(P.sum(-1), 1.0, atol=1e-12)
    off = ~allowed[:, :, None, :].repeat(8, axis=2)
    assert (P[off] == 0.0).all()
    assert (P[~off] > 0.0).all()


def test_full_selection_equals_dense_causal_sdpa():
    B, T, H = 1, 16, 128
    q, kv, kpe, _ = _tiny_attn_inputs(40, B, T, H)
    topk = np.tile(np.arange(T, dtype=np.int32), (B, T, 1))   # every key; causality trims
    scale = oracle.softmax_scale()
    out = oracle.sparse_prefill_attn(q, kv, kpe, topk, scale)
    qt = torch.from_numpy(q).double().permute(0, 2, 1, 3)
    k = torch.cat([torch.from_numpy(kv[..., :128]).double(),
                   torch.from_numpy(kpe).double()[:, None].expand(B, H, T, 64)], -1)
    v = torch.from_numpy(kv[..., 128:]).double()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, is_causal=True, scale=scale)
    ref = ref.permute(0, 2, 1, 3).float().to(torch.bfloat16).float().numpy()
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert (np.abs(out - ref) <= step).all()


def test_query_zero_and_self_only_selection_return_the_value_row():
    B, T, H = 2, 12, 128
    q, kv, kpe, topk = _tiny_attn_inputs(50, B, T, H, K=4)
    out = oracle.sparse_prefill_attn(q, kv, kpe, topk, oracle.softmax_scale())
    assert np.array_equal(out[:, 0], kv[:, :, 0, 128:])
    self_only = np.arange(T, dtype=np.int32)[None, :, None].repeat(B, 0)
    out = oracle.sparse_prefill_attn(q, kv, kpe, self_only, oracle.softmax_scale())
    assert np.array_equal(out, kv[..., 128:].transpose(0, 2, 1, 3))


def _sdpa_with_selection(q, kv, kpe, topk, scale):
    """torch's scaled_dot_product_attention in float64 with a boolean mask built row by row from
    each query's index set (Keys page, MHA-prefill excerpt: the index mask plus the causal mask,
    shared by every head). Returns [B, T, H, 128] rounded to bf16 by torch's cast."""
    B, T, H, _ = q.shape
    allow = torch.zeros((B, 1, T, T), dtype=torch.bool)
    for b in range(B):
        for s in range(T):
            for t in {int(e) for e in topk[b, s]}:
                if 0 <= t <= s:
                    allow[b, 0, s, t] = True
    qt = torch.from_numpy(np.asarray(q, np.float64)).permute(0, 2, 1, 3)
    kt = torch.cat([torch.from_numpy(np.asarray(kv[..., :128], np.float64)),
                    torch.from_numpy(np.asarray(kpe, np.float64))[:, None].expand(B, H, T, 64)], -1)
    vt = torch.from_numpy(np.asarray(kv[..., 128:], np.float64))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allow, scale=scale)
    return o.permute(0, 2, 1, 3).float().to(torch.bfloat16).float().numpy()


def test_matches_torch_sdpa_with_a_selection_mask():
    """The selection with duplicates, -1 padding and future positions, as a boolean mask handed
    to torch's attention routine."""
    B, T, H, K = 2, 16, 128, 6
    q, kv, kpe, topk = _tiny_attn_inputs(60, B, T, H, K)
    topk[0, 9, :3] = [4, 4, 15]          # a repeated entry and a future position
    topk[1, 3, 1:] = -1
    scale = oracle.softmax_scale()
    out = oracle.sparse_prefill_attn(q, kv, kpe, topk, scale)
    ref = _sdpa_with_selection(q, kv, kpe, topk, scale)
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert (np.abs(out - ref) <= step).all()


def _torch_prefill(x, wd, gain, wu, q, topk, scale, eps=1e-6):
    """The whole path composed from torch library routines only (linear, rms_norm, complex
    multiply, attention), each stage consuming this function's own previous stage."""
    bfr = lambda t: t.float().to(torch.bfloat16).float().double()
    x, wd, wu = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, wd, wu))
    B, T, _ = x.shape
    kv_raw = bfr(torch.nn.functional.linear(x, wd))
    c, pe = kv_raw[..., :512], kv_raw[..., 512:]
    c_kv = bfr(torch.nn.functional.rms_norm(c.float(), (512,), weight=torch.from_numpy(gain), eps=eps))
    ang = torch.arange(T, dtype=torch.float64)[:, None] * 10000.0 ** (-torch.arange(0, 64, 2, dtype=torch.float64) / 64)
    z = torch.view_as_complex(pe.reshape(B, T, 32, 2).contiguous()) * torch.polar(torch.ones_like(ang), ang)
    k_pe = bfr(torch.view_as_real(z).reshape(B, T, 64))
    kv = bfr(torch.nn.functional.linear(c_kv, wu)).reshape(B, T, 128, 256).permute(0, 2, 1, 3)
    out = _sdpa_with_selection(q, kv.numpy(), k_pe.numpy(), topk, scale)
    return {"kv_raw": kv_raw.numpy(), "c_kv": c_kv.numpy(), "k_pe": k_pe.numpy(), "kv": kv.numpy(), "out": out}


def test_mla_prefill_matches_an_independent_torch_composition():
    """oracle.mla_prefill end to end from x (the down-projection page's key-value excerpt, then
    the Keys page's MHA-prefill excerpt) against the same steps written with torch routines."""
    B, T, K = 2, 12, 5
    x = bf(100, (B, T, 7168))
    wd = bf(101, (576, 7168), 7168 ** -0.5)
    wu = bf(102, (32768, 512), 512 ** -0.5)
    gain = (1.0 + bf(103, (512,), 0.1 ** 0.5)).astype(np.float32)
    gain = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(gain))
    q = bf(104, (B, T, 128, 192))
    topk = synth.random_topk(105, B, T, K)
    scale = oracle.softmax_scale()
    got = oracle.mla_prefill(x, wd, gain, wu, q, topk, scale)
    ref = _torch_prefill(x, wd, gain, wu, q, topk, scale)
    for name in ("kv_raw", "c_kv", "k_pe", "kv"):
        r = ref[name]
        step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 7)
        assert (np.abs(got[name] - r) <= step).all(), name
    d = got["out"] - ref["out"]
    assert np.linalg.norm(d) <= 1e-3 * np.linalg.norm(ref["out"])
    assert np.abs(d).max() <= 2e-2
    # the composition tells the inputs apart: swapping the two weights' roles is impossible by
    # shape, but a path without the norm, or with the rotary key left unrotated, is not this one
    no_norm = oracle.sparse_prefill_attn(q, oracle.kv_up(got["kv_raw"][..., :512], wu),
                                         got["k_pe"], topk, scale)
    assert np.abs(no_norm - ref["out"]).max() > 0.1
    unrotated = oracle.sparse_prefill_attn(q, got["kv"], got["kv_raw"][..., 512:], topk, scale)
    assert np.abs(unrotated - ref["out"]).max() > 0.1


def test_regrouped_products_equal_the_unrounded_form():
    """Associativity: scoring the latent rows with the absorbed query W_UK^T q_nope, mixing the
    latent rows and mapping the mix through W_UV gives the pages' attention computed without
    the bf16 rounding of the per-head keys and values (``kv_up(..., rounded=False)``)."""
    B, T, K = 1, 20, 6
    q = bf(110, (B, T, 128, 192))
    c = bf(111, (B, T, 512))
    kpe = bf(112, (B, T, 64))
    wu = bf(113, (32768, 512), 512 ** -0.5)
    topk = synth.random_topk(114, B, T, K)
    scale = oracle.softmax_scale()
    out = oracle.sparse_prefill_attn(q, oracle.kv_up(c, wu, rounded=False), kpe, topk, scale)
    W = torch.from_numpy(wu.astype(np.float64)).reshape(128, 256, 512)
    wuk, wuv = W[:, :128], W[:, 128:]                       # [h, 128, 512]
    qt = torch.from_numpy(q.astype(np.float64))[0]         # [T, h, 192]
    ct = torch.from_numpy(c.astype(np.float64))[0]         # [T, 512]
    pt = torch.from_numpy(kpe.astype(np.float64))[0]       # [T, 64]
    ref = np.zeros((T, 128, 128))
    for s in range(T):
        ids = sorted({int(e) for e in topk[0, s] if 0 <= e <= s})
        q_lat = torch.bmm(qt[s, :, None, :128], wuk)[:, 0]                      # [h, 512]
        sc = scale * (q_lat @ ct[ids].T + qt[s, :, 128:] @ pt[ids].T)           # [h, n]
        o_lat = torch.softmax(sc, -1) @ ct[ids]                                 # [h, 512]
        ref[s] = torch.bmm(wuv, o_lat[:, :, None])[:, :, 0].numpy()
    ref = oracle.bf16(ref)
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert (np.abs(out[0] - ref) <= step).all()


def test_rounding_of_the_per_head_values_alone_exceeds_the_attention_bound():
    """The pages' order rounds every head's values to bf16 before mixing them. For queries with
    few keys the output has the magnitude of single value rows, where one bf16 step is 2^-5
    (|out| >= 4): the unrounded form and the rounded form then differ by more than 2e-2 in some
    elements, while their rel-L2 distance stays far below 1e-2. A regrouped computation, which
    never forms the values, is therefore held to the attention bound against the unrounded
    form."""
    B, T, K = 3, 130, 7
    seed = 5137
    q = synth.bf16_bits_to_f32(synth.random_bf16(seed, (B, T, 128, 192)))
    c = synth.bf16_bits_to_f32(synth.random_bf16(seed + 1, (B, T, 512)))
    kpe = synth.bf16_bits_to_f32(synth.random_bf16(seed + 2, (B, T, 64)))
    wu = synth.bf16_bits_to_f32(synth.random_bf16(seed + 3, (32768, 512), 512 ** -0.5))
    topk = synth.random_topk(seed + 4, B, T, K)
    scale = oracle.softmax_scale()
    rounded = oracle.sparse_prefill_attn(q, oracle.kv_up(c, wu), kpe, topk, scale)
    exact = oracle.sparse_prefill_attn(q, oracle.kv_up(c, wu, rounded=False), kpe, topk, scale)
    d = np.abs(rounded.astype(np.float64) - exact)
    assert d.max() > 2e-2
    assert np.linalg.norm(rounded - exact) <= 5e-3 * np.linalg.norm(exact)
    # every difference is the values' rounding carried through the weights: at most one bf16
    # step of the largest value row involved plus one output rounding
    vmax = np.abs(oracle.kv_up(c, wu)[..., 128:]).max()
    assert d.max() <= 2.0 ** (np.floor(np.log2(vmax)) - 7) + 2.0 ** (np.floor(np.log2(np.abs(exact).max())) - 7)


def test_pure_python_brute_force_tiny():
    B, T, H, K = 1, 7, 3, 3
    q, kv, kpe, topk = _tiny_attn_inputs(70, B, T, H, K)
    scale = oracle.softmax_scale()
    out = oracle.sparse_prefill_attn(q, kv, kpe, topk, scale)
    for s in range(T):
        keys = sorted({int(t) for t in topk[0, s] if 0 <= t <= s})
        for h in range(H):
            sc = []
            for t in keys:
                kk = list(kv[0, h, t, :128]) + list(kpe[0, t])
                sc.append(scale * math.fsum(float(a) * float(b) for a, b in zip(q[0, s, h], kk)))
            mx = max(sc)
            e = [math.exp(x - mx) for x in sc]
            z = math.fsum(e)
            for d in range(0, 128, 9):
                val = math.fsum(e[n] / z * float(kv[0, h, t, 128 + d]) for n, t in enumerate(keys))
                ulp = 2.0 ** (math.frexp(abs(val))[1] - 8) if val else 0.0
                assert abs(out[0, s, h, d] - val) <= 0.5 * ulp + 1e-12


def test_gather_rows_form_matches_dense_form():
    B, T, H, K = 2, 96, 128, 20
    q, kv, kpe, topk = _tiny_attn_inputs(80, B, T, H, K)
    scale = oracle.softmax_scale()
    dense = oracle.sparse_prefill_attn(q, kv, kpe, topk, scale)
    rows = [0, 1, 19, 20, 21, 50, 95]
    for b in range(B):
        got = oracle.sparse_prefill_attn_rows(q, kv, kpe, topk, scale, b, rows)
        step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(dense[b, rows]), 1e-30))) - 7)
        assert (np.abs(got - dense[b, rows]) <= step).all()


def test_masked_keys_never_matter_and_order_is_irrelevant():
    B, T, H, K = 1, 40, 16, 7
    q, kv, kpe, topk = _tiny_attn_inputs(90, B, T, H, K)
    scale = oracle.softmax_scale()
    base = oracle.sparse_prefill_attn(q, kv, kpe, topk, scale)
    allowed = oracle.selection_mask(topk, T)
    ever = allowed[0].any(axis=0)                 # keys selected by some query
    # poison keys no query selects with large finite values
    kv2, kpe2 = kv.copy(), kpe.copy()
    kv2[0][:, ~ever] = 1e4
    kpe2[0][~ever] = -1e4
    assert np.array_equal(oracle.sparse_prefill_attn(q, kv2, kpe2, topk, scale), base)
    rng = np.random.default_rng(4)
    shuffled = np.stack([[rng.permutation(r) for r in topk[0]]])
    assert np.array_equal(oracle.sparse_prefill_attn(q, kv, kpe, shuffled, scale), base)


def test_empty_allowed_set_is_rejected():
    q, kv, kpe, _ = _tiny_attn_inputs(95, 1, 4, H=2)
    topk = np.full((1, 4, 2), -1, np.int32)
    topk[0, :, 0] = np.arange(4)
    topk[0, 2, 0] = 3            # row 2 selects only a future key
    with pytest.raises(ValueError):
        oracle.sparse_prefill_attn(q, kv, kpe, topk, 0.1)


def test_topk_defects_brute_force():
    """Counts of out-of-range, future and repeated entries and of empty rows, against a plain
    loop over every row's entries with a Python set."""
    rng = np.random.default_rng(7)
    B, T, K = 2, 23, 9
    topk = rng.integers(-4, T + 4, (B, T, K)).astype(np.int32)
    topk[0, 5] = -1                      # an all-padding row
    topk[1, 0] = [3, 7, 22, -1, -1, -1, 30, 1, 2]   # query 0 with only later positions
    topk[1, 9, :4] = [2, 2, 2, 9]
    want = {"invalid": 0, "future": 0, "repeated": 0, "empty_rows": 0}
    for b in range(B):
        for s in range(T):
            seen = set()
            for e in topk[b, s]:
                e = int(e)
                if e < -1 or e >= T:
                    want["invalid"] += 1
                elif e > s:
                    want["future"] += 1
                elif e >= 0:
                    if e in seen:
                        want["repeated"] += 1
                    seen.add(e)
            want["empty_rows"] += not seen
    assert oracle.topk_defects(topk, T) == want
    assert want["empty_rows"] >= 2 and want["repeated"] >= 2
    clean = synth.random_topk(8, 1, 40, 12)
    assert oracle.topk_defects(clean, 40) == {"invalid": 0, "future": 0, "repeated": 0, "empty_rows": 0}
