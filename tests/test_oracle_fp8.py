"""Pins for the FP8 round trip, cache-write and window-KV oracle: each check compares it with
something that does not come from it (the page's block size, torch's float8 type, closed
forms, the pages' two ring-buffer branches against each other, brute force). CPU only."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import fp8_cache as f8

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def bf(seed, shape, std=1.0):
    return synth.bf16_bits_to_f32(synth.random_bf16(seed, shape, std))


def torch_e4m3(y):
    """torch's own float32 -> float8_e4m3fn -> float32 cast (a library routine the oracle
    does not call)."""
    t = torch.from_numpy(np.asarray(y, np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float32).numpy()


# ------------------------------------------------------------------------------ the fp8 format
def test_block_size_is_the_pages():
    assert f8.FP8_BLOCK == GOLD["fp8_block_size"]["value"]


def test_e4m3_table_matches_torch_float8():
    codes = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    assert np.array_equal(f8.e4m3_values(), codes.numpy())
    assert torch.isnan(torch.tensor([127], dtype=torch.uint8).view(torch.float8_e4m3fn)
                       .to(torch.float32)).all()
    assert f8.E4M3_MAX == 448.0 == float(torch.finfo(torch.float8_e4m3fn).max)
    assert f8.e4m3_values()[1] == 2.0 ** -9            # smallest subnormal


def test_e4m3_round_matches_torch_cast():
    v = f8.e4m3_values()
    mids = (v[:-1] + v[1:]) / 2                                      # exact ties
    eps = np.float32(1e-6)
    rng = np.random.default_rng(7)
    ys = np.concatenate([v, mids, mids * (1 + eps), mids * (1 - eps),
                         rng.uniform(-448, 448, 20000), rng.uniform(-0.02, 0.02, 20000),
                         np.ldexp(rng.uniform(-1, 1, 5000), -12),
                         [448.00003, 455.0, 463.99997, 464.0]]).astype(np.float32)
    ys = np.concatenate([ys, -ys])
    got = f8.e4m3_round(ys).astype(np.float32)
    assert np.array_equal(got, torch_e4m3(ys))


def test_e4m3_round_rejects_out_of_range():
    with pytest.raises(ValueError):
        f8.e4m3_round(np.array([464.5]))


# ------------------------------------------------------------------------------ the scale
def test_scale_formats():
    amax = np.abs(bf(1, (4000,))).astype(np.float32) + np.float32(1e-3)
    s = f8.fp8_scale(amax, "fp32")
    assert s.dtype == np.float32
    assert np.all(np.abs(s.astype(np.float64) * 448 / amax - 1) < 2 ** -23)
    p = f8.fp8_scale(amax, "ue8m0").astype(np.float64)
    m, _ = np.frexp(p)
    assert np.all(m == 0.5)                                          # powers of two
    assert np.all(p >= amax / 448.0) and np.all(p / 2 < amax / 448.0)
    assert f8.fp8_scale(np.float32(0), "fp32") == 1.0
    with pytest.raises(ValueError):
        f8.fp8_scale(amax, "e5m2")


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_largest_element_takes_the_largest_code(fmt):
    x = bf(2, (64, 512))
    _, q, _ = f8.fp8_round_trip(x, fmt, return_parts=True)
    qb = np.abs(q.reshape(-1, 128))
    xb = np.abs(x.reshape(-1, 128))
    at = np.argmax(xb, axis=1)
    top = qb[np.arange(len(at)), at]
    if fmt == "fp32":
        assert np.all(top == 448.0)
    else:                                                            # scale >= amax / 448
        assert np.all(top <= 448.0) and np.all(top > 224.0 * (1 - 2 ** -4))


# ------------------------------------------------------------------------------ the round trip
@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_round_trip_exact_on_representable_blocks(fmt):
    rng = np.random.default_rng(3)
    v = f8.e4m3_values()
    blocks = []
    for k in (-20, -3, 0, 5):
        b = rng.choice(v, 128) * rng.choice([-1.0, 1.0], 128)
        b[rng.integers(128)] = -448.0 if k % 2 else 448.0
        blocks.append(np.ldexp(b, k))
    x = np.stack(blocks).reshape(2, 256).astype(np.float32)        # two rows of two blocks
    assert np.array_equal(oracle.bf16(x), x)
    assert np.array_equal(f8.fp8_round_trip(x, fmt), x)


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_round_trip_error_bound(fmt):
    x = bf(4, (200, 512), std=2.0)
    d, q, s = f8.fp8_round_trip(x, fmt, return_parts=True)
    sx = np.repeat(s, 128, axis=-1).astype(np.float64)
    err = np.abs(d.astype(np.float64) - x)
    # half an e4m3 step (relative 2^-4 above 2^-6, absolute 2^-10 below) times the scale,
    # then one bf16 rounding of the product
    bound = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * sx + 2.0 ** -8 * np.abs(d) + 1e-7 * np.abs(x)
    assert np.all(err <= bound)
    assert np.all(np.sign(d)[d != 0] == np.sign(x)[d != 0])
    # the dequantised values are e4m3 codes times the block scale, rounded to bf16
    assert np.array_equal(d, oracle.bf16((q * sx.astype(np.float32)).astype(np.float32)))


def test_round_trip_blocks_are_independent():
    x = bf(5, (3, 512))
    x[:, 128:256] *= 1e-3                                           # one quiet block per row
    full = f8.fp8_round_trip(x)
    for blk in range(4):
        part = f8.fp8_round_trip(x[:, 128 * blk:128 * (blk + 1)])
        assert np.array_equal(full[:, 128 * blk:128 * (blk + 1)], part)
    # a whole-row scale would flush the quiet block to a few codes; per-block keeps ~4 bits
    quiet = full[:, 128:256]
    assert np.all(np.abs(quiet - x[:, 128:256]) <= 2.0 ** -4 * np.abs(x[:, 128:256]) * 1.01
                  + 2.0 ** -8 * np.abs(quiet) + 1e-12)


def test_round_trip_zero_and_sign_symmetry():
    z = np.zeros((2, 256), np.float32)
    assert np.array_equal(f8.fp8_round_trip(z), z)
    x = bf(6, (10, 256))
    assert np.array_equal(f8.fp8_round_trip(-x), -f8.fp8_round_trip(x))


def test_round_trip_against_brute_force_quantiser():
    """Each element against an exhaustive search over all signed codes (tiny case)."""
    x = bf(8, (2, 128), std=0.7)
    s = f8.fp8_scale(np.max(np.abs(x), axis=-1), "fp32")
    v = f8.e4m3_values()
    allv = np.concatenate([-v[::-1], v])
    for r in range(2):
        for j in range(128):
            y = np.float32(x[r, j]) / s[r]
            dist = np.abs(allv - np.float64(y))
            best = allv[dist == dist.min()]
            if len(best) > 1:      # a tie: the code with an even mantissa (last bit 0)
                best = [b for b in best
                        if (np.searchsorted(v, abs(b)) % 2 == 0)]
            want = oracle.bf16(np.float32(np.float32(best[0]) * s[r]))
            assert f8.fp8_round_trip(x[r:r + 1], "fp32")[0, j] == want


# ------------------------------------------------------------------------------ f2 cache writes
def test_cache_write_positions():
    B, T, Bc, L, p = 2, 5, 3, 12, 4
    c = bf(9, (B, T, 512))
    pe = bf(10, (B, T, 64))
    kc0 = bf(11, (Bc, L, 512))
    pc0 = bf(12, (Bc, L, 64))
    kc, pc = f8.cache_write(c, pe, kc0, pc0, p)
    for b in range(Bc):
        for t in range(L):
            inside = b < B and p <= t < p + T
            assert np.array_equal(kc[b, t], c[b, t - p] if inside else kc0[b, t])
            assert np.array_equal(pc[b, t], pe[b, t - p] if inside else pc0[b, t])
    with pytest.raises(ValueError):
        f8.cache_write(c, pe, kc0, pc0, L - T + 1)


def test_kv_latent_cache_matches_front_end_at_shifted_positions():
    """Rows at start_pos p are the same tokens that a sequence with p leading tokens holds at
    positions p.. (the rotary angle depends only on the position)."""
    B, T, p = 1, 6, 9
    x = bf(13, (B, T, 7168))
    w = bf(14, (576, 7168), std=7168 ** -0.5)
    g = oracle.bf16(1 + bf(15, (512,), std=0.1 ** 0.5))
    kc0 = np.zeros((1, 32, 512), np.float32)
    pc0 = np.zeros((1, 32, 64), np.float32)
    kv_raw, c_norm, c_kv, k_pe, kc, pc = f8.kv_latent_cache(x, w, g, kc0, pc0, start_pos=p)
    xp = np.concatenate([bf(16, (B, p, 7168)), x], axis=1)
    raw2, c2, pe2 = oracle.kv_latent(xp, w, g)
    assert np.array_equal(kv_raw, raw2[:, p:])
    assert np.array_equal(c_norm, c2[:, p:])
    assert np.array_equal(k_pe, pe2[:, p:])
    assert np.array_equal(c_kv, f8.fp8_round_trip(c2[:, p:]))
    assert np.array_equal(kc[0, p:p + T], c_kv[0]) and not kc[0, :p].any()
    assert np.array_equal(pc[0, p:p + T], k_pe[0]) and not pc[0, p + T:].any()


# ------------------------------------------------------------------------------ f4 window KV
@pytest.mark.parametrize("S,W", [(3, 8), (8, 8), (13, 8), (21, 5)])
def test_window_prefill_equals_token_by_token_decode(S, W):
    """The excerpt's prefill branch seeds the ring buffer so that decoding continues it: one
    prefill of S positions leaves the same buffer as a one-position prefill followed by S-1
    single-position decode calls (every step is per position)."""
    B = 2
    raw = bf(17, (B, S, 512))
    g = oracle.bf16(1 + bf(18, (512,), std=0.1 ** 0.5))
    cache0 = bf(19, (B + 1, W, 512))
    _, kv_all, cache_a = f8.window_kv(raw, g, cache0, start_pos=0)
    _, kv0, cache_b = f8.window_kv(raw[:, :1], g, cache0, start_pos=0)
    steps = [kv0]
    for t in range(1, S):
        _, kv_t, cache_b = f8.window_kv(raw[:, t:t + 1], g, cache_b, start_pos=t)
        steps.append(kv_t)
    assert np.array_equal(np.concatenate(steps, axis=1), kv_all)
    # slots the prefill never reaches (S < W) keep the old contents in both
    assert np.array_equal(cache_a, cache_b)
    assert np.array_equal(cache_a[B:], cache0[B:])


def test_window_rotates_only_the_tail_and_normalises_with_eps_1e20():
    B, S = 1, 4
    raw = bf(20, (B, S, 512))
    g = oracle.bf16(1 + bf(21, (512,), std=0.1 ** 0.5))
    pre, kv, _ = f8.window_kv(raw, g, np.zeros((1, 8, 512), np.float32))
    y = oracle.rms_norm(raw, g, 1e-20)
    assert np.array_equal(pre[..., :448], y[..., :448])
    assert np.array_equal(pre[:, 0], y[:, 0])                       # position 0: angle 0
    a = pre[..., 448:].astype(np.float64).reshape(B, S, 32, 2)
    b = y[..., 448:].astype(np.float64).reshape(B, S, 32, 2)
    assert np.allclose(np.hypot(a[..., 0], a[..., 1]), np.hypot(b[..., 0], b[..., 1]),
                       rtol=2 ** -7, atol=1e-6)
    assert np.array_equal(kv, f8.fp8_round_trip(pre))
    # eps 1e-20 by default: a row of equal magnitudes 2^-16 (mean square 2^-32, far above
    # 1e-20 but far below 1e-6) still normalises to gain * sign
    tiny = np.full((1, 1, 512), 2.0 ** -16, np.float32) * np.sign(bf(22, (1, 1, 512)))
    pre_t, _, _ = f8.window_kv(tiny, g, np.zeros((1, 4, 512), np.float32))
    assert np.array_equal(pre_t[0, 0, :448], oracle.bf16(g[:448] * np.sign(tiny[0, 0, :448])))
