"""GPU parity of the FP8 latent round trip with the cache writes, and of the V4.1 window-KV front
end, through the C ABI.

Criteria: the round trip and every cache or ring-buffer row are compared bit for bit with the
oracle applied to the GPU's own values before the round trip (both sides take every rounding
decision in fp32); those values themselves are within one bf16 step of the oracle's norm and
rotary (the norm's criterion)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import fp8_cache as f8
import sparse_latent_attention_wkv_amd as mla

from _gpu import assert_within_one_step, bf16_step, dev, say, to_dev, to_host

pytestmark = pytest.mark.gpu

FMT = {0: "fp32", 1: "ue8m0"}


def bf(seed, shape, std=1.0):
    return synth.random_bf16(seed, shape, std)


def f32(bits):
    return synth.bf16_bits_to_f32(bits)


def _gain(seed=7):
    g = 1.0 + np.sqrt(0.1) * np.random.default_rng(seed).standard_normal(512)
    return oracle.bf16(g).astype(np.float32)


def _spice(x_bits, seed):
    """Rows with hard blocks: a zero block, a block with a few huge and many tiny features (codes
    in the e4m3 subnormal range), an all-zero row."""
    x = f32(x_bits).copy()
    n = x.shape[0]
    rng = np.random.default_rng(seed)
    if n >= 3:
        x[0, 0:128] = 0.0
        x[0, 128:136] = -0.0                                  # signed zeros keep their sign
        x[1, 128:256] *= np.where(rng.random(128) < 0.9, 1e-4, 1.0)
        x[2, :512] = 0.0
    return synth.f32_to_bf16_bits(x)


def _check_pre(got, ref, what):
    assert_within_one_step(got, ref, what=what)


def same_bits(a, b):
    """Bit-for-bit equality of two float32 arrays of bf16 values (signed zeros included)."""
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    return a.shape == b.shape and np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------------------------ f2
CASES = [  # B, T, start_pos, scale_fmt, cache_batch, cache_len
    (1, 64, 0, 0, 1, 64),
    (2, 77, 5, 1, 3, 100),
    (1, 1, 0, 0, 1, 1),
    (2, 300, 1000, 0, 2, 1400),
    (3, 130, 17, 1, 4, 160),
]


@pytest.mark.parametrize("B,T,sp,fmt,cb,cl", CASES)
def test_kv_latent_cache_matches_oracle(B, T, sp, fmt, cb, cl):
    say(f"kv_latent_cache B={B} T={T} start_pos={sp} fmt={fmt} cache=[{cb},{cl}]")
    seed = 5000 + 7 * T + sp
    x = bf(seed, (B, T, 7168))
    w = bf(seed + 1, (576, 7168), std=7168 ** -0.5)
    gain = _gain(seed)
    kc0 = bf(seed + 2, (cb, cl, 512))
    pc0 = bf(seed + 3, (cb, cl, 64))
    kc, pc = to_dev(kc0), to_dev(pc0)
    g = torch.from_numpy(gain).to(dev())
    kv_raw, c_kv, k_pe, c_norm = mla.mla_kv_latent_cache(to_dev(x), to_dev(w), g, kc, pc,
                                                         start_pos=sp, scale_fmt=fmt,
                                                         want_norm=True)
    torch.cuda.synchronize()
    raw, ckv, kpe, cn = to_host(kv_raw), to_host(c_kv), to_host(k_pe), to_host(c_norm)
    # the steps before the round trip, from the GPU's own down-projection output
    _check_pre(cn, oracle.rms_norm(raw[..., :512], gain), "c_norm")
    pe = raw[..., 512:]
    ref = oracle.rotary(pe, oracle.rope_angles(sp + np.arange(T)))
    mag = np.hypot(pe[..., 0::2].astype(np.float64), pe[..., 1::2].astype(np.float64)).repeat(2, -1)
    assert_within_one_step(kpe, ref, extra=4 * 2.0 ** -24 * mag, what="k_pe")
    # the round trip, bit for bit
    assert same_bits(ckv, f8.fp8_round_trip(cn, FMT[fmt])), "c_kv round trip"
    # cache rows, bit for bit; rows outside the call untouched
    want_kc, want_pc = f8.cache_write(ckv, kpe, f32(kc0), f32(pc0), sp)
    assert same_bits(to_host(kc), want_kc), "kv_cache"
    assert same_bits(to_host(pc), want_pc), "pe_cache"


def test_norm_rope_cache_step_alone_and_without_c_norm():
    B, T, sp = 2, 200, 9
    say(f"kv_norm_rope_cache B={B} T={T} start_pos={sp}")
    raw_bits = _spice(bf(61, (B * T, 576)), 62).reshape(B, T, 576)
    gain = _gain(63)
    g = torch.from_numpy(gain).to(dev())
    kc, pc = to_dev(np.zeros((B, 256, 512), np.uint16)), to_dev(np.zeros((B, 256, 64), np.uint16))
    raw = to_dev(raw_bits)
    c_kv, k_pe, c_norm = mla.mla_kv_norm_rope_cache(raw, g, kc, pc, start_pos=sp, want_norm=True)
    kc2, pc2 = torch.zeros_like(kc), torch.zeros_like(pc)
    c_kv2, k_pe2 = mla.mla_kv_norm_rope_cache(raw, g, kc2, pc2, start_pos=sp)
    torch.cuda.synchronize()
    cn = to_host(c_norm)
    _check_pre(cn, oracle.rms_norm(f32(raw_bits)[..., :512], gain), "c_norm")
    got = to_host(c_kv)
    assert same_bits(got, f8.fp8_round_trip(cn))
    assert not got[0, 0, :128].any() and not got[0, 2, :].any()       # zero block, zero row
    assert same_bits(got, to_host(c_kv2)) and same_bits(to_host(k_pe), to_host(k_pe2))
    assert torch.equal(kc, kc2) and torch.equal(pc, pc2)
    # the unfused norm/rotary kernel gives the same normalised latent and rotated key
    flat = raw.reshape(B * T, 576)
    cs = mla.mla_rope_table(sp + T, dev())[sp:].contiguous()
    c_plain, k_plain = mla.mla_kv_norm_rope(flat, g, 1e-6, cs, T)
    torch.cuda.synchronize()
    assert same_bits(to_host(c_plain).reshape(B, T, 512), cn)
    assert_within_one_step(to_host(k_pe), to_host(k_plain).reshape(B, T, 64), what="k_pe vs plain")


def test_norm_rope_cache_front_end_workload_rows():
    """The latent front-end workload's prefill rows (B=8, T=4096), the launch that is timed:
    every row of the round trip and of the caches, bit for bit against the oracle on the GPU's
    own normalised latent."""
    B, T = 8, 4096
    say(f"kv_norm_rope_cache workload B={B} T={T}")
    raw_bits = bf(71, (B, T, 576))
    gain = _gain(72)
    g = torch.from_numpy(gain).to(dev())
    kc = torch.zeros((B, T, 512), dtype=torch.bfloat16, device=dev())
    pc = torch.zeros((B, T, 64), dtype=torch.bfloat16, device=dev())
    c_kv, k_pe, c_norm = mla.mla_kv_norm_rope_cache(to_dev(raw_bits), g, kc, pc, want_norm=True)
    torch.cuda.synchronize()
    cn = to_host(c_norm)
    rows = np.random.default_rng(73).choice(B * T, 2048, replace=False)
    _check_pre(cn.reshape(-1, 512)[rows],
               oracle.rms_norm(f32(raw_bits).reshape(-1, 576)[rows, :512], gain), "c_norm rows")
    ckv = to_host(c_kv)
    assert same_bits(ckv, f8.fp8_round_trip(cn))
    assert same_bits(to_host(kc), ckv)
    assert same_bits(to_host(pc), to_host(k_pe))


# ------------------------------------------------------------------------------ f4
WCASES = [  # B, S, start_pos, window, scale_fmt
    (2, 5, 0, 8, 0),         # prefill shorter than the window
    (2, 21, 0, 8, 1),        # prefill longer: split at S mod W
    (1, 64, 0, 64, 0),       # exactly one window
    (3, 1, 37, 16, 0),       # one decode position
    (256, 1, 1000, 128, 0),  # the decode workload's shape: 256 sequences, one position each
]


@pytest.mark.parametrize("B,S,sp,W,fmt", WCASES)
def test_window_kv_matches_oracle(B, S, sp, W, fmt):
    say(f"window_kv B={B} S={S} start_pos={sp} window={W} fmt={fmt}")
    seed = 9000 + B + S + sp
    raw_bits = _spice(bf(seed, (B * S, 512)), seed + 1).reshape(B, S, 512)
    gain = _gain(seed)
    cache0 = bf(seed + 2, (B + 1, W, 512))
    cache = to_dev(cache0)
    kv, pre = mla.mla_window_kv(to_dev(raw_bits), torch.from_numpy(gain).to(dev()), cache,
                                start_pos=sp, scale_fmt=fmt, want_pre=True)
    torch.cuda.synchronize()
    kvh, preh = to_host(kv), to_host(pre)
    ref_pre, _, _ = f8.window_kv(f32(raw_bits), gain, f32(cache0), start_pos=sp,
                                 scale_fmt=FMT[fmt])
    # The tail is rotated after the bf16 rounding of the norm, where the GPU may sit one step
    # from the oracle: a pair's rotation moves such a difference by up to one step of each of
    # its two inputs, plus the fp32 arithmetic.
    y = oracle.rms_norm(f32(raw_bits), gain, 1e-20).astype(np.float64)
    extra = np.zeros_like(y)
    re, im = y[..., 448::2], y[..., 449::2]
    pair = bf16_step(re) + bf16_step(im) + 4 * 2.0 ** -24 * np.hypot(re, im)
    extra[..., 448:] = pair.repeat(2, -1)
    assert_within_one_step(preh, ref_pre, extra=extra, what="kv_pre")
    assert same_bits(kvh, f8.fp8_round_trip(preh, FMT[fmt])), "round trip"
    assert same_bits(to_host(cache), f8.ring_write(kvh, f32(cache0), sp)), "ring buffer"


def test_window_prefill_then_decode_steps():
    """A prefill longer than the window, then decode steps that wrap the ring: after every call
    the buffer equals the pages' branches applied to the GPU's own outputs."""
    B, S0, W = 2, 13, 8
    say(f"window_kv prefill {S0} + decode, window {W}")
    gain = _gain(81)
    g = torch.from_numpy(gain).to(dev())
    cache = torch.zeros((B, W, 512), dtype=torch.bfloat16, device=dev())
    cs = mla.mla_rope_table(S0 + 12, dev())
    want = np.zeros((B, W, 512), np.float32)
    raw_bits = bf(82, (B, S0 + 12, 512))
    kv = mla.mla_window_kv(to_dev(raw_bits[:, :S0]), g, cache, start_pos=0, rope_cs=cs)
    torch.cuda.synchronize()
    want = f8.ring_write(to_host(kv), want, 0)
    assert same_bits(to_host(cache), want)
    for p in range(S0, S0 + 12):
        kv = mla.mla_window_kv(to_dev(raw_bits[:, p:p + 1]), g, cache, start_pos=p, rope_cs=cs)
        torch.cuda.synchronize()
        want = f8.ring_write(to_host(kv), want, p)
        assert same_bits(to_host(cache), want), f"after decode position {p}"
