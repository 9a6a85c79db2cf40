"""Helpers shared by the GPU tests: moving seeded bf16 data to the device and back, and the
comparison criteria (bf16 lattice steps, fp32 accumulation bounds, attention tolerances)."""
import sys

import numpy as np
import torch

import synth


def dev():
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits_u16):
    """uint16 bf16 patterns -> torch.bfloat16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).view(torch.bfloat16).to(dev())


def f32_to_dev_bf16(a):
    return to_dev(synth.f32_to_bf16_bits(np.asarray(a, np.float32)))


def to_host(t):
    """torch bf16 tensor -> float32 numpy array (exact)."""
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return synth.bf16_bits_to_f32(bits)


def bf16_step(x):
    """Spacing of the bf16 lattice at |x| (normal range)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(ax)).astype(np.int64) - 7)


def assert_within_one_step(got, ref, extra=None, what=""):
    """|got - ref| <= one bf16 step of ref (plus an optional per-element allowance)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    allow = bf16_step(ref)
    if extra is not None:
        allow = allow + extra
    bad = np.abs(got - ref) > allow
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements beyond one bf16 step; "
                             f"first {idx.tolist()} got {got[bad][:5]} ref {ref[bad][:5]}")


def fp32_dot_bound(absprod_sum, n):
    """Error bound of an n-term fp32 recursive sum of products: n * 2^-24 * sum |x_k w_k|."""
    return n * 2.0 ** -24 * np.asarray(absprod_sum, np.float64)


def attention_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(got - ref).max()
    say(f"  {what}: rel-L2 {rel:.3e}, max-abs {mx:.3e}")
    assert rel <= 1e-2, f"{what}: rel-L2 {rel}"
    assert mx <= 2e-2, f"{what}: max-abs {mx}"
    return rel, mx


def pack_mask(allowed):
    """Boolean [B, T, T] allowed set -> uint32 words [B, ceil(T/32), T] in the library's layout."""
    B, T, _ = allowed.shape
    W = (T + 31) // 32
    pad = np.zeros((B, T, W * 32), bool)
    pad[:, :, :T] = allowed
    bits = pad.reshape(B, T, W, 32).astype(np.uint64)
    words = (bits << np.arange(32, dtype=np.uint64)).sum(-1).astype(np.uint32)   # [B, T, W]
    return words.transpose(0, 2, 1).copy()
