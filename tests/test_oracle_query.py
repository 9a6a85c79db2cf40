"""Pins for the query-path oracle: shapes from the constructor the pages print, GEMM orientation
with one-hot weights, torch's own linear and RMSNorm, the rotary's position properties shared
with the key, brute force on a tiny case. CPU only."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import query as qo


def bf(seed, shape, std=1.0):
    return synth.bf16_bits_to_f32(synth.random_bf16(seed, shape, std))


def _weights(seed, r=64, heads=128):
    w_qa = bf(seed, (r, 7168), std=7168 ** -0.5)
    gain = oracle.bf16(1 + bf(seed + 1, (r,), std=0.1 ** 0.5))
    w_qb = bf(seed + 2, (heads * 192, r), std=r ** -0.5)
    return w_qa, gain, w_qb


def test_query_parameter_shapes_follow_the_constructor():
    shp = qo.query_parameter_shapes()
    assert shp["wq_a"] == (qo.Q_LORA_RANK, oracle.HIDDEN)
    assert shp["q_norm"] == (qo.Q_LORA_RANK,)
    # n_heads * qk_head_dim, qk_head_dim = nope 128 + rope 64
    assert shp["wq_b"] == (128 * 192, qo.Q_LORA_RANK)


def test_one_hot_weights_route_features():
    """wq_a row i picks hidden feature p(i); wq_b row (h, j) picks low-rank feature f(h, j):
    the output must be those features (normalised, then rotated in the rope part)."""
    r = 64
    rng = np.random.default_rng(0)
    p = rng.permutation(7168)[:r]
    w_qa = np.zeros((r, 7168), np.float32)
    w_qa[np.arange(r), p] = 1.0
    f = rng.integers(0, r, 128 * 192)
    w_qb = np.zeros((128 * 192, r), np.float32)
    w_qb[np.arange(128 * 192), f] = 1.0
    x = bf(1, (1, 3, 7168))
    gain = np.ones(r, np.float32)
    qa, qr, q = qo.query_path(x, w_qa, gain, w_qb)
    assert np.array_equal(qa, x[..., p])
    want = qr[..., f].reshape(1, 3, 128, 192)
    assert np.array_equal(q[..., :128], want[..., :128])
    assert np.array_equal(q[:, 0, :, 128:], want[:, 0, :, 128:])        # position 0: no rotation


def test_matches_torch_linear_and_rms_norm():
    x = bf(2, (2, 5, 7168))
    w_qa, gain, w_qb = _weights(3)
    qa, qr, q = qo.query_path(x, w_qa, gain, w_qb)
    t_qa = torch.nn.functional.linear(torch.from_numpy(x).double(), torch.from_numpy(w_qa).double())
    assert np.array_equal(qa, oracle.bf16(t_qa.numpy()))
    t_qr = torch.nn.functional.rms_norm(torch.from_numpy(qa), (64,), torch.from_numpy(gain), 1e-6)
    steps = np.abs(qr - oracle.bf16(t_qr.numpy()))
    assert np.all(steps <= np.abs(qr) * 2.0 ** -7)                          # within one bf16 step
    t_q = torch.nn.functional.linear(torch.from_numpy(qr).double(), torch.from_numpy(w_qb).double())
    q0 = oracle.bf16(t_q.numpy()).reshape(2, 5, 128, 192)
    assert np.array_equal(q[..., :128], q0[..., :128])


def test_rope_part_rotates_like_the_key():
    """Rotated query and key parts at positions s and t score like positions s+d and t+d
    (the rotation depends on the position difference only), and every head uses the same
    angles as the shared key's rotation."""
    r = 64
    w_qa, gain, w_qb = _weights(4, r)
    x = bf(5, (1, 1, 7168))
    _, _, q_a = qo.query_path(x, w_qa, gain, w_qb, start_pos=7)
    _, _, q_b = qo.query_path(x, w_qa, gain, w_qb, start_pos=7 + 300)
    pe = bf(6, (1, 1, 64))
    k_a = oracle.rotary(pe, oracle.rope_angles(np.array([3])))
    k_b = oracle.rotary(pe, oracle.rope_angles(np.array([3 + 300])))
    s_a = q_a[0, 0, :, 128:].astype(np.float64) @ k_a[0, 0].astype(np.float64)
    s_b = q_b[0, 0, :, 128:].astype(np.float64) @ k_b[0, 0].astype(np.float64)
    scale = np.abs(q_a[0, 0, :, 128:]).sum(-1) * np.abs(pe).max()
    assert np.all(np.abs(s_a - s_b) <= 4 * 2.0 ** -8 * scale)
    # head h's rope part equals the key rotary applied to that head's unrotated part
    _, _, q0 = qo.query_path(x, w_qa, gain, w_qb, start_pos=0)
    for h in (0, 77, 127):
        want = oracle.rotary(q0[0, 0, h, 128:], oracle.rope_angles(np.array([7]))[0])
        assert np.array_equal(q_a[0, 0, h, 128:], want)


def test_tiny_brute_force():
    """Pure-Python sums for one token and a few outputs (r = 16)."""
    r = 16
    x = bf(7, (1, 2, 7168))
    w_qa = bf(8, (r, 7168), std=7168 ** -0.5)
    gain = oracle.bf16(1 + bf(9, (r,), std=0.1 ** 0.5))
    w_qb = bf(10, (128 * 192, r), std=r ** -0.5)
    qa, qr, q = qo.query_path(x, w_qa, gain, w_qb, start_pos=5)
    t = 1
    for i in (0, 9, 15):
        s = sum(float(x[0, t, k]) * float(w_qa[i, k]) for k in range(7168))
        assert qa[0, t, i] == oracle.bf16(s)
    for h, j in ((0, 3), (64, 100), (127, 127)):
        s = sum(float(qr[0, t, k]) * float(w_qb[h * 192 + j, k]) for k in range(r))
        assert q[0, t, h, j] == oracle.bf16(s)
    # one rotated pair of one head, written out: position 6, pair i = 5
    h, i = 31, 5
    re = oracle.bf16(sum(float(qr[0, t, k]) * float(w_qb[h * 192 + 128 + 2 * i, k]) for k in range(r)))
    im = oracle.bf16(sum(float(qr[0, t, k]) * float(w_qb[h * 192 + 129 + 2 * i, k]) for k in range(r)))
    phi = 6 * 10000.0 ** (-2 * i / 64)
    assert q[0, t, h, 128 + 2 * i] == oracle.bf16(float(re) * np.cos(phi) - float(im) * np.sin(phi))
    assert q[0, t, h, 129 + 2 * i] == oracle.bf16(float(re) * np.sin(phi) + float(im) * np.cos(phi))


def test_shape_errors():
    w_qa, gain, w_qb = _weights(11)
    with pytest.raises(ValueError):
        qo.query_path(bf(12, (1, 2, 7168)), w_qa, gain, w_qb[:-192])
