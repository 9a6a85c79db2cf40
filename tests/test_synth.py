"""The seeded synthetic inputs: shapes, distributions and the selection recipe (CPU only)."""
import numpy as np

import synth


def test_topk_recipe():
    B, T, K = 2, 300, 40
    topk = synth.random_topk(5, B, T, K)
    assert topk.shape == (B, T, K) and topk.dtype == np.int32
    for b in range(B):
        for s in range(T):
            row = topk[b, s]
            k = min(K, s + 1)
            valid = row[:k]
            assert (row[k:] == -1).all()
            assert len(set(valid.tolist())) == k          # distinct
            assert s in valid                              # self always included
            assert valid.min() >= 0 and valid.max() <= s   # causal prefix only


def test_workload_draws_are_deterministic_and_shaped():
    a = synth.make("tiny")
    b = synth.make("tiny")
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["x"].shape == (1, 64, 7168) and a["x"].dtype == np.uint16
    assert a["w_dkv"].shape == (576, 7168)
    assert a["w_ukv"].shape == (32768, 512)
    assert a["q"].shape == (1, 64, 128, 192)
    assert a["gain"].shape == (512,) and a["gain"].dtype == np.float32
    assert a["topk"].shape == (1, 64, 16)
    # a subset request draws the same values
    assert np.array_equal(synth.make("tiny", ("q",))["q"], a["q"])


def test_distributions():
    d = synth.make("1k", ("x", "w_dkv", "gain"))
    x = synth.bf16_bits_to_f32(d["x"])
    w = synth.bf16_bits_to_f32(d["w_dkv"])
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert abs(w.std() * np.sqrt(7168) - 1) < 0.01
    g = d["gain"]
    assert abs(g.mean() - 1) < 0.05 and abs(g.std() - np.sqrt(0.1)) < 0.05
    assert np.array_equal(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(g)), g)


def test_bf16_bit_helpers_round_to_nearest_even():
    v = np.array([1.0, 1.00390625, 1.01171875, -2.5, 0.0], np.float32)
    bits = synth.f32_to_bf16_bits(v)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0000]
