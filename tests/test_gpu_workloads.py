"""GPU parity at the full workload sizes, through the same three library calls the benchmark
times (mla_kv_latent, mla_kv_up, mla_sparse_prefill_attn).

The oracle checks sampled outputs (sampled token rows of the projections, sampled query rows of
the attention, each from the GPU's own upstream tensors); the latent norm/rotary step and the
selection bitmap are checked on every row, and the headline attention on every output. The 1k
workload is small enough for the oracle to compute every output of the path.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import (assert_within_one_step, attention_close, dev, fp32_dot_bound,
                  pack_mask, say, to_dev, to_host)

mla = pytest.importorskip("sparse_latent_attention_wkv_amd")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]

SCALE = oracle.softmax_scale()
f32 = synth.bf16_bits_to_f32


def run_path(w):
    say(f"workload {w.name}: drawing inputs")
    d = synth.make(w)
    say(f"workload {w.name}: running the three calls")
    x, wd, wu, q = to_dev(d["x"]), to_dev(d["w_dkv"]), to_dev(d["w_ukv"]), to_dev(d["q"])
    gain = torch.from_numpy(d["gain"]).to(dev())
    topk = torch.from_numpy(d["topk"]).to(dev())
    kv_raw, c_kv, k_pe = mla.mla_kv_latent(x, wd, gain, 1e-6)
    kv = mla.mla_kv_up(c_kv, wu)
    out = mla.mla_sparse_prefill_attn(q, kv, k_pe, topk, SCALE)
    out2 = mla.mla_sparse_prefill_attn(q, kv, k_pe, topk, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "attention is not deterministic"
    return d, kv_raw, c_kv, k_pe, kv, out


def check_front_end(d, kv_raw_t, c_kv_t, k_pe_t, rows):
    B, T = d["x"].shape[:2]
    kv_raw = to_host(kv_raw_t).reshape(-1, 576)
    xr = d["x"].reshape(-1, 7168)[rows]
    ref = oracle.kv_down(f32(xr), f32(d["w_dkv"]))
    bound = fp32_dot_bound(np.abs(f32(xr)).astype(np.float64) @ np.abs(f32(d["w_dkv"])).astype(np.float64).T, 7168)
    assert_within_one_step(kv_raw[rows], ref, extra=bound, what="kv_raw")
    c_kv = to_host(c_kv_t).reshape(-1, 512)
    assert_within_one_step(c_kv, oracle.rms_norm(kv_raw[:, :512], d["gain"]), what="c_kv")
    pe = kv_raw[:, 512:]
    ref = oracle.rotary(pe, oracle.rope_angles(np.arange(B * T) % T))
    mag = np.hypot(pe[:, 0::2].astype(np.float64), pe[:, 1::2].astype(np.float64)).repeat(2, -1)
    assert_within_one_step(to_host(k_pe_t).reshape(-1, 64), ref, extra=4 * 2.0 ** -24 * mag, what="k_pe")
    return c_kv


def check_up(d, c_kv, kv_t, rows, T):
    wu = f32(d["w_ukv"])
    for m in rows:
        b, t = divmod(int(m), T)
        got = to_host(kv_t[b, :, t, :])                                      # [128, 256]
        ref = oracle.kv_up(c_kv[m][None, None], wu)[0, :, 0, :]
        bound = fp32_dot_bound(np.abs(c_kv[m]).astype(np.float64) @ np.abs(wu).astype(np.float64).T, 512)
        assert_within_one_step(got, ref, extra=bound.reshape(128, 256), what=f"kv row {m}")


def check_attention_rows(d, kv_t, k_pe_t, out_t, b, rows):
    q = f32(d["q"][b:b + 1])
    kv = to_host(kv_t[b:b + 1])
    kpe = to_host(k_pe_t[b:b + 1])
    ref = oracle.sparse_prefill_attn_rows(q, kv, kpe, d["topk"][b:b + 1], SCALE, 0, rows)
    got = to_host(out_t[b, rows])
    attention_close(got, ref, f"batch {b}, {len(rows)} sampled rows")
    # the first query sees only key 0: its output is that key's value row, exactly
    if 0 in rows:
        i = list(rows).index(0)
        assert np.array_equal(got[i], kv[0, :, 0, 128:])


def test_headline_workload_sampled():
    w = synth.WORKLOADS["headline"]
    d, kv_raw, c_kv, k_pe, kv, out = run_path(w)
    B, T, K = w.B, w.T, w.K
    say("checking selection bitmap (all rows)")
    bm = mla.mla_selection_bitmap(torch.from_numpy(d["topk"]).to(dev())).cpu().numpy().view(np.uint32)
    assert np.array_equal(bm, pack_mask(oracle.selection_mask(d["topk"], T)))
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([[0, 1, 4095, 4096, B * T - 1], rng.integers(0, B * T, 27)]))
    say("checking front end")
    c = check_front_end(d, kv_raw, c_kv, k_pe, rows)
    say("checking up-projection rows")
    check_up(d, c, kv, rows[:12], T)
    for b in range(B):
        qrows = sorted(set([0, 1, 31, 32, K - 1, K, K + 1, T - 1] + rng.integers(0, T, 16).tolist()))
        say(f"checking attention rows of batch {b}")
        check_attention_rows(d, kv, k_pe, out, b, qrows)


def test_headline_attention_every_output():
    """Every output of the headline attention (both sequences, all 128 heads, every query row)
    against the oracle's dense-masked form on the GPU's own keys, values and rotary keys: the
    persistent kernel's pairing of query tiles and its per-XCD walk over heads is checked on all
    of its work items."""
    w = synth.WORKLOADS["headline"]
    d, kv_raw, c_kv, k_pe, kv, out = run_path(w)
    for b in range(w.B):
        say(f"oracle on all of batch {b} ({w.T} queries x 128 heads)")
        q = f32(d["q"][b:b + 1])
        ref = oracle.sparse_prefill_attn(q, to_host(kv[b:b + 1]), to_host(k_pe[b:b + 1]),
                                         d["topk"][b:b + 1], SCALE)
        attention_close(to_host(out[b:b + 1]), ref, f"headline batch {b}, every output")


def test_long_workload_sampled():
    w = synth.WORKLOADS["long"]
    d, kv_raw, c_kv, k_pe, kv, out = run_path(w)
    T, K = w.T, w.K
    rng = np.random.default_rng(32)
    rows = np.unique(np.concatenate([[0, 1, T // 2, T - 1], rng.integers(0, T, 12)]))
    say("checking front end")
    c = check_front_end(d, kv_raw, c_kv, k_pe, rows)
    say("checking up-projection rows")
    check_up(d, c, kv, rows[:6], T)
    qrows = sorted(set([0, 1, K - 1, K, 8191, 12000, T - 2, T - 1] + rng.integers(0, T, 8).tolist()))
    say("checking attention rows")
    check_attention_rows(d, kv, k_pe, out, 0, qrows)


def test_1k_workload_every_output():
    w = synth.WORKLOADS["1k"]
    d, kv_raw, c_kv, k_pe, kv, out = run_path(w)
    say("oracle on the whole 1k workload")
    ref = oracle.mla_prefill(f32(d["x"]), f32(d["w_dkv"]), d["gain"], f32(d["w_ukv"]), f32(d["q"]),
                             d["topk"], SCALE)
    # stage by stage from the GPU's own inputs
    kvr = to_host(kv_raw)
    assert_within_one_step(to_host(c_kv), oracle.rms_norm(kvr[..., :512], d["gain"]), what="c_kv")
    kvg = to_host(kv)
    kpe = to_host(k_pe)
    got = to_host(out)
    attention_close(got, oracle.sparse_prefill_attn(f32(d["q"]), kvg, kpe, d["topk"], SCALE), "1k attention")
    ckv = to_host(c_kv)
    wu = f32(d["w_ukv"])
    kv_ref = oracle.kv_up(ckv, wu)
    bound = fp32_dot_bound(np.abs(ckv[0]).astype(np.float64) @ np.abs(wu).astype(np.float64).T, 512)
    bound = bound.reshape(1, -1, 128, 256).transpose(0, 2, 1, 3)
    assert_within_one_step(kvg, kv_ref, extra=bound, what="kv")
    # end to end from x: report, and bound loosely (bf16 re-rounding of every stage)
    rel = np.linalg.norm(got - ref["out"]) / np.linalg.norm(ref["out"])
    say(f"  end-to-end rel-L2 from x: {rel:.3e}")
    assert rel < 3e-2
