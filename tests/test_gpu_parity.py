"""GPU parity: every stage of the HIP path against the CPU oracle on the same seeded inputs.

Stage tests feed each kernel inputs whose oracle result is computed from the very same bf16
values (for downstream stages, the GPU's own upstream outputs), so a mismatch names its stage.
Criteria: GEMM outputs within one bf16 step plus the fp32 summation bound; normalised latent and
rotary key within one bf16 step; selection bitmap bit-exact; attention rel-L2 <= 1e-2 and
max-abs <= 2e-2; exact probes bitwise.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import (assert_within_one_step, attention_close, bf16_step, dev, f32_to_dev_bf16,
                  fp32_dot_bound, pack_mask, say, to_dev, to_host)

mla = pytest.importorskip("sparse_latent_attention_wkv_amd")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]

SCALE = oracle.softmax_scale()


def bf(seed, shape, std=1.0):
    return synth.random_bf16(seed, shape, std)


def f32(bits):
    return synth.bf16_bits_to_f32(bits)


# ------------------------------------------------------------------------------------ rotary table
@pytest.mark.parametrize("T", [1, 64, 4096, 16384])
def test_rope_table(T):
    say(f"rope table T={T}")
    cs = mla.mla_rope_table(T, dev()).cpu().numpy().astype(np.float64)
    ang = oracle.rope_angles(np.arange(T))
    assert np.abs(cs[..., 0] - np.cos(ang)).max() <= 6e-8
    assert np.abs(cs[..., 1] - np.sin(ang)).max() <= 6e-8


# ------------------------------------------------------------------------------------ norm + rotary
@pytest.mark.parametrize("rows,T,rope,eps", [(64, 64, True, 1e-6), (1000, 333, True, 1e-6),
                                             (256, 1, False, 1e-20), (8 * 4096, 4096, True, 1e-6),
                                             (3, 3, False, 1e-6)])
def test_norm_rope(rows, T, rope, eps):
    say(f"norm_rope rows={rows} T={T} rope={rope} eps={eps}")
    width = 576 if rope else 512
    raw = bf(100 + rows, (rows, width))
    gain = synth.make("tiny", ("gain",))["gain"]
    cs = mla.mla_rope_table(T, dev()) if rope else None
    c_kv, k_pe = mla.mla_kv_norm_rope(to_dev(raw), torch.from_numpy(gain).to(dev()), eps, cs, T)
    torch.cuda.synchronize()
    x = f32(raw)
    assert_within_one_step(to_host(c_kv), oracle.rms_norm(x[:, :512], gain, eps), what="c_kv")
    if rope:
        pe = x[:, 512:]
        ref = oracle.rotary(pe, oracle.rope_angles(np.arange(rows) % T))
        mag = np.hypot(pe[:, 0::2].astype(np.float64), pe[:, 1::2].astype(np.float64)).repeat(2, 1)
        assert_within_one_step(to_host(k_pe), ref, extra=4 * 2.0 ** -24 * mag, what="k_pe")


def test_norm_constant_rows_are_gain_times_sign():
    gain = synth.make("tiny", ("gain",))["gain"]
    rows = np.array([0.5, -3.0, 7.0, -0.0078125], np.float32)
    raw = np.repeat(rows[:, None], 512, 1)
    c_kv, _ = mla.mla_kv_norm_rope(f32_to_dev_bf16(raw), torch.from_numpy(gain).to(dev()), 1e-20)
    got = to_host(c_kv)
    want = oracle.bf16(gain[None, :] * np.sign(rows)[:, None])
    assert np.array_equal(got, want)


# ------------------------------------------------------------------------------------ front end
def _front_end_case(B, T, seed):
    d = synth.make(synth.Workload("case", B, T, None, seed), ("x", "w_dkv", "gain"))
    x, w, gain = d["x"], d["w_dkv"], d["gain"]
    kv_raw, c_kv, k_pe = mla.mla_kv_latent(to_dev(x), to_dev(w), torch.from_numpy(gain).to(dev()), 1e-6)
    torch.cuda.synchronize()
    return x, w, gain, to_host(kv_raw), to_host(c_kv), to_host(k_pe)


def _check_down(x_rows, w, got_rows):
    xf, wf = f32(x_rows).astype(np.float64), f32(w).astype(np.float64)
    ref = oracle.kv_down(f32(x_rows), f32(w))
    bound = fp32_dot_bound(np.abs(xf) @ np.abs(wf).T, 7168)
    assert_within_one_step(got_rows, ref, extra=bound, what="kv_raw")
    exact_or_step = np.abs(got_rows - ref) <= bf16_step(ref)
    assert exact_or_step.mean() >= 0.999


@pytest.mark.parametrize("B,T", [(1, 64), (2, 77), (1, 1024)])
def test_kv_latent(B, T):
    say(f"kv_latent B={B} T={T}")
    x, w, gain, kv_raw, c_kv, k_pe = _front_end_case(B, T, 2000 + T)
    _check_down(x.reshape(-1, 7168), w, kv_raw.reshape(-1, 576))
    # downstream steps from the GPU's own down-projection output
    assert_within_one_step(c_kv, oracle.rms_norm(kv_raw[..., :512], gain), what="c_kv")
    pe = kv_raw[..., 512:]
    ref = oracle.rotary(pe, oracle.rope_angles(np.arange(T)))
    mag = np.hypot(pe[..., 0::2].astype(np.float64), pe[..., 1::2].astype(np.float64)).repeat(2, -1)
    assert_within_one_step(k_pe, ref, extra=4 * 2.0 ** -24 * mag, what="k_pe")
    # end to end from x
    _, c_ref, kpe_ref = oracle.kv_latent(f32(x), f32(w), gain)
    rel = np.linalg.norm(c_kv - c_ref) / np.linalg.norm(c_ref)
    say(f"  end-to-end c_kv rel-L2 {rel:.2e}")
    assert rel < 1e-2


def test_kv_latent_frontend_workload_sampled():
    """The latent front-end workload, x [8, 4096, 7168]: sampled rows of the GEMM, every row of
    the norm/rotary step."""
    w = synth.WORKLOADS["frontend"]
    say("kv_latent frontend B=8 T=4096")
    x, wd, gain, kv_raw, c_kv, k_pe = _front_end_case(w.B, w.T, w.seed)
    rng = np.random.default_rng(7)
    rows = np.concatenate([[0, 1, 4095, 4096, 8 * 4096 - 1], rng.integers(0, 8 * 4096, 59)])
    _check_down(x.reshape(-1, 7168)[rows], wd, kv_raw.reshape(-1, 576)[rows])
    assert_within_one_step(c_kv, oracle.rms_norm(kv_raw[..., :512], gain), what="c_kv")
    pe = kv_raw[..., 512:]
    ref = oracle.rotary(pe, oracle.rope_angles(np.arange(w.T)))
    mag = np.hypot(pe[..., 0::2].astype(np.float64), pe[..., 1::2].astype(np.float64)).repeat(2, -1)
    assert_within_one_step(k_pe, ref, extra=4 * 2.0 ** -24 * mag, what="k_pe")


# ------------------------------------------------------------------------------------ up-projection
def _check_up(c_rows, w, got):       # c_rows [n, 512], got [n, 128, 256]
    cf, wf = f32(c_rows).astype(np.float64), f32(w).astype(np.float64)
    ref = oracle.kv_up(f32(c_rows)[None], f32(w))[0].transpose(1, 0, 2)      # [n, H, 256]
    bound = fp32_dot_bound(np.abs(cf) @ np.abs(wf).T, 512).reshape(ref.shape)
    assert_within_one_step(got, ref, extra=bound, what="kv")
    assert (np.abs(got - ref) <= bf16_step(ref)).mean() >= 0.999


@pytest.mark.parametrize("B,T", [(1, 64), (2, 77), (1, 1024), (3, 5), (9, 33), (3, 700)])
def test_kv_up(B, T):
    """(3, 5) and (9, 33): sequences shorter than a 32-token output block, and blocks that
    cross one sequence boundary, so the epilogue's row-to-(sequence, position) stepping is used.
    (1, 1024) and (3, 700): several tiles per persistent workgroup, the latter with a ragged last
    token tile (2100 tokens), so the next tile's loads overlap an epilogue."""
    say(f"kv_up B={B} T={T}")
    c = bf(3000 + T, (B, T, 512))
    w = synth.make("tiny", ("w_ukv",))["w_ukv"]
    kv = to_host(mla.mla_kv_up(to_dev(c), to_dev(w)))
    assert kv.shape == (B, 128, T, 256)
    for b in range(B):
        _check_up(c[b], w, kv[b].transpose(1, 0, 2))


# ------------------------------------------------------------------------------------ selection
def _garbage_topk(seed, B, T, K):
    rng = np.random.default_rng(seed)
    t = rng.integers(-3, T + 5, (B, T, K)).astype(np.int32)
    t[..., 0] = np.arange(T)[None]                 # self
    t[..., 1] = t[..., 2]                          # a duplicate
    return t


@pytest.mark.parametrize("case", ["tiny", "ragged", "garbage", "kgt", "1k", "headline"])
def test_selection_bitmap_bit_exact(case):
    if case == "tiny":
        topk = synth.make("tiny", ("topk",))["topk"]
    elif case == "ragged":
        topk = synth.random_topk(11, 2, 100, 37)      # K not a multiple of 4
    elif case == "garbage":
        topk = _garbage_topk(12, 2, 257, 64)
    elif case == "kgt":
        topk = synth.random_topk(13, 1, 45, 300)      # K > T
    elif case == "1k":
        topk = synth.make("1k", ("topk",))["topk"]
    else:
        topk = synth.make("headline", ("topk",))["topk"]
    B, T, K = topk.shape
    say(f"bitmap {case} B={B} T={T} K={K}")
    bm = mla.mla_selection_bitmap(torch.from_numpy(topk).to(dev())).cpu().numpy().view(np.uint32)
    want = pack_mask(oracle.selection_mask(topk, T))
    assert bm.shape == want.shape
    assert np.array_equal(bm, want)


# ------------------------------------------------------------------------------------ attention
def _attn_inputs(seed, B, T, K):
    q = bf(seed, (B, T, 128, 192))
    kv = bf(seed + 1, (B, 128, T, 256))
    kpe = bf(seed + 2, (B, T, 64))
    topk = synth.random_topk(seed + 3, B, T, K)
    return q, kv, kpe, topk


def _run_attn(q, kv, kpe, topk, scale=SCALE):
    out = mla.mla_sparse_prefill_attn(to_dev(q) if isinstance(q, np.ndarray) else q,
                                      to_dev(kv) if isinstance(kv, np.ndarray) else kv,
                                      to_dev(kpe) if isinstance(kpe, np.ndarray) else kpe,
                                      torch.from_numpy(topk).to(dev()), scale)
    torch.cuda.synchronize()
    return to_host(out)


# (1, 1100, 300): five query tiles of 256 (an odd count: the middle tile is a unit of its own)
# and more units than workgroups, so workgroups of the persistent grid take two units.
@pytest.mark.parametrize("B,T,K", [(1, 64, 16), (2, 200, 48), (1, 1024, 256), (1, 333, 400),
                                   (1, 1, 1), (3, 130, 7), (1, 1100, 300)])
def test_attention_matches_oracle(B, T, K):
    say(f"attention B={B} T={T} K={K}")
    q, kv, kpe, topk = _attn_inputs(4000 + T + K, B, T, K)
    got = _run_attn(q, kv, kpe, topk)
    ref = oracle.sparse_prefill_attn(f32(q), f32(kv), f32(kpe), topk, SCALE)
    attention_close(got, ref, f"B{B} T{T} K{K}")
    # query 0 attends only to key 0: its output is that key's value row, exactly
    assert np.array_equal(got[:, 0], f32(kv)[:, :, 0, 128:])


def test_attention_full_selection_is_dense_causal():
    B, T = 1, 300
    q, kv, kpe, _ = _attn_inputs(4100, B, T, 1)
    topk = np.tile(np.arange(T, dtype=np.int32), (B, T, 1))
    got = _run_attn(q, kv, kpe, topk)
    ref = oracle.sparse_prefill_attn(f32(q), f32(kv), f32(kpe), topk, SCALE)
    attention_close(got, ref, "full selection")


def test_attention_self_only_returns_values_exactly():
    B, T = 2, 300
    q, kv, kpe, _ = _attn_inputs(4200, B, T, 1)
    topk = np.arange(T, dtype=np.int32)[None, :, None].repeat(B, 0).copy()
    got = _run_attn(q, kv, kpe, topk)
    assert np.array_equal(got, f32(kv)[..., 128:].transpose(0, 2, 1, 3))


def test_attention_one_hot_probe_reads_off_the_selection():
    """q = 0 gives uniform weights over A(s); V[h, t, j] = [t == 128h + j] then makes
    out[s, h, j] = 1/|A(s)| exactly where key 128h + j is allowed, and exactly 0 elsewhere."""
    B, T, K = 1, 700, 90
    topk = synth.random_topk(4300, B, T, K)
    q = np.zeros((B, T, 128, 192), np.uint16)
    kv = np.zeros((B, 128, T, 256), np.float32)
    for t in range(T):
        kv[0, t // 128, t, 128 + t % 128] = 1.0
    kpe = bf(4301, (B, T, 64))
    got = _run_attn(q, synth.f32_to_bf16_bits(kv), kpe, topk)
    allowed = oracle.selection_mask(topk, T)[0]                    # [s, t]
    probe = np.zeros((T, 128 * 128), bool)
    probe[:, :T] = allowed
    nz = got[0].reshape(T, 128 * 128) != 0
    assert np.array_equal(nz, probe)
    cnt = allowed.sum(1)
    want = oracle.bf16(1.0 / cnt)
    vals = got[0].reshape(T, -1)
    for s in range(T):
        v = vals[s, :T][allowed[s]]
        assert np.all(np.abs(v - want[s]) <= bf16_step(want[s])), s


def test_attention_ignores_poisoned_unselected_keys_and_index_order():
    B, T, K = 1, 400, 60
    q, kv, kpe, _ = _attn_inputs(4400, B, T, K)
    rng = np.random.default_rng(3)
    topk = np.full((B, T, K), -1, np.int32)
    for s in range(T):
        cand = np.array([t for t in range(s + 1) if t % 3 != 1])
        pick = rng.choice(cand, min(K - 1, len(cand)), replace=False)
        topk[0, s, :len(pick)] = pick
        topk[0, s, len(pick)] = 0
    base = _run_attn(q, kv, kpe, topk)
    ref = oracle.sparse_prefill_attn(f32(q), f32(kv), f32(kpe), topk, SCALE)
    attention_close(base, ref, "structured selection")
    kvp, kpep = f32(kv).copy(), f32(kpe).copy()
    never = np.arange(T) % 3 == 1
    kvp[0][:, never, :] = 1e4 * np.where(rng.random((128, never.sum(), 256)) < 0.5, -1, 1)
    kpep[0][never] = -1e4
    poisoned = _run_attn(q, synth.f32_to_bf16_bits(kvp), synth.f32_to_bf16_bits(kpep), topk)
    assert np.array_equal(poisoned, base)
    shuffled = topk.copy()
    for s in range(T):
        shuffled[0, s] = rng.permutation(shuffled[0, s])       # moves the -1 pads too
    assert np.array_equal(_run_attn(q, kv, kpe, shuffled), base)
    # bitwise deterministic
    assert np.array_equal(_run_attn(q, kv, kpe, topk), base)


def test_prepared_attention_on_a_second_stream_matches_one_call():
    """mla_attn_prepare on another stream (ordered with an event) followed by
    mla_sparse_prefill_attn_prepared gives the one-call result bit for bit; a stale workspace
    from another selection is fully overwritten."""
    B, T, K = 2, 300, 64
    say(f"prepared attention B={B} T={T} K={K}")
    q, kv, k_pe, topk = _attn_inputs(4500, B, T, K)
    qd, kvd, ped = to_dev(q), to_dev(kv), to_dev(k_pe)
    tk = torch.from_numpy(topk).to(dev())
    scale = mla.mla_default_softmax_scale()
    one = mla.mla_sparse_prefill_attn(qd, kvd, ped, tk, scale)
    ws = torch.empty(mla.mla_attn_workspace_bytes(B, T, K), dtype=torch.uint8, device=dev())
    other = torch.from_numpy(synth.random_topk(4501, B, T, K)).to(dev())
    mla.mla_attn_prepare(other, ws)                      # stale contents first
    side = torch.cuda.Stream(dev())
    main = torch.cuda.current_stream(dev())
    start = torch.cuda.Event()
    start.record(main)
    side.wait_event(start)
    mla.mla_attn_prepare(tk, ws, stream=side)
    ready = torch.cuda.Event()
    ready.record(side)
    main.wait_event(ready)
    two = mla.mla_sparse_prefill_attn_prepared(qd, kvd, ped, ws, scale)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))
