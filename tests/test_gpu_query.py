"""GPU parity of the query path (wq_a, q_norm, wq_b, rotary of each head's rotary part) through
the C ABI.

Each step is checked from the GPU's own input to that step: the GEMM outputs within one bf16
step plus the fp32 accumulation bound, the norm within one bf16 step (the norm's criterion), the
rotated part within one step plus one step of each of its two bf16 inputs (the GPU rotates its own
rounded product, which may sit one step from the oracle's); end to end from x by rel-L2."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import query as qo
import sparse_latent_attention_wkv_amd as mla

from _gpu import assert_within_one_step, bf16_step, dev, fp32_dot_bound, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def f32(bits):
    return synth.bf16_bits_to_f32(bits)


def _inputs(seed, B, T):
    x = synth.random_bf16(seed, (B, T, 7168))
    w_qa = synth.random_bf16(seed + 1, (1536, 7168), 7168 ** -0.5)
    gain = oracle.bf16(1 + np.sqrt(0.1) * np.random.default_rng(seed + 2).standard_normal(1536))
    w_qb = synth.random_bf16(seed + 3, (128 * 192, 1536), 1536 ** -0.5)
    return x, w_qa, gain.astype(np.float32), w_qb


def _check_rows(x, w_qa, gain, w_qb, qa, qr, q, rows_bt, sp):
    """rows_bt: (b, t) pairs to check against the oracle, from the GPU's intermediates."""
    xa = f32(x).astype(np.float64)
    wa = f32(w_qa).astype(np.float64)
    wb = f32(w_qb).astype(np.float64)
    for b, t in rows_bt:
        xr = xa[b, t]
        ref_qa = oracle.bf16(wa @ xr)
        assert_within_one_step(qa[b, t], ref_qa, extra=fp32_dot_bound(np.abs(wa) @ np.abs(xr), 7168),
                               what=f"qa[{b},{t}]")
        assert_within_one_step(qr[b, t], oracle.rms_norm(qa[b, t], gain), what=f"qr[{b},{t}]")
        qrr = qr[b, t].astype(np.float64)
        prod = wb @ qrr
        bound = fp32_dot_bound(np.abs(wb) @ np.abs(qrr), 1536).reshape(128, 192)
        pre = oracle.bf16(prod).reshape(128, 192)
        assert_within_one_step(q[b, t, :, :128], pre[:, :128], extra=bound[:, :128],
                               what=f"q_nope[{b},{t}]")
        ref_pe = oracle.rotary(pre[:, 128:], oracle.rope_angles(np.array([sp + t]))[0])
        re, im = pre[:, 128::2].astype(np.float64), pre[:, 129::2].astype(np.float64)
        pair = bf16_step(re) + bf16_step(im) + 2 * np.maximum(bound[:, 128::2], bound[:, 129::2]) \
            + 4 * 2.0 ** -24 * np.hypot(re, im)
        assert_within_one_step(q[b, t, :, 128:], ref_pe, extra=pair.repeat(2, -1),
                               what=f"q_pe[{b},{t}]")


CASES = [(1, 64, 0), (2, 77, 13), (1, 1, 0), (1, 3, 5), (2, 150, 2), (1, 300, 4000), (3, 130, 0)]


@pytest.mark.parametrize("B,T,sp", CASES)
def test_query_path_matches_oracle(B, T, sp):
    say(f"q_path B={B} T={T} start_pos={sp}")
    x, w_qa, gain, w_qb = _inputs(7000 + T + sp, B, T)
    qa_t, qr_t, q_t = mla.mla_q_path(to_dev(x), to_dev(w_qa), torch.from_numpy(gain).to(dev()),
                                     to_dev(w_qb), start_pos=sp)
    torch.cuda.synchronize()
    qa, qr, q = to_host(qa_t), to_host(qr_t), to_host(q_t)
    rng = np.random.default_rng(T)
    rows = [(b, t) for b in range(B) for t in sorted(set([0, T - 1] + list(rng.integers(0, T, 6))))]
    _check_rows(x, w_qa, gain, w_qb, qa, qr, q, rows, sp)
    # end to end from x on a few rows (the oracle numbers them 0.., so only the non-rotary part,
    # which does not depend on the position, is compared)
    sel = sorted(set([0, T - 1, T // 2]))
    _, _, q_ref = qo.query_path(f32(x)[:1, sel], f32(w_qa), gain, f32(w_qb))
    got = q[0, sel]
    rel = np.linalg.norm(got[..., :128] - q_ref[..., :128]) / np.linalg.norm(q_ref[..., :128])
    say(f"  end-to-end q_nope rel-L2 {rel:.2e}")
    assert rel < 1e-2


def test_query_path_headline_rows():
    """The headline shape (B=2, T=4096): 24 sampled rows of each output."""
    B, T = 2, 4096
    say(f"q_path B={B} T={T} sampled rows")
    x, w_qa, gain, w_qb = _inputs(7100, B, T)
    qa_t, qr_t, q_t = mla.mla_q_path(to_dev(x), to_dev(w_qa), torch.from_numpy(gain).to(dev()),
                                     to_dev(w_qb))
    torch.cuda.synchronize()
    qa, qr, q = to_host(qa_t), to_host(qr_t), to_host(q_t)
    rng = np.random.default_rng(7101)
    rows = [(int(b), int(t)) for b, t in zip(rng.integers(0, B, 24), rng.integers(0, T, 24))]
    rows += [(0, 0), (1, T - 1), (1, 127), (0, 128)]     # first and last rows of M tiles
    _check_rows(x, w_qa, gain, w_qb, qa, qr, q, rows, 0)
    assert np.isfinite(q).all()
