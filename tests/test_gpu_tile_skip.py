"""GPU checks of the attention's key-tile skipping.

mla_attn_prepare writes, after the selection bitmap, one flag per (256-query tile, 64-key tile)
that holds an allowed key for at least one of the tile's queries; the attention scores only the
flagged tiles. The flags are compared bit for bit with the oracle's allowed set, and the
attention with selections that leave whole tiles empty (a window of recent keys plus a few
leading keys, block-structured choices, query tiles without any allowed key) is compared with
the oracle like every other attention case.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import attention_close, dev, pack_mask, say, to_dev, to_host

mla = pytest.importorskip("sparse_latent_attention_wkv_amd")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]

SCALE = oracle.softmax_scale()
f32 = synth.bf16_bits_to_f32


def window_topk(B, T, window, sinks=4):
    """Each query selects its `window` most recent keys (itself included) and keys 0..sinks-1;
    positions before the sequence are -1."""
    s = np.arange(T)[:, None]
    win = s - np.arange(window)[None, :]
    win[win < 0] = -1
    sink = np.broadcast_to(np.arange(sinks)[None, :], (T, sinks))
    t = np.concatenate([win, sink], 1).astype(np.int32)
    return np.broadcast_to(t, (B, T, window + sinks)).copy()


def block_topk(seed, B, T, K, blocks_per_tile=3):
    """Per 256-query tile, a random choice of 64-key blocks; every query selects itself and up
    to K - 1 keys at random inside its tile's blocks (at or before itself), -1 elsewhere."""
    rng = np.random.default_rng(seed)
    out = np.full((B, T, K), -1, np.int32)
    for b in range(B):
        for q0 in range(0, T, 256):
            nblk = (min(T, q0 + 256) + 63) // 64
            blks = rng.choice(nblk, min(blocks_per_tile, nblk), replace=False)
            keys = np.concatenate([np.arange(64 * k, min(T, 64 * k + 64)) for k in blks])
            for s in range(q0, min(T, q0 + 256)):
                out[b, s, 0] = s
                cand = keys[keys < s]
                if len(cand):
                    pick = rng.choice(cand, min(K - 1, len(cand)), replace=False)
                    out[b, s, 1:1 + len(pick)] = pick
    return out


def flags_from_allowed(allowed):
    """allowed [B, T(query), T(key)] -> uint32 flags [B, ceil(T/256), ceil(ceil(T/64)/32)]:
    bit kt of tile qt is set when any (query, key) pair of the two tiles is allowed."""
    B, T, _ = allowed.shape
    nqt, nkt = (T + 255) // 256, (T + 63) // 64
    flags = np.zeros((B, nqt, (nkt + 31) // 32), np.uint32)
    for b in range(B):
        for qt in range(nqt):
            rows = allowed[b, 256 * qt:256 * qt + 256]
            for kt in range(nkt):
                if rows[:, 64 * kt:64 * kt + 64].any():
                    flags[b, qt, kt // 32] |= np.uint32(1 << (kt % 32))
    return flags


def flags_from_topk(topk):
    """The same flags straight from the index rows (valid entries at or before their query), for
    lengths where the dense allowed set is too large to form."""
    B, T, K = topk.shape
    nqt, nkt = (T + 255) // 256, (T + 63) // 64
    flags = np.zeros((B, nqt, (nkt + 31) // 32), np.uint32)
    for b in range(B):
        for qt in range(nqt):
            rows = topk[b, 256 * qt:256 * qt + 256].astype(np.int64)
            s = np.arange(256 * qt, 256 * qt + len(rows))[:, None]
            for kt in np.unique(rows[(rows >= 0) & (rows < T) & (rows <= s)] // 64):
                flags[b, qt, kt // 32] |= np.uint32(1 << int(kt % 32))
    return flags


def prepared(topk):
    B, T, K = topk.shape
    ws = torch.full((mla.mla_attn_workspace_bytes(B, T, K),), 0xA5, dtype=torch.uint8, device=dev())
    mla.mla_attn_prepare(torch.from_numpy(topk).to(dev()), ws)
    torch.cuda.synchronize()
    words = ws.cpu().numpy().view(np.uint32)
    Wp, Tpad = 2 * ((T + 63) // 64), 256 * ((T + 255) // 256)
    nbm = B * Wp * Tpad
    bitmap = words[:nbm].reshape(B, Wp, Tpad)
    nqt, fw = Tpad // 256, (Wp // 2 + 31) // 32
    flags = words[nbm:nbm + B * nqt * fw].reshape(B, nqt, fw)
    return bitmap, flags


CASES = {
    "uniform": lambda: synth.random_topk(5000, 1, 1100, 300),
    "window": lambda: window_topk(2, 2000, 100),
    "blocks": lambda: block_topk(5001, 2, 1300, 96),
    "long_window": lambda: window_topk(1, 12000, 64, sinks=1),
}


@pytest.mark.parametrize("case", list(CASES))
def test_prepare_writes_bitmap_and_tile_flags(case):
    topk = CASES[case]()
    B, T, K = topk.shape
    say(f"tile flags {case} B={B} T={T} K={K}")
    bitmap, flags = prepared(topk)
    want = flags_from_topk(topk)
    if T <= 4096:
        allowed = oracle.selection_mask(topk, T)
        plain = pack_mask(allowed)                                   # [B, ceil(T/32), T]
        W = plain.shape[1]
        assert np.array_equal(bitmap[:, :W, :T], plain)
        assert not bitmap[:, W:, :].any() and not bitmap[:, :, T:].any()
        assert np.array_equal(flags_from_allowed(allowed), want)
    assert np.array_equal(flags, want)
    nkt = (T + 63) // 64
    causal = sum(min(nkt, (min(T, 256 * qt + 256) - 1) // 64 + 1) for qt in range((T + 255) // 256))
    set_bits = sum(bin(int(w)).count("1") for w in want.ravel())
    say(f"  flagged key tiles {set_bits} of {causal * B} causal")


def _attention_case(topk, seed):
    B, T, K = topk.shape
    q = synth.random_bf16(seed, (B, T, 128, 192))
    kv = synth.random_bf16(seed + 1, (B, 128, T, 256))
    kpe = synth.random_bf16(seed + 2, (B, T, 64))
    out = mla.mla_sparse_prefill_attn(to_dev(q), to_dev(kv), to_dev(kpe), torch.from_numpy(topk).to(dev()), SCALE)
    torch.cuda.synchronize()
    return q, kv, kpe, to_host(out)


@pytest.mark.parametrize("case", ["window", "blocks"])
def test_attention_with_empty_key_tiles_matches_oracle(case):
    topk = CASES[case]()
    B, T, K = topk.shape
    say(f"attention with skipped tiles: {case} B={B} T={T} K={K}")
    q, kv, kpe, got = _attention_case(topk, 5100)
    ref = oracle.sparse_prefill_attn(f32(q), f32(kv), f32(kpe), topk, SCALE)
    attention_close(got, ref, case)


def test_attention_query_tiles_without_any_allowed_key_give_zeros():
    """Queries 256..767 of the second sequence select nothing (-1 everywhere): their work items
    have no flagged tile and their rows are zeros; every other row matches the oracle."""
    B, T, K = 2, 1000, 80
    topk = synth.random_topk(5200, B, T, K)
    topk[1, 256:768] = -1
    say(f"attention with empty query tiles B={B} T={T} K={K}")
    q, kv, kpe, got = _attention_case(topk, 5201)
    assert not got[1, 256:768].any()
    keep = np.ones((B, T), bool)
    keep[1, 256:768] = False
    for b in range(B):
        rows = np.flatnonzero(keep[b])
        ref = oracle.sparse_prefill_attn_rows(f32(q[b:b + 1]), f32(kv[b:b + 1]), f32(kpe[b:b + 1]),
                                              topk[b:b + 1], SCALE, 0, rows)
        attention_close(got[b, rows], ref, f"sequence {b}, rows with allowed keys")


def test_long_window_attention_sampled():
    """T = 12000 with a 64-key window and one leading key: at most seven flagged tiles per query
    tile, so the call does a small fraction of the causal tiles; sampled rows against the oracle."""
    topk = CASES["long_window"]()
    B, T, K = topk.shape
    say(f"long window attention B={B} T={T} K={K}")
    q, kv, kpe, got = _attention_case(topk, 5300)
    rows = np.array([0, 1, 63, 64, 255, 256, 4095, 8191, 8192, 10000, T - 1])
    ref = oracle.sparse_prefill_attn_rows(f32(q), f32(kv), f32(kpe), topk, SCALE, 0, rows)
    attention_close(got[0, rows], ref, "long window, sampled rows")
