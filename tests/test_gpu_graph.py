"""Decode steps of the V4.1 window-KV front end (256 sequences, one position each) captured once in
a HIP graph and replayed: the launch-bound inner loop of decoding, without a host launch per
step. Eight consecutive steps (positions start..start+7 written into a ring of 128 slots) are
captured on a side stream; each replay starts from the same ring contents, with the program's own
eager work and synchronisations between replays, and must reproduce the eager sequence bit for
bit (every step's output and the final ring)."""
import numpy as np
import pytest
import torch

import synth
from _gpu import dev, say, to_dev

mla = pytest.importorskip("sparse_latent_attention_wkv_amd")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def test_window_decode_steps_replayed_from_a_graph():
    B, W, N, sp0 = 256, 128, 8, 1000
    say(f"graph of {N} window-KV decode steps, B={B}, ring {W}")
    raw = [to_dev(synth.random_bf16(7000 + i, (B, 1, 512))) for i in range(N)]
    g = 1.0 + 0.1 * np.random.default_rng(7100).standard_normal(512)
    gain = torch.from_numpy(g.astype(np.float32)).to(dev())
    cs = mla.mla_rope_table(sp0 + N, dev())
    ring0 = to_dev(synth.random_bf16(7200, (B, W, 512)))

    ring_e = ring0.clone()
    outs_e = [mla.mla_window_kv(raw[i], gain, ring_e, start_pos=sp0 + i, rope_cs=cs) for i in range(N)]
    torch.cuda.synchronize()
    want = [_bits(o) for o in outs_e]
    want_ring = _bits(ring_e)

    ring_g = ring0.clone()
    outs_g = [torch.empty((B, 1, 512), dtype=torch.bfloat16, device=dev()) for _ in range(N)]
    side = torch.cuda.Stream(dev())
    side.wait_stream(torch.cuda.current_stream(dev()))
    with torch.cuda.stream(side):            # one eager pass on the capture stream first
        for i in range(N):
            mla.mla_window_kv(raw[i], gain, ring_g, start_pos=sp0 + i, rope_cs=cs, out=(outs_g[i],))
    torch.cuda.current_stream(dev()).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(N):
            mla.mla_window_kv(raw[i], gain, ring_g, start_pos=sp0 + i, rope_cs=cs, out=(outs_g[i],))
    torch.cuda.synchronize()
    for rep in range(3):
        ring_g.copy_(ring0)                   # eager work between the replays
        for o in outs_g:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(N):
            assert np.array_equal(_bits(outs_g[i]), want[i]), f"replay {rep}, step {i}"
        assert np.array_equal(_bits(ring_g), want_ring), f"replay {rep}, ring"
    say("  3 replays bit-identical to the eager steps")
