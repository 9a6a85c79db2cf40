"""GPU check of mla_sparse_prefill_attn_noalloc, the attention entry point that allocates nothing
(its selection bitmap lives in the library's fixed per-device scratch): through the C ABI, its
output equals mla_sparse_prefill_attn's bit for bit, on two calls in a row of which the second is
smaller (the scratch keeps the first call's contents), and again after a larger one."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import dev, say, to_dev

mla = pytest.importorskip("sparse_latent_attention_wkv_amd")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]

SCALE = oracle.softmax_scale()


def _inputs(seed, B, T, K):
    q = to_dev(synth.random_bf16(seed, (B, T, 128, 192)))
    kv = to_dev(synth.random_bf16(seed + 1, (B, 128, T, 256)))
    kpe = to_dev(synth.random_bf16(seed + 2, (B, T, 64)))
    topk = torch.from_numpy(synth.random_topk(seed + 3, B, T, K)).to(dev())
    return q, kv, kpe, topk


def _both(q, kv, kpe, topk):
    B, T = q.shape[:2]
    out = torch.empty((B, T, 128, 128), dtype=torch.bfloat16, device=dev())
    got = mla.mla_sparse_prefill_attn_noalloc(q, kv, kpe, topk, SCALE, out=out)
    ref = mla.mla_sparse_prefill_attn(q, kv, kpe, topk, SCALE)
    torch.cuda.synchronize()
    return got, ref


def test_noalloc_matches_the_workspace_entry_point_on_consecutive_calls():
    for (B, T, K) in [(2, 1100, 300), (1, 200, 48), (1, 64, 16), (2, 4096, 2048), (1, 333, 400)]:
        say(f"noalloc attention B={B} T={T} K={K}, scratch {mla.mla_noalloc_scratch_bytes(B, T)} bytes")
        got, ref = _both(*_inputs(8800 + T + B, B, T, K))
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (B, T, K)
        assert torch.isfinite(got.float()).all()


def test_noalloc_rejects_problems_beyond_its_scratch():
    q, kv, kpe, topk = _inputs(8900, 1, 64, 16)
    with pytest.raises(mla.MLAError, match="SCRATCH"):
        # B = 17, T = 4096 would need 34 MiB; sizes are checked before any launch, so
        # the small tensors below are never read: pass them with a reshaped topk of that shape
        lib = mla.lib()
        st = lib.mla_sparse_prefill_attn_noalloc(mla._ptr(q), mla._ptr(kv), mla._ptr(kpe), mla._ptr(topk),
                                                 17, 4096, 16, SCALE, mla._ptr(q), mla._stream(q.device))
        mla._check(st)
