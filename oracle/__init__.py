"""CPU oracle for the sparse latent-attention prefill (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package. It shares no code with the GPU library.
"""
from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import (bf16, kv_down, kv_latent, kv_up, mla_prefill, parameter_shapes,  # noqa: F401
                         rms_norm, rope_angles, rotary, selection_mask, softmax_scale,
                         sparse_prefill_attn, sparse_prefill_attn_rows)
