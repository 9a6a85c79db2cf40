"""Plain CPU oracle for the query path: low-rank query projection, query RMSNorm, per-head
up-projection and rotary rotation of the rotary part of every head.

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or run it. It shares no code with the
GPU library and imports nothing from it.

Sources: "DeepSeek-V3.2-Exp · Key-value down-projection", MLA constructor excerpt: ``wq_a`` maps
the hidden size to ``q_lora_rank``, ``q_norm`` is an RMSNorm over ``q_lora_rank`` (class default
eps), ``wq_b`` maps ``q_lora_rank`` to n_heads * qk_head_dim = 128 * 192; "DeepSeek-V3.2-Exp ·
Keys", MHA-prefill excerpt: the query is the concatenation [q_nope | q_pe] per head, and the
indexer receives the normalised low-rank query ``qr``.

Readings where the pages are silent (each is listed in the design notes):
* The query forward itself is not shown. Reading: qr = q_norm(wq_a(x)); q = wq_b(qr) viewed as
  [B, T, 128, 192] and split [128 | 64]; the 64-wide part of every head is rotated exactly as
  the shared key (adjacent pairs as complex numbers, angle pos * 10000^(-2i/64), pos =
  start_pos + t); each Linear output and the rotated part are rounded to bf16.
* ``q_lora_rank`` is not on the pages. Reading: 1536 (``Q_LORA_RANK``); the functions below
  take any width from the weights' shapes.

Pins: ``tests/test_oracle_query.py``.
"""
from __future__ import annotations

import numpy as np

from .mla_oracle import (HIDDEN, N_HEADS, QK_HEAD_DIM, QK_NOPE_HEAD_DIM, QK_ROPE_HEAD_DIM,
                         RMS_EPS_DEFAULT, ROPE_THETA, bf16, rms_norm, rope_angles, rotary)

Q_LORA_RANK = 1536


def query_parameter_shapes(q_lora_rank: int = Q_LORA_RANK) -> dict:
    """Weight shapes of the query modules as the MLA constructor builds them ([out, in])."""
    return {
        "wq_a": (q_lora_rank, HIDDEN),
        "q_norm": (q_lora_rank,),
        "wq_b": (N_HEADS * QK_HEAD_DIM, q_lora_rank),
    }


def query_path(x, w_qa, q_gain, w_qb, start_pos: int = 0, eps: float = RMS_EPS_DEFAULT,
               theta: float = ROPE_THETA, n_heads: int = N_HEADS):
    """x [B, T, 7168] -> (qa [B, T, r], qr [B, T, r], q [B, T, H, 192]).

    qa = bf16(x W_qa^T) (float64 products and sums); qr = the RMSNorm of qa with gain q_gain
    (float32, as the RMSNorm excerpt computes it); q = bf16(qr W_qb^T) viewed per head, with
    features 128..191 of every head rotated at position start_pos + t and rounded to bf16."""
    x = np.asarray(x, np.float64)
    w_qa = np.asarray(w_qa, np.float64)
    w_qb = np.asarray(w_qb, np.float64)
    if x.shape[-1] != w_qa.shape[1] or w_qb.shape[1] != w_qa.shape[0] \
            or w_qb.shape[0] != n_heads * QK_HEAD_DIM:
        raise ValueError("query weight shapes do not agree")
    B, T, _ = x.shape
    qa = bf16(x @ w_qa.T)
    qr = rms_norm(qa, q_gain, eps)
    q = bf16(np.asarray(qr, np.float64) @ w_qb.T).reshape(B, T, n_heads, QK_HEAD_DIM)
    ang = rope_angles(start_pos + np.arange(T), QK_ROPE_HEAD_DIM, theta)[:, None, :]   # [T, 1, 32]
    q_pe = rotary(q[..., QK_NOPE_HEAD_DIM:], ang)
    q = np.concatenate([q[..., :QK_NOPE_HEAD_DIM], q_pe], axis=-1).astype(np.float32)
    return qa, qr, q
