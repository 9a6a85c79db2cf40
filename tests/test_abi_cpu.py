"""The C ABI on the host: libmla.so loads, exports every function include/mla.h declares, and
rejects bad arguments before any HIP call (no GPU needed; no kernel is launched here)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

mla = pytest.importorskip("sparse_latent_attention_wkv_amd")


def _lib():
    if not os.path.exists(mla.LIB_PATH):
        pytest.fail("libmla.so is not built (run __graft_entry__.build())")
    return mla.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_path_calls():
    names = declared_functions()
    for n in ("mla_kv_latent", "mla_kv_up", "mla_sparse_prefill_attn"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in mla._SIGS, f"binding does not declare {name}"


def test_host_only_helpers():
    lib = _lib()
    s = lib.mla_default_softmax_scale()
    m = 1 + 0.1 * math.log(40)
    assert s == pytest.approx(m * m / math.sqrt(192), rel=1e-7)
    assert lib.mla_status_string(0) == b"MLA_OK"
    for code in range(-9, 0):
        assert lib.mla_status_string(code).startswith(b"MLA_E_")
    assert b"gfx950" in lib.mla_build_info()
    # bitmap: B * (2 * ceil(T/64)) words x (256 * ceil(T/256)) query columns x 4 bytes; then the
    # key-tile flags, B * ceil(T/256) * ceil(ceil(T/64) / 32) words, rounded up to 256 bytes
    assert lib.mla_attn_workspace_bytes(2, 4096, 2048) == 2 * 128 * 4096 * 4 + 256
    assert lib.mla_attn_workspace_bytes(1, 100, 7) == 4 * 256 * 4 + 256
    assert lib.mla_attn_workspace_bytes(3, 16384, 2048) == 3 * 512 * 16384 * 4 + 3 * 64 * 8 * 4
    assert lib.mla_attn_workspace_bytes(1, 32768, 2048) == 1024 * 32768 * 4 + 128 * 16 * 4
    assert lib.mla_attn_workspace_bytes(0, 4096, 2048) == 0
    assert lib.mla_attn_workspace_bytes(1, 40000, 2048) == 0
    assert lib.mla_last_hip_error() == 0


# Fake but aligned addresses: every call below must fail validation before touching them.
A, B_, C, D, E, F, G = (0x100000 * i for i in range(1, 8))
NOSTREAM = None


def test_kv_latent_validation():
    lib = _lib()
    ok = dict(x=A, w=B_, g=C, eps=1e-6, cs=D, B=1, T=4, raw=E, ckv=F, kpe=G)

    def call(**kw):
        a = {**ok, **kw}
        return lib.mla_kv_latent(a["x"], a["w"], a["g"], a["eps"], a["cs"], a["B"], a["T"],
                                 a["raw"], a["ckv"], a["kpe"], NOSTREAM)
    assert call(x=None) == -1
    assert call(kpe=None) == -1
    assert call(B=0) == -2
    assert call(T=-3) == -2
    assert call(B=1 << 13, T=1 << 12) == -2            # B*T beyond MLA_MAX_ROWS
    assert call(x=A + 2) == -3
    assert call(ckv=F + 8) == -3
    assert call(eps=0.0) == -7
    assert call(eps=float("nan")) == -7
    assert call(raw=A) == -8                            # output overlapping x
    assert call(kpe=F) == -8                            # two outputs overlapping


def test_norm_rope_validation():
    lib = _lib()

    def call(src=A, rows=4, stride=576, rope=1, g=C, eps=1e-6, cs=D, T=4, ckv=E, kpe=F):
        return lib.mla_kv_norm_rope(src, rows, stride, rope, g, eps, cs, T, ckv, kpe, NOSTREAM)
    assert call(src=None) == -1
    assert call(cs=None) == -1
    assert call(rows=0) == -2
    assert call(stride=500) == -2
    assert call(stride=512, rope=1) == -2               # rotary needs the 576-wide rows
    assert call(T=0) == -2
    assert call(g=C + 4) == -3
    assert call(eps=-1.0) == -7
    assert call(ckv=A + 16) == -8


def test_kv_up_validation():
    lib = _lib()
    assert lib.mla_kv_up(None, B_, 1, 4, C, NOSTREAM) == -1
    assert lib.mla_kv_up(A, B_, 0, 4, C, NOSTREAM) == -2
    assert lib.mla_kv_up(A, B_ + 2, 1, 4, C, NOSTREAM) == -3
    assert lib.mla_kv_up(A, B_, 1, 4, B_ + 1024, NOSTREAM) == -8


def test_attention_and_bitmap_validation():
    lib = _lib()
    ws = lib.mla_attn_workspace_bytes(1, 64, 16)

    def call(q=A, kv=B_, kpe=C, topk=D, B=1, T=64, K=16, scale=0.135, out=E, w=F, wsb=ws):
        return lib.mla_sparse_prefill_attn(q, kv, kpe, topk, B, T, K, scale, out, w, wsb, NOSTREAM)
    assert call(topk=None) == -1
    assert call(w=None) == -1
    assert call(K=0) == -2
    assert call(T=40000) == -2
    assert call(K=70000) == -2
    assert call(out=E + 4) == -3
    assert call(wsb=ws - 1) == -4
    assert call(scale=0.0) == -7
    assert call(scale=float("inf")) == -7
    assert call(out=A + 64) == -8
    assert call(w=E) == -8
    assert lib.mla_selection_bitmap(None, 1, 64, 16, E, NOSTREAM) == -1
    assert lib.mla_selection_bitmap(D, 1, 64, 16, None, NOSTREAM) == -1
    assert lib.mla_selection_bitmap(D, 1, 0, 16, E, NOSTREAM) == -2
    assert lib.mla_selection_bitmap(D + 4, 1, 64, 16, E, NOSTREAM) == -3
    assert lib.mla_selection_bitmap(D, 1, 64, 16, D, NOSTREAM) == -8
    assert lib.mla_rope_table(0, 10000.0, A, NOSTREAM) == -2
    assert lib.mla_rope_table(8, 10000.0, None, NOSTREAM) == -1
    assert lib.mla_rope_table(8, -1.0, A, NOSTREAM) == -7


def test_check_topk_validation():
    lib = _lib()

    def call(topk=D, B=1, T=64, K=16, counts=E):
        return lib.mla_check_topk(topk, B, T, K, counts, NOSTREAM)
    assert call(topk=None) == -1
    assert call(counts=None) == -1
    assert call(B=0) == -2
    assert call(T=40000) == -2
    assert call(K=0) == -2
    assert call(topk=D + 4) == -3
    assert call(counts=E + 8) == -3
    assert call(counts=D + 16) == -8                  # counts inside the selection


def test_noalloc_attention_validation():
    lib = _lib()
    assert mla.NOALLOC_SCRATCH_BYTES == (32 << 20) + (128 << 10)
    assert lib.mla_noalloc_scratch_bytes(2, 4096) == lib.mla_attn_workspace_bytes(2, 4096, 2048)
    assert lib.mla_noalloc_scratch_bytes(1, 16384) == (32 << 20) + 2048
    assert lib.mla_noalloc_scratch_bytes(16, 4096) <= mla.NOALLOC_SCRATCH_BYTES
    assert lib.mla_noalloc_scratch_bytes(17, 4096) > mla.NOALLOC_SCRATCH_BYTES
    assert lib.mla_noalloc_scratch_bytes(0, 64) == 0

    def call(q=A, kv=B_, kpe=C, topk=D, B=1, T=64, K=16, scale=0.135, out=E):
        return lib.mla_sparse_prefill_attn_noalloc(q, kv, kpe, topk, B, T, K, scale, out, NOSTREAM)
    assert call(q=None) == -1
    assert call(out=None) == -1
    assert call(K=0) == -2
    assert call(T=40000) == -2
    assert call(out=E + 4) == -3
    assert call(scale=-1.0) == -7
    assert call(out=A + 64) == -8
    assert call(T=32768) == -9                        # bitmap of 128 MiB: beyond the scratch
    assert call(B=17, T=4096) == -9                   # 34 MiB
    assert call(B=16, T=4096, out=A + 64) == -8       # 32 MiB fits; then the alias check
    assert lib.mla_status_string(-9).startswith(b"MLA_E_SCRATCH")


def test_latent_attention_and_lists_validation():
    lib = _lib()
    assert lib.mla_selection_list_stride(4096, 2048) == 2048
    assert lib.mla_selection_list_stride(100, 2048) == 128
    assert lib.mla_selection_list_stride(64, 16) == 64
    assert lib.mla_selection_list_stride(0, 16) == 0
    ws = lib.mla_attn_latent_workspace_bytes(1, 64, 16)
    # transposed key weights, then per token: count, flag, list, absorbed query, latent output
    assert ws >= 128 * 512 * 128 * 2 + 64 * (4 + 4 + 4 * 64 + 2 * 128 * 512 * 2)
    assert ws % 256 == 0
    assert lib.mla_attn_latent_workspace_bytes(0, 64, 16) == 0
    assert lib.mla_attn_latent_workspace_bytes(1, 40000, 16) == 0
    GB = 1 << 30                        # far apart: the workspace spans tens of MB
    Q, CKV, KPE, W, TK, OUT, WS = (GB * i for i in range(1, 8))

    def call(q=Q, ckv=CKV, kpe=KPE, w=W, topk=TK, B=1, T=64, K=16, scale=0.135, out=OUT, wk=WS, wsb=ws):
        return lib.mla_sparse_prefill_attn_latent(q, ckv, kpe, w, topk, B, T, K, scale, out, wk, wsb,
                                                  NOSTREAM)
    assert call(q=None) == -1
    assert call(w=None) == -1
    assert call(wk=None) == -1
    assert call(B=0) == -2
    assert call(T=40000) == -2
    assert call(ckv=CKV + 2) == -3
    assert call(wk=WS + 8) == -3
    assert call(wsb=ws - 1) == -4
    assert call(scale=-1.0) == -7
    assert call(out=Q) == -8
    assert call(wk=W) == -8
    assert lib.mla_selection_lists(None, 1, 64, 16, OUT, WS, NOSTREAM) == -1
    assert lib.mla_selection_lists(TK, 1, 64, 16, None, WS, NOSTREAM) == -1
    assert lib.mla_selection_lists(TK, 1, 0, 16, OUT, WS, NOSTREAM) == -2
    assert lib.mla_selection_lists(TK, 1, 64, 16, OUT + 4, WS, NOSTREAM) == -3
    assert lib.mla_selection_lists(TK, 1, 64, 16, TK, WS, NOSTREAM) == -8
    assert lib.mla_selection_lists(TK, 1, 64, 16, OUT, OUT + 64, NOSTREAM) == -8


def test_auto_split_and_validation():
    lib = _lib()
    assert lib.mla_attn_auto_split(16384, 2048) == 8192
    assert lib.mla_attn_auto_split(4096, 2048) == 4096          # every row head-major
    assert lib.mla_attn_auto_split(1100, 100) == 256
    assert lib.mla_attn_auto_split(300, 40) == 0                # every row in the latent form
    assert lib.mla_attn_auto_split(0, 16) == -1
    assert lib.mla_attn_auto_workspace_bytes(0, 64, 16) == 0
    # all head-major: per-head keys/values, bitmap and key-tile flags of both sequences, no
    # latent part
    ws = lib.mla_attn_auto_workspace_bytes(2, 4096, 2048)
    assert ws == 2 * (128 * 4096 * 256 * 2 + 128 * 4096 * 4) + 256
    GB = 1 << 30
    Q, CKV, KPE, W, TK, OUT, WS = (GB * i for i in range(1, 8))
    wsb = lib.mla_attn_auto_workspace_bytes(1, 1100, 100)

    def call(q=Q, out=OUT, wk=WS, wsb=wsb, T=1100, scale=0.135):
        return lib.mla_sparse_prefill_attn_auto(q, CKV, KPE, W, TK, 1, T, 100, scale, out, wk, wsb, NOSTREAM)
    assert call(q=None) == -1
    assert call(T=0) == -2
    assert call(out=OUT + 2) == -3
    assert call(wsb=wsb - 1) == -4
    assert call(scale=float("nan")) == -7
    assert call(out=Q) == -8


def test_kv_latent_cache_validation():
    lib = _lib()
    MB = 1 << 26                                       # 64 MiB apart: caches span a few MB
    X, W, G_, CS, RAW, CKV, KPE, KC, PC, CN = (MB * i for i in range(1, 11))
    ok = dict(x=X, w=W, g=G_, eps=1e-6, cs=CS, B=2, T=8, sp=4, fmt=0, raw=RAW, ckv=CKV, kpe=KPE,
              kc=KC, pc=PC, cb=2, cl=16, cn=CN)

    def call(**kw):
        a = {**ok, **kw}
        return lib.mla_kv_latent_cache(a["x"], a["w"], a["g"], a["eps"], a["cs"], a["B"], a["T"],
                                       a["sp"], a["fmt"], a["raw"], a["ckv"], a["kpe"], a["kc"],
                                       a["pc"], a["cb"], a["cl"], a["cn"], NOSTREAM)

    def norm_call(**kw):
        a = {**ok, **kw}
        return lib.mla_kv_norm_rope_cache(a["raw"], a["B"], a["T"], a["sp"], a["g"], a["eps"],
                                          a["cs"], a["fmt"], a["ckv"], a["kpe"], a["kc"], a["pc"],
                                          a["cb"], a["cl"], a["cn"], NOSTREAM)
    for f in (call, norm_call):
        assert f() == -5                               # valid: only the device check fails here
        assert f(raw=None) == -1
        assert f(kc=None) == -1
        assert f(pc=None) == -1
        assert f(B=0) == -2
        assert f(sp=-1) == -2
        assert f(cl=11) == -2                          # start_pos + T = 12 > cache_len
        assert f(cb=1) == -2                           # cache_batch < B
        assert f(kc=KC + 2) == -3
        assert f(cn=CN + 8) == -3
        assert f(fmt=2) == -7
        assert f(eps=0.0) == -7
        assert f(kc=CKV) == -8                         # cache overlapping the rounded latent
        assert f(pc=KC + 1024) == -8                   # the two caches overlapping
        assert f(cn=RAW) == -8
        assert f(cs=KC) == -8                          # rotary table inside an output
    assert call(x=None) == -1
    assert call(w=W + 4) == -3
    assert call(raw=X) == -8
    assert call(kc=W) == -8
    assert norm_call(ckv=RAW + 64) == -8               # output inside the input rows


def test_window_kv_validation():
    lib = _lib()
    MB = 1 << 24
    RAW, G_, CS, OUT, WC, PRE = (MB * i for i in range(1, 7))
    ok = dict(raw=RAW, B=4, S=1, sp=100, g=G_, eps=1e-20, cs=CS, fmt=1, win=8, out=OUT, wc=WC,
              cb=4, pre=PRE)

    def call(**kw):
        a = {**ok, **kw}
        return lib.mla_window_kv(a["raw"], a["B"], a["S"], a["sp"], a["g"], a["eps"], a["cs"],
                                 a["fmt"], a["win"], a["out"], a["wc"], a["cb"], a["pre"], NOSTREAM)
    assert call() == -5
    assert call(pre=None) == -5
    assert call(raw=None) == -1
    assert call(wc=None) == -1
    assert call(out=None) == -1
    assert call(S=0) == -2
    assert call(win=0) == -2
    assert call(cb=3) == -2
    assert call(sp=-5) == -2
    assert call(sp=(1 << 24)) == -2                    # positions beyond MLA_MAX_ROWS
    assert call(pre=PRE + 4) == -3
    assert call(fmt=-1) == -7
    assert call(eps=float("inf")) == -7
    assert call(out=RAW) == -8
    assert call(pre=OUT) == -8
    assert call(wc=CS) == -8


def test_q_path_validation():
    lib = _lib()
    MB = 1 << 27
    X, WA, G_, WB, CS, QA, QR, Q = (MB * i for i in range(1, 9))
    ok = dict(x=X, wa=WA, g=G_, eps=1e-6, wb=WB, cs=CS, B=2, T=16, sp=3, r=1536, qa=QA, qr=QR, q=Q)

    def call(**kw):
        a = {**ok, **kw}
        return lib.mla_q_path(a["x"], a["wa"], a["g"], a["eps"], a["wb"], a["cs"], a["B"], a["T"],
                              a["sp"], a["r"], a["qa"], a["qr"], a["q"], NOSTREAM)
    assert call() == -5
    assert call(x=None) == -1
    assert call(wb=None) == -1
    assert call(q=None) == -1
    assert call(B=0) == -2
    assert call(sp=-1) == -2
    assert call(r=1024) == -2                          # q_lora_rank is fixed at 1536
    assert call(qr=QR + 2) == -3
    assert call(eps=0.0) == -7
    assert call(qa=X) == -8
    assert call(q=QR + 64) == -8
    assert call(cs=Q) == -8


def test_attn_prepare_and_prepared_validation():
    lib = _lib()
    GB = 1 << 30
    Q, KV, KPE, TK, OUT, WS = (GB * i for i in range(1, 7))
    ws = lib.mla_attn_workspace_bytes(2, 256, 16)

    def prep(topk=TK, B=2, T=256, K=16, wk=WS, wsb=ws):
        return lib.mla_attn_prepare(topk, B, T, K, wk, wsb, NOSTREAM)

    def attn(q=Q, kv=KV, kpe=KPE, B=2, T=256, scale=0.135, out=OUT, wk=WS, wsb=ws):
        return lib.mla_sparse_prefill_attn_prepared(q, kv, kpe, B, T, scale, out, wk, wsb, NOSTREAM)
    assert prep() == -5 and attn() == -5
    assert prep(topk=None) == -1 and prep(wk=None) == -1
    assert prep(K=0) == -2 and prep(T=40000) == -2
    assert prep(wk=WS + 4) == -3
    assert prep(wsb=ws - 1) == -4
    assert prep(wk=TK) == -8                           # bitmap written over the indices
    assert attn(q=None) == -1 and attn(wk=None) == -1
    assert attn(B=0) == -2 and attn(T=40000) == -2
    assert attn(out=OUT + 2) == -3
    assert attn(wsb=ws - 1) == -4
    assert attn(scale=0.0) == -7
    assert attn(out=KV) == -8
    assert attn(out=WS) == -8                          # output over the prepared bitmap
