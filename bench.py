#!/usr/bin/env python3
"""Benchmark of the sparse latent-attention prefill on one MI355X.

One step = the whole hot path on one batch of seeded synthetic inputs already resident in HBM:
mla_kv_latent (down-projection + RMSNorm + rotary), mla_kv_up (up-projection) and
mla_sparse_prefill_attn (selection bitmap + sparse attention), all on one stream.
Default workload: B=2, T=4096, top-k 2048, 128 heads (the headline prefill shape).

Prints one JSON line. `value` is tokens/s of the whole path (B*T tokens per step). `roofline`
prices the dominant call (the attention) at its algorithmic work: 640 FLOP per selected
(query, head, key) = 2*192 for q.k plus 2*128 for p.v, against the bf16 dense MFMA peak.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.

`--path latent` replaces the up-projection and the head-major attention by
mla_sparse_prefill_attn_latent (the latent-space form for long sequences), `--path auto` by
mla_sparse_prefill_attn_auto (head-major rows below the split, latent above); the roofline keeps
the same algorithmic unit, and `latent_mfma_flop_per_launch` gives the FLOPs the latent form
executes.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0
METRIC = "MLA sparse-prefill tokens/s + % bf16 MFMA peak (T=4096, top-k 2048)"


def selected_pairs(topk: np.ndarray) -> int:
    """Number of (b, s, t) with t selected for query s and t <= s (set semantics)."""
    B, T, K = topk.shape
    n = 0
    s = np.arange(T)[:, None]
    for b in range(B):
        t = topk[b].astype(np.int64)
        ok = (t >= 0) & (t <= s)
        # distinct entries per row
        key = np.where(ok, t, -1)
        key.sort(axis=1)
        distinct = ok.sum(1) - ((key[:, 1:] == key[:, :-1]) & (key[:, 1:] >= 0)).sum(1)
        n += int(distinct.sum())
    return n


def traffic_record(kernel: str):
    """HBM bytes per launch measured with rocprofv3 counters, if the record matches the current
    kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.txt")
    src = os.path.join(ROOT, "sparse_latent_attention_wkv_amd", "csrc", "attn.hip")
    if not os.path.exists(path) or not os.path.exists(src):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if kv.get("source_sha") != sha or "bytes_per_launch" not in kv:
        return None
    return float(kv["bytes_per_launch"])


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_name() -> str:
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:   # noqa: BLE001
        return "unknown"


_POOL_STATE = {}


def _attn_heads(heads):
    """Worker: the oracle's attention for some heads (inputs inherited at fork)."""
    import oracle
    st = _POOL_STATE
    oracle.sparse_prefill_attn(st["q"], st["kv"], st["k_pe"], st["topk"], st["scale"], heads=heads)
    return len(heads)


def cpu_baseline_child(workload: str) -> dict:
    """The CPU oracle timed on the host cores (runs in a child process that never touches the GPU).

    The whole workload: its front end and up-projection for all tokens with BLAS on every core of
    the affinity mask, then the dense-masked attention of all 128 heads over a process pool (one
    worker per core of the mask, at most 16, one BLAS thread each, heads dealt round-robin). Then
    the tiny and 1k workloads end to end on one core (one process, one BLAS thread)."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    import oracle
    import synth
    f32 = synth.bf16_bits_to_f32
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(16, cores))
    w = synth.WORKLOADS[workload]
    d = synth.make(w)
    B, T = w.B, w.T
    scale = oracle.softmax_scale()
    with threadpool_limits(cores):
        t0 = time.perf_counter()
        kv_raw, c_kv, k_pe = oracle.kv_latent(f32(d["x"]), f32(d["w_dkv"]), d["gain"])
        t1 = time.perf_counter()
        kv = oracle.kv_up(c_kv, f32(d["w_ukv"]))
        t2 = time.perf_counter()
    _POOL_STATE.update(q=f32(d["q"]), kv=kv, k_pe=k_pe, topk=d["topk"], scale=scale)
    chunks = [list(range(i, 128, workers)) for i in range(workers)]
    ctx = mp.get_context("fork")
    with threadpool_limits(1):
        t3 = time.perf_counter()
        with ctx.Pool(workers) as pool:
            assert sum(pool.map(_attn_heads, chunks)) == 128
        t4 = time.perf_counter()
    total = (t1 - t0) + (t2 - t1) + (t4 - t3)
    one_core = {}
    with threadpool_limits(1):
        for name in ("tiny", "1k"):
            wl = synth.WORKLOADS[name]
            dd = synth.make(wl)
            s0 = time.perf_counter()
            oracle.mla_prefill(f32(dd["x"]), f32(dd["w_dkv"]), dd["gain"], f32(dd["w_ukv"]), f32(dd["q"]),
                               dd["topk"], scale)
            sec = time.perf_counter() - s0
            one_core[name] = {"tokens_per_s": wl.B * wl.T / sec, "seconds": round(sec, 2)}
    return {"value": B * T / total, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": (f"the whole workload ({B} x {T} tokens): front end + up-projection "
                       f"({t1 - t0:.1f} s + {t2 - t1:.1f} s, BLAS on {cores} cores), dense-masked "
                       f"attention of all 128 heads ({t4 - t3:.1f} s, {workers} worker processes x 1 "
                       f"BLAS thread); float64 NumPy"),
            "sample_seconds": round(t4 - t0, 2), "affinity_cores": cores, "cpu_model": _cpu_model(),
            "blas": _blas_name(), "one_core_end_to_end": one_core}


def cpu_baseline(workload: str) -> dict:
    """Run cpu_baseline_child in a fresh interpreter (a child process: this one holds the GPU)."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-only", "--workload", workload],
                       capture_output=True, text=True, timeout=900)
    if r.returncode != 0:
        return {"value": None, "unit": "tokens/s", "cores": None, "kind": "oracle",
                "sample": f"failed: {r.stderr[-500:]}"}
    return json.loads(r.stdout.strip().splitlines()[-1])


def flagged_tiles(topk: np.ndarray) -> np.ndarray:
    """Key tiles the attention kernel scores per (b, 256-query tile): the 64-key tiles holding an
    allowed key (a valid entry at or before its query) of some query of the tile; at least one."""
    B, T, K = topk.shape
    nqt = (T + 255) // 256
    n = np.zeros((B, nqt), np.int64)
    for b in range(B):
        for qt in range(nqt):
            rows = topk[b, 256 * qt:256 * qt + 256].astype(np.int64)
            s = np.arange(256 * qt, 256 * qt + len(rows))[:, None]
            n[b, qt] = max(1, len(np.unique(rows[(rows >= 0) & (rows < T) & (rows <= s)] // 64)))
    return n


def executed_mfma_flop(tiles: np.ndarray) -> float:
    """MFMA work sparse_attn_kernel executes on its tile schedule: per (b, h) and query tile of 256
    with n scored key tiles (flagged_tiles), each of the 8 waves runs 24 score MFMAs on its first
    tile, then 24 + 16 per tile (the last iteration also scores one tile more, discarded), at
    2 * 32 * 32 * 16 FLOP each."""
    per_b = 8 * (24 + 40 * np.asarray(tiles, np.int64))
    return float(per_b.sum()) * 128 * 2 * 32 * 32 * 16


def causal_tiles(T: int) -> int:
    """Key tiles at or before the last query of each 256-query tile, summed over the tiles."""
    return sum((min(T, 256 * qt + 256) - 1) // 64 + 1 for qt in range((T + 255) // 256))


def window_attention_measurement(torch, mla, dev, stream, q, kv, k_pe, B: int, T: int, K: int,
                                 scale: float) -> dict:
    """The attention call on the benchmarked tensors with a selection that has locality: every
    query selects its K most recent keys (itself included). Key tiles outside each query tile's
    window hold no allowed key and are skipped, so the time follows the selected pairs rather
    than the causal ones. Algorithmic FLOP = 640 x selected pairs x 128 heads."""
    s = torch.arange(T, device=dev, dtype=torch.int32)[:, None]
    win = s - torch.arange(K, device=dev, dtype=torch.int32)[None, :]
    topk = torch.where(win < 0, torch.full_like(win, -1), win).expand(B, T, K).contiguous()
    ws = torch.empty(mla.mla_attn_workspace_bytes(B, T, K), dtype=torch.uint8, device=dev)
    mla.mla_attn_prepare(topk, ws)
    out = torch.empty((B, T, 128, 128), dtype=torch.bfloat16, device=dev)
    us = timed_us(torch, stream, lambda: mla.mla_sparse_prefill_attn_prepared(q, kv, k_pe, ws, scale, out=out),
                  reps=10, warm=3)
    pairs = B * sum(min(K, t + 1) for t in range(T))
    flop = 640.0 * pairs * 128
    tiles = flagged_tiles(topk.cpu().numpy())
    ex = executed_mfma_flop(tiles)
    tf = flop / (us * 1e-6) / 1e12
    del ws, out, topk
    return {"selection": f"window of the {K} most recent keys", "us": us, "TFLOP_s": tf,
            "frac_mfma": tf / PEAK_BF16_TFLOPS, "selected_pairs": pairs,
            "scored_tiles": int(tiles.sum()), "causal_tiles": B * causal_tiles(T),
            "executed_over_algorithmic": ex / flop}


def sample_gfx_clock(torch, fn, reps: int) -> float | None:
    """Median GFX clock (MHz) read through amdsmi while fn() runs `reps` times, or None."""
    try:
        import threading

        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception:   # noqa: BLE001
        return None
    vals, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                c = m.get("current_gfxclks") or m.get("current_gfxclk")
                if isinstance(c, (list, tuple)):
                    c = [x for x in c if isinstance(x, (int, float)) and 0 < x < 10000]
                    c = sum(c) / len(c) if c else None
                if isinstance(c, (int, float)) and 400 < c < 10000:   # below the 500 MHz floor: idle
                    vals.append(float(c))
            except Exception:   # noqa: BLE001
                pass
            time.sleep(0.002)

    th = threading.Thread(target=poll, daemon=True)
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    th.start()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:   # noqa: BLE001
        pass
    return float(np.median(vals)) if vals else None


def timed_us(torch, stream, fn, reps: int = 20, warm: int = 5) -> float:
    """Mean GPU time of fn() in microseconds: events around `reps` back-to-back calls."""
    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def side_measurements(torch, mla, dev, stream, topk, B: int, T: int, K: int) -> dict:
    """Bandwidth-bound kernels against the HBM roofline, outside the timed step: the latent
    norm/rotary at the front-end shape (8 x 4096 rows of 576; 2304 B per row) and the selection
    bitmap at the benchmarked shape (reads B*T*K*4 B, writes B*ceil(T/32)*T*4 B)."""
    torch.manual_seed(1005)
    rows, t_rope = 8 * 4096, 4096
    kv_raw = torch.randn((rows, 576), device=dev).to(torch.bfloat16)
    gain = 1.0 + 0.1 * torch.randn(512, device=dev)
    rope_cs = mla.mla_rope_table(t_rope, dev)
    c_kv = torch.empty((rows, 512), dtype=torch.bfloat16, device=dev)
    k_pe = torch.empty((rows, 64), dtype=torch.bfloat16, device=dev)
    us = timed_us(torch, stream, lambda: mla.mla_kv_norm_rope(kv_raw, gain, 1e-6, rope_cs, t_rope, out=(c_kv, k_pe)))
    nbytes = 2304.0 * rows
    norm = {"rows": rows, "us": us, "GB_s": nbytes / (us * 1e-6) / 1e9,
            "frac_hbm": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, "bytes": nbytes}
    bm = torch.empty((B, (T + 31) // 32, T), dtype=torch.int32, device=dev)
    us_bm = timed_us(torch, stream, lambda: mla.mla_selection_bitmap(topk, out=bm))
    bm_bytes = 4.0 * B * T * K + 4.0 * B * ((T + 31) // 32) * T
    bitmap = {"us": us_bm, "GB_s": bm_bytes / (us_bm * 1e-6) / 1e9,
              "frac_hbm": bm_bytes / (us_bm * 1e-6) / 1e9 / PEAK_HBM_GBS, "bytes": bm_bytes}
    # The same rows with the fp8 round trip and both cache writes (one pass: reads the 1152-byte
    # row, writes the rounded latent, the key and the two cache rows: 3456 B per row).
    kv3 = kv_raw.view(8, 4096, 576)
    kc = torch.empty((8, 4096, 512), dtype=torch.bfloat16, device=dev)
    pc = torch.empty((8, 4096, 64), dtype=torch.bfloat16, device=dev)
    c3, k3 = c_kv.view(8, 4096, 512), k_pe.view(8, 4096, 64)
    us_c = timed_us(torch, stream, lambda: mla.mla_kv_norm_rope_cache(kv3, gain, kc, pc, rope_cs=rope_cs,
                                                                      out=(c3, k3)))
    c_bytes = 3456.0 * rows
    cache = {"rows": rows, "us": us_c, "GB_s": c_bytes / (us_c * 1e-6) / 1e9,
             "frac_hbm": c_bytes / (us_c * 1e-6) / 1e9 / PEAK_HBM_GBS, "bytes": c_bytes}
    # V4.1 window keys/values, decode: 256 sequences, one position each, eps 1e-20, a ring of
    # 128 positions (reads 1024 B, writes 1024 B out + 1024 B ring per row; launch-bound).
    wraw = torch.randn((256, 1, 512), device=dev).to(torch.bfloat16)
    wcache = torch.zeros((256, 128, 512), dtype=torch.bfloat16, device=dev)
    wout = torch.empty((256, 1, 512), dtype=torch.bfloat16, device=dev)
    wcs = mla.mla_rope_table(1001, dev)
    mla.mla_window_kv(wraw, gain, wcache, start_pos=1000, rope_cs=wcs, out=(wout,))   # checks once
    # timed through the C entry point with prepared arguments: the call is shorter than the
    # binding's own argument checks
    L, P = mla.lib(), (lambda t: ctypes.c_void_p(t.data_ptr()))
    wargs = (P(wraw), 256, 1, 1000, P(gain), 1e-20, P(wcs), 0, 128, P(wout), P(wcache), 256, None,
             ctypes.c_void_p(stream.cuda_stream))
    us_w = timed_us(torch, stream, lambda: L.mla_window_kv(*wargs), reps=200, warm=20)
    w_bytes = 3072.0 * 256
    window = {"rows": 256, "us": us_w, "GB_s": w_bytes / (us_w * 1e-6) / 1e9, "bytes": w_bytes}
    # The same decode step at 64 consecutive positions, captured once in a HIP graph (one eager
    # pass on the capture stream first) and replayed: no host launch per step.
    steps = 64
    gcs = mla.mla_rope_table(1000 + steps, dev)
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        for i in range(steps):
            mla.mla_window_kv(wraw, gain, wcache, start_pos=1000 + i, rope_cs=gcs, out=(wout,))
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for i in range(steps):
            mla.mla_window_kv(wraw, gain, wcache, start_pos=1000 + i, rope_cs=gcs, out=(wout,))
    torch.cuda.synchronize()
    us_g = timed_us(torch, stream, graph.replay, reps=20, warm=3) / steps
    window.update({"graph_steps": steps, "graph_us_per_step": us_g,
                   "graph_GB_s": w_bytes / (us_g * 1e-6) / 1e9})
    del graph
    del kv_raw, c_kv, k_pe, bm, kc, pc, wraw, wcache, wout
    # The front-end workload's decode variant: 256 rows of 512, RMSNorm eps 1e-20, no rotary
    # (1024 B read + 1024 B written per row; launch-bound), through the C entry point.
    draw = torch.randn((256, 512), device=dev).to(torch.bfloat16)
    dout = torch.empty((256, 512), dtype=torch.bfloat16, device=dev)
    mla.mla_kv_norm_rope(draw, gain, 1e-20, out=(dout, None))                       # checks once
    dargs = (P(draw), 256, 512, 0, P(gain), 1e-20, None, 1, P(dout), None,
             ctypes.c_void_p(stream.cuda_stream))
    us_d = timed_us(torch, stream, lambda: L.mla_kv_norm_rope(*dargs), reps=200, warm=20)
    decode = {"rows": 256, "us": us_d, "GB_s": 2048.0 * 256 / (us_d * 1e-6) / 1e9, "bytes": 2048.0 * 256}
    side = {"norm_rope_frontend_B8_T4096": norm, "selection_bitmap": bitmap,
            "norm_decode_B256_eps1e-20": decode,
            "norm_rope_fp8_cache_B8_T4096": cache, "window_kv_decode_B256": window}
    side["query_path"] = query_path_measurement(torch, mla, dev, stream, B, T)
    return side


def query_path_measurement(torch, mla, dev, stream, B: int, T: int) -> dict:
    """The query path (wq_a 7168 -> 1536, q_norm, wq_b 1536 -> 128 x 192 with the rotary part of
    every head rotated) at the benchmarked batch and length, against the MFMA roofline:
    2*M*1536*7168 + 2*M*24576*1536 FLOP for M = B*T tokens. Random weights of the layer's shapes."""
    torch.manual_seed(1006)
    M = B * T
    x = torch.randn((B, T, 7168), device=dev).to(torch.bfloat16)
    wa = (torch.randn((1536, 7168), device=dev) * 7168 ** -0.5).to(torch.bfloat16)
    g = 1.0 + 0.1 ** 0.5 * torch.randn(1536, device=dev)
    wb = (torch.randn((128 * 192, 1536), device=dev) * 1536 ** -0.5).to(torch.bfloat16)
    cs = mla.mla_rope_table(T, dev)
    out = mla.mla_q_path(x, wa, g, wb, rope_cs=cs)
    us = timed_us(torch, stream, lambda: mla.mla_q_path(x, wa, g, wb, rope_cs=cs, out=out), reps=10, warm=3)
    flop = 2.0 * M * 1536 * 7168 + 2.0 * M * 24576 * 1536
    tf = flop / (us * 1e-6) / 1e12
    del x, wa, wb, out
    return {"tokens": M, "us": us, "TFLOP_s": tf, "frac_mfma": tf / PEAK_BF16_TFLOPS, "flop": flop}


def attn_counter_record(key: str):
    """A figure of the attention kernel's rocprofv3 counter record (profiles/sparse_attn_traffic.txt),
    if the record matches the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "sparse_attn_traffic.txt")
    src = os.path.join(ROOT, "sparse_latent_attention_wkv_amd", "csrc", "attn.hip")
    if not os.path.exists(path) or not os.path.exists(src):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if kv.get("source_sha") != sha or key not in kv:
        return None
    return float(kv[key])


def mfma_busy_record():
    """MFMA-busy fraction of the attention kernel from a rocprofv3 counter run, or None."""
    return attn_counter_record("mfma_busy_frac")


# An engine clock read while the attention runs is taken only inside this range (MHz): the
# kernel keeps the matrix units about half busy, and its counters put the clock near 1.9 GHz.
CLOCK_PLAUSIBLE_MHZ = (1000.0, 2600.0)


def attention_clock(sampled):
    """(clock MHz, source): the sampled engine clock if plausible, else the clock from the counter
    record (GRBM_GUI_ACTIVE per XCD over the kernel's duration), else (None, None)."""
    if sampled is not None and CLOCK_PLAUSIBLE_MHZ[0] <= sampled <= CLOCK_PLAUSIBLE_MHZ[1]:
        return sampled, "amdsmi current_gfxclk, median while the attention runs"
    rec = attn_counter_record("gfx_clock_mhz")
    if rec is not None:
        why = "no amdsmi reading" if sampled is None else f"amdsmi read {sampled:.0f} MHz, outside {CLOCK_PLAUSIBLE_MHZ}"
        return rec, f"rocprofv3 counters (profiles/sparse_attn_traffic.txt); {why}"
    return None, None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="headline", choices=["headline", "1k", "long", "tiny"])
    ap.add_argument("--path", default="head-major", choices=["head-major", "latent", "auto"],
                    help="head-major: mla_kv_up + mla_sparse_prefill_attn; latent: "
                         "mla_sparse_prefill_attn_latent (no per-head keys and values); auto: "
                         "mla_sparse_prefill_attn_auto (head-major below the split row, latent above)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="time the CPU oracle only and print its JSON record (used as a child process)")
    ap.add_argument("--no-clock-sample", action="store_true",
                    help="skip the engine-clock sampling (profiler runs)")
    ap.add_argument("--side-only", action="store_true",
                    help="run only the measurements outside the step (bandwidth-bound kernels, query path) "
                         "and print them; a profiler run of this mode sees each of those kernels alone")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run a plain 256 MiB fill and copy so a counter "
                         "run can scale FETCH_SIZE / WRITE_SIZE against known byte counts")
    args = ap.parse_args()

    if args.cpu_baseline_only:
        print(json.dumps(cpu_baseline_child(args.workload)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU runs are not supported by this build", file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))

    import torch
    import synth
    import sparse_latent_attention_wkv_amd as mla

    w = synth.WORKLOADS[args.workload]
    B, T, K = w.B, w.T, w.K
    t_gen = time.perf_counter()
    d = synth.make(w)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    x, w_dkv, w_ukv, q = up(d["x"]), up(d["w_dkv"]), up(d["w_ukv"]), up(d["q"])
    gain = torch.from_numpy(d["gain"]).to(dev)
    topk = torch.from_numpy(d["topk"]).to(dev)
    rope_cs = mla.mla_rope_table(T, dev)           # the model's freqs_cis: built once
    kv_raw = torch.empty((B, T, 576), dtype=torch.bfloat16, device=dev)
    c_kv = torch.empty((B, T, 512), dtype=torch.bfloat16, device=dev)
    k_pe = torch.empty((B, T, 64), dtype=torch.bfloat16, device=dev)
    latent = args.path == "latent"
    auto = args.path == "auto"
    kv = None if (latent or auto) else torch.empty((B, 128, T, 256), dtype=torch.bfloat16, device=dev)
    out = torch.empty((B, T, 128, 128), dtype=torch.bfloat16, device=dev)
    ws_bytes = (mla.mla_attn_latent_workspace_bytes(B, T, K) if latent else
                int(mla.lib().mla_attn_auto_workspace_bytes(B, T, K)) if auto else
                mla.mla_attn_workspace_bytes(B, T, K))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    scale = mla.mla_default_softmax_scale()
    stream = torch.cuda.current_stream(dev)
    # Head-major path: the selection bitmap depends only on the top-k indices, so it is built on a
    # second stream (default priority) from the step's start, on the compute units the
    # down-projection (192 workgroups) leaves free and beside the up-projection (measured in one
    # process: 1.898 ms per step against 1.904 ms when it starts after the down-projection; both
    # faster than sequential). The second stream first waits for the main stream, so the previous
    # step's attention, which reads the same workspace, has finished.
    side = torch.cuda.Stream(dev)
    sync_start, sync_ready = torch.cuda.Event(), torch.cuda.Event()

    def step(ev=None, split=False):
        # ev: timing events at the step's start, before the attention and at the step's end;
        # split: one more between the down- and up-projections (kept out of the timed steps)
        if ev is not None:
            ev[0].record(stream)
        if kv is not None:
            sync_start.record(stream)
            side.wait_event(sync_start)
            mla.mla_attn_prepare(topk, ws, stream=side)
            sync_ready.record(side)
        mla.mla_kv_latent(x, w_dkv, gain, 1e-6, rope_cs, out=(kv_raw, c_kv, k_pe))
        if split:
            ev[1].record(stream)
        if kv is not None:
            mla.mla_kv_up(c_kv, w_ukv, out=kv)
        if ev is not None:
            ev[2].record(stream)
        if latent:
            mla.mla_sparse_prefill_attn_latent(q, c_kv, k_pe, w_ukv, topk, scale, workspace=ws, out=out)
        elif auto:
            mla.mla_sparse_prefill_attn_auto(q, c_kv, k_pe, w_ukv, topk, scale, workspace=ws, out=out)
        else:
            stream.wait_event(sync_ready)
            mla.mla_sparse_prefill_attn_prepared(q, kv, k_pe, ws, scale, out=out)
        if ev is not None:
            ev[3].record(stream)

    if args.side_only:
        print(json.dumps({"bandwidth_kernels": side_measurements(torch, mla, dev, stream, topk, B, T, K)}),
              flush=True)
        return
    # The measurements outside the step run first: on a GPU that was idle, the first milliseconds
    # of load run at a lower engine clock (the attention's first launches take up to 30% longer),
    # and the timed steps are meant to show the steady state.
    side_meas = side_measurements(torch, mla, dev, stream, topk, B, T, K)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    att = np.mean([e[2].elapsed_time(e[3]) for e in evs])
    gpu_step = np.mean([e[0].elapsed_time(e[3]) for e in evs])
    ms_per_step = wall * 1e3 / args.steps
    # the split of the first part of the step into its two calls, from a few more (untimed) steps
    evs_split = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(min(args.steps, 10))]
    for e in evs_split:
        step(e, split=True)
    torch.cuda.synchronize()
    lat = np.mean([e[0].elapsed_time(e[1]) for e in evs_split])
    upm = np.mean([e[1].elapsed_time(e[2]) for e in evs_split])

    clock_mhz, clock_src = None, None
    if kv is not None:
        sampled = None
        if not args.no_clock_sample:
            stream.wait_event(sync_ready)
            sampled = sample_gfx_clock(torch, lambda: mla.mla_sparse_prefill_attn_prepared(q, kv, k_pe, ws, scale,
                                                                                           out=out), 400)
        if args.workload == "headline" and args.path == "head-major":
            clock_mhz, clock_src = attention_clock(sampled)
        elif sampled is not None and CLOCK_PLAUSIBLE_MHZ[0] <= sampled <= CLOCK_PLAUSIBLE_MHZ[1]:
            clock_mhz, clock_src = sampled, "amdsmi current_gfxclk, median while the attention runs"

    window = None
    if kv is not None:
        stream.wait_event(sync_ready)
        window = window_attention_measurement(torch, mla, dev, stream, q, kv, k_pe, B, T, K, scale)

    if args.copy_calibration:
        src = torch.ones(1 << 26, dtype=torch.int32, device=dev)      # writes 256 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)                                                 # reads + writes 256 MiB
        torch.cuda.synchronize()
        del src, dst

    pairs = selected_pairs(d["topk"])
    attn_flop = 640.0 * pairs * 128
    tiles = flagged_tiles(d["topk"]) if kv is not None else None
    exec_flop = executed_mfma_flop(tiles) if kv is not None else None
    causal_pairs = B * T * (T + 1) // 2
    achieved = attn_flop / (att * 1e-3) / 1e12
    flop_down = 2.0 * B * T * 7168 * 576
    flop_up = 2.0 * B * T * 512 * 32768
    tokens = B * T
    # the counter records were taken on the headline workload (head-major path) only
    headline = args.workload == "headline" and args.path == "head-major"
    traffic = traffic_record("sparse_attn") if headline else None

    res = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"sparse MLA prefill {args.workload}: B={B}, T={T}, top-k {K}, "
                               "128 heads, qk 192 / v 128, hidden 7168, latent 512+64"
                               + (", latent-space attention" if latent else "")
                               + (f", split form (latent from row {mla.mla_attn_auto_split(T, K)})" if auto else ""),
                   "B": B, "T": T, "top_k": K, "heads": 128, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "kernel": ("mla_sparse_prefill_attn_latent call (lists, absorbed-query GEMM, "
                                "latent attention, value GEMM)" if latent else
                                "mla_sparse_prefill_attn_auto call (head-major below the split, "
                                "latent form above)" if auto else
                                "sparse_attn kernel (mla_sparse_prefill_attn_prepared; the selection "
                                "bitmap is built by mla_attn_prepare on a second stream during the "
                                "projections)"),
                     "algorithmic_flop_per_launch": attn_flop,
                     "executed_mfma_flop_per_launch": exec_flop,
                     "executed_over_algorithmic": None if exec_flop is None else exec_flop / attn_flop,
                     "scored_tiles": None if tiles is None else int(tiles.sum()),
                     "causal_tiles": B * causal_tiles(T),
                     "measured_gfx_clock_mhz": clock_mhz,
                     "clock_source": clock_src,
                     "peak_at_measured_clock": None if clock_mhz is None else PEAK_BF16_TFLOPS * clock_mhz / 2400.0,
                     "frac_at_measured_clock": (None if clock_mhz is None else
                                                achieved / (PEAK_BF16_TFLOPS * clock_mhz / 2400.0))},
        "stages_ms": {"kv_latent": lat, "kv_up": upm, "sparse_attn": att, "gpu_step": gpu_step},
        "stage_tflops": {"kv_latent": flop_down / (lat * 1e-3) / 1e12,
                         "kv_up": None if kv is None else flop_up / (upm * 1e-3) / 1e12},
        "attention_only_tokens_per_s": tokens / (att * 1e-3),
        "attention_mfma_busy_frac": mfma_busy_record() if headline else None,
        "bandwidth_kernels": side_meas,
        "attention_window_selection": window,
        "selected_pairs_all_batches": pairs,
        "latent_mfma_flop_per_launch": (2176.0 * pairs * 128 + 2 * 2.0 * tokens * 128 * 128 * 512) if latent else None,
        "causal_over_selected": causal_pairs / pairs,
        "input_generation_s": round(t_gen, 2),
    }
    if rank == 0 and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.workload)
    if rank == 0:
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
