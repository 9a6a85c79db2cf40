"""The C ABI's host code under AddressSanitizer (no GPU): the argument checks, workspace-size
arithmetic and alias checks of csrc/mla_api.hip, built with host-side ASan instrumentation
(sparse_latent_attention_wkv_amd.build_asan), run every case of test_abi_cpu.py in a child
process that preloads clang's ASan runtime. Any invalid host memory access in those paths ends
the child with an AddressSanitizer report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

build_asan = pytest.importorskip("sparse_latent_attention_wkv_amd.build_asan")


def test_abi_checks_run_clean_under_host_asan():
    rt = build_asan.asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    lib = build_asan.build()
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms, "the library is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", MLA_LIBRARY=lib)
    probe = subprocess.run([sys.executable, "-c", "import sparse_latent_attention_wkv_amd as m; print(m.LIB_PATH)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.strip() == lib
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
