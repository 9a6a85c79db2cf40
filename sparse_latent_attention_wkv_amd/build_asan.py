"""Build a copy of libmla.so whose host code for the C ABI (the argument checks, workspace sizes
and launch sequencing in csrc/mla_api.hip) is instrumented with AddressSanitizer.

Usage: python -m sparse_latent_attention_wkv_amd.build_asan  ->  _build_asan/libmla_asan.so
The device code is the ordinary gfx950 build; only the host side of mla_api.hip is instrumented,
the other objects come from the ordinary build. The library leaves the sanitizer's runtime
symbols unresolved: load it into a process that preloads clang's shared ASan runtime
(asan_runtime() gives its path), with MLA_LIBRARY pointing at it so the binding loads it.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from . import build as _b

BUILD = os.path.join(_b.PKG, "_build_asan")
LIB = os.path.join(BUILD, "libmla_asan.so")
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str | None:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    plain = os.path.join(_b.BUILD, "")
    if not os.path.exists(_b.LIB):
        _b.build()
    api = os.path.join(_b.CSRC, "mla_api.hip")
    obj = os.path.join(BUILD, "mla_api.hip.o")
    cmd = [_b.HIPCC, *_b.CFLAGS, *HOST_ASAN, "-c", api, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {api}:\n{r.stdout}\n{r.stderr}")
    others = sorted(o for o in glob.glob(plain + "*.hip.o") if not o.endswith("mla_api.hip.o"))
    tmp = LIB + ".tmp"
    r = subprocess.run([_b.HIPCC, f"--offload-arch={_b.ARCH}", "-shared", "-fPIC", obj, *others, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
