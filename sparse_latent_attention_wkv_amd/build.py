"""Build libmla.so in-tree from csrc/*.hip with hipcc for gfx950.

Usage: python -m sparse_latent_attention_wkv_amd.build   (or __graft_entry__.build()).
Each source compiles to an object under _build/ in parallel; the objects link into
sparse_latent_attention_wkv_amd/libmla.so.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every warning is an error, except the one clang gives for naming m0 in the clobber list of
    # the global->LDS load helpers (mla_device.hpp): m0 is a reserved register, and the generated
    # code of every kernel writes and reads m0 only inside those helpers, so no value of the
    # compiler's own lives in m0 across them
    "-Wall", "-Wextra", "-Werror", "-Wno-inline-asm", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


# Extra flags per source file.
#  attn.hip, latent.hip: -fno-honor-nans lets fmaxf map to plain v_max (no NaN canonicalisation
#  of MFMA results; the kernels never produce NaN from finite inputs).
FILE_FLAGS = {
    "attn.hip": ["-fno-honor-nans"],
    "latent.hip": ["-fno-honor-nans"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    with ThreadPoolExecutor(max(1, min(8, len(srcs), os.cpu_count() or 1))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
