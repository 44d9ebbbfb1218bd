"""Build libbi.so (the HIP library behind include/bi.h) in-tree with hipcc for gfx950,
and libbi_testing.so: the same kernels with the C ABI compiled with -DBI_TESTING,
which adds the tile-forcing values of `tc` that the tile-identity tests and the
tile benchmark use (the production library rejects them).

Compiled fresh on every call.  Flags:
  -ffp-contract=off   the only fused multiply-adds are the explicit fmaf calls
                      of the scalar tier; no other expression is contracted
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed f32 VALU instructions are generated
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libbi.so")
LIB_TESTING = os.path.join(HERE, "libbi_testing.so")
SOURCES = ["bi_api.cpp", "scalar_tier.hip", "mfma_tier.hip", "mfma_fwd.hip", "mfma_dx.hip",
           "mfma_dw.hip", "mfma_grouped.hip", "fp8_tier.hip", "fp8_dl.hip",
           "quant.hip", "bias_grad.hip", "mfma_bwd.hip", "mfma_gbwd.hip", "static_scratch.hip"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str, objdir: str, testing: bool = False) -> str:
    stem = os.path.splitext(src)[0] + ("_testing" if testing else "")
    obj = os.path.join(objdir, stem + ".o")
    lang = ["-x", "hip"]
    defs = ["-DBI_TESTING"] if testing else []
    cmd = [_hipcc()] + lang + COMMON + defs + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + [("bi_api.cpp", True)]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], objdir, j[1]), jobs))
    kernels = objs[1:len(SOURCES)]
    _link([objs[0]] + kernels, LIB)
    _link([objs[-1]] + kernels, LIB_TESTING)
    if verbose:
        print("built", LIB, "and", LIB_TESTING)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
