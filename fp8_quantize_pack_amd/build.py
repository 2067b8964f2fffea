"""Build libmxq.so (HIP, gfx950) in-tree with hipcc.

Every HIP source is compiled to an object in parallel, then linked into
``fp8_quantize_pack_amd/libmxq.so``; the streaming reference kernels that
measure the practical HBM ceiling go into ``libmxq_roofline.so``.  Flags that matter for bit-exactness:
no fast-math, no contraction of a*b+c into fma (the kernels call fmaf
explicitly where they want one), correctly rounded float32 division, and
denormals kept.  Packed-FP32 instructions are disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmxq.so")
ROOFLINE_LIB = os.path.join(HERE, "libmxq_roofline.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["mxq_api.cpp", "k_mxfp4.hip", "k_nvfp4.hip", "k_cache.hip",
           "mxq_api_gemm.cpp", "k_grouped_mm.hip",
           "mxq_api_ext.cpp", "k_mxfp8.hip", "k_fp4_static.hip", "k_kv.hip",
           "mxq_api_noalloc.hip"]
ROOFLINE_SOURCES = ["k_roofline_ref.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _obj(src: str, out_dir: str) -> str:
    return os.path.join(out_dir, os.path.splitext(src)[0] + ".o")


def build(verbose: bool = False, out: str = LIB, extra_flags=()) -> str:
    """Compile every source for gfx950 and link the shared library."""
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    procs = []
    for src in SOURCES + ROOFLINE_SOURCES:
        path = os.path.join(CSRC, src)
        lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [HIPCC, *lang, f"--offload-arch={ARCH}", *COMMON, *extra_flags,
               "-c", path, "-o", _obj(src, out_dir)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        log, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, log))
        elif verbose and log.strip():
            print(log)
    if failed:
        msg = "\n".join(f"--- {s}\n{l}" for s, l in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    for target, srcs in ((out, SOURCES), (ROOFLINE_LIB, ROOFLINE_SOURCES)):
        tmp = target + ".tmp"
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
                *[_obj(s, out_dir) for s in srcs]]
        subprocess.run(link, check=True)
        os.replace(tmp, target)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
