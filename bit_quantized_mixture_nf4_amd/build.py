"""Build the HIP library ``libe4b.so`` in-tree for gfx950.

Usage: ``python -m bit_quantized_mixture_nf4_amd.build`` (or ``build()``).
Every source is compiled by hipcc (``--offload-arch=gfx950``) into an object
under ``_build/`` and linked into ``bit_quantized_mixture_nf4_amd/libe4b.so``.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libe4b.so")

SOURCES = ["plan.cpp", "quant.hip", "route.hip", "gemm_wide.hip", "combine.hip", "decode.hip", "lora.hip", "mx.hip",
           "api.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 VALU forms are disabled in device code; fp32 denormals are kept.
COMMON = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-I", INCLUDE,
    "-Wno-unused-result",
]


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(
        ln for ln in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in ln
    )
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    return obj, errs


def build(verbose=False):
    """Compile every source and link ``libe4b.so`` (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    if verbose:
        for (obj, errs), src in zip(results, SOURCES):
            if errs.strip():
                print(f"[{src}]\n{errs}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "--offload-arch=gfx950", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
