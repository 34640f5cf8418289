"""Build libawq355.so in-tree with hipcc for gfx950.

Usage: python -m bit_weight_only_quantize_amd.build [--verbose]

Every HIP translation unit is compiled with:
  * --offload-arch=gfx950, -O3, -std=c++17, -fPIC;
  * -ffp-contract=off: multiply-adds are fused only where the source asks for
    an fma, so the quantizer's arithmetic is exactly the written IEEE sequence;
  * the packed-fp32 target feature disabled (packed fp32 VALU forms are not
    used by this library).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB_NAME = "libawq355.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = [
    "quantize_pack.hip",
    "linear_gemv.hip",
    "linear_batched.hip",
    "linear_gemm.hip",
    "gemm_f16.hip",
    "search.hip",
    "api.cpp",
]

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-I", CSRC,
        "-Wall",
        "-Wno-unused-function",
    ]


def compile_one(src: str, obj: str, verbose: bool) -> None:
    cmd = [hipcc(), *common_flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).strip()
    # hipcc's host pass does not know the device-only feature flag; that
    # warning is expected and harmless.
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if lines and verbose:
        print("\n".join(lines))


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel, one hipcc per translation unit) and
    link LIB_PATH (always rebuilds)."""
    from concurrent.futures import ThreadPoolExecutor

    with tempfile.TemporaryDirectory(prefix="awq355_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(src)[0] + ".o") for src in SOURCES]
        jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            for fut in [pool.submit(compile_one, src, obj, verbose)
                        for src, obj in zip(SOURCES, objs)]:
                fut.result()
        tmp_lib = os.path.join(tmp, LIB_NAME)
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
        shutil.copy2(tmp_lib, LIB_PATH + ".tmp")
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
