"""Build the HIP library libsharq.so (gfx950) in-tree with hipcc, and the
measurement library libsharq_yardstick.so that bench.py's MFMA yardstick
loads (not part of the sharq ABI).

Each source compiles to its own object (in parallel, with its own extra
flags), then one hipcc link per library."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsharq.so")
YARDSTICK_LIB = os.path.join(HERE, "libsharq_yardstick.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # bit-exact quantization: no contraction into FMA, IEEE fp32 division and
    # square root, fp32 denormals kept
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]

# source -> extra flags.  The NVFP4 GEMM and the MXFP4 GEMM on the FP8 sparse
# MFMA keep their MFMA accumulators in VGPRs: the 2:4 MFMA (v_smfmac)
# accumulates in VGPRs only, so accumulators in AGPRs were copied between the
# two register files around every sparse MFMA, and the NVFP4 dense kernels fit
# two wavefronts per SIMD only without AGPRs.
SOURCES = {
    "sharq_abi.cpp": [],
    "prep.hip": [],
    "gemm_mx.hip": [],
    "gemm_nv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    # the MXFP4 backbone on the 2:4 FP8 MFMA (v_smfmac, VGPR accumulators)
    "gemm_mx_fp8sp.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}
YARDSTICK_SOURCES = {"yardstick.hip": []}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for srcs in (SOURCES, YARDSTICK_SOURCES):
        for src, extra in srcs.items():
            obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
            jobs.append(([HIPCC, *FLAGS, *extra, "-c", "-o", obj, os.path.join(CSRC, src)], obj))
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        for f in [ex.submit(_run, cmd, verbose) for cmd, _ in jobs]:
            f.result()
    for lib, srcs in ((LIB, SOURCES), (YARDSTICK_LIB, YARDSTICK_SOURCES)):
        objs = [os.path.join(OBJ, os.path.splitext(src)[0] + ".o") for src in srcs]
        tmp = lib + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-o", tmp, *objs], verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
