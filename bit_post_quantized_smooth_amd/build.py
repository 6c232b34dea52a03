"""Build libsvdq.so in-tree: hipcc for the gfx950 kernels, g++ for the host side.

Usage: ``python -m bit_post_quantized_smooth_amd.build`` (or ``build()``).
The library lands next to this file; intermediates go to ``_build/``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsvdq.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_SOURCES = ["k1_quant_down.hip", "k2_w4a4_gemm.hip", "k2_mx_gemm.hip", "k2_w4a16_gemm.hip",
               "k2_w4a4_tiled.hip", "gelu.hip", "lowrank_pack.hip", "clock_probe.hip",
               "abi_device.hip",
               "abi_noalloc.hip"]
HOST_SOURCES = {
    # the quantizer's fp32 divide/multiply must round exactly: no contraction
    "host_prep.cpp": ["-ffp-contract=off"],
    # the eigen-solver only needs fp64 accuracy; let it use FMA and AVX2
    "host_eigen.cpp": ["-mavx2", "-mfma", "-ffp-contract=fast"],
}

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no implicit contraction anywhere: the method fixes its rounding points
    # (e.g. Xhat = fp32(x * inv), then fp16(Xhat)), and contraction would fuse
    # that product and its fp16 conversion into one v_fma_mixlo_f16 (a single
    # rounding). Every FMA the kernels want is written as __builtin_fmaf.
    "-ffp-contract=off",
    # no packed fp32 (v_pk_fma_f32 and friends) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results straight into VGPRs: the rescale reads every element
    # with VALU ops, and an AGPR destination would add a v_accvgpr_read each
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
]
GXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fopenmp", "-D__HIP_PLATFORM_AMD__",
             f"-I{ROCM}/include"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False) -> str:
    """Compile every source and link libsvdq.so. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src, extra in HOST_SOURCES.items():
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append(["g++", *GXX_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-fopenmp",
          f"-L{ROCM}/lib", "-lamdhip64", "-lgomp"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
