"""Build librs.so in-tree: HIP kernels for gfx950 plus the C++ host library.

    python -m vit_token_pruning_amd.build

Device sources are compiled by hipcc for gfx950 only; the host library (validation,
schedule, launch sequence) by g++ with -ffp-contract=off so that the kept-count rule
floor(r*L + 1/2) rounds exactly like IEEE double arithmetic everywhere else.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librs.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

DEVICE_SOURCES = ["rs_gemm.hip", "rs_mlp.hip", "rs_lin.hip", "rs_attn.hip", "rs_attn_map.hip", "rs_rowops.hip", "rs_noalloc.hip", "rs_probe.hip"]
HOST_SOURCES = ["rs_api.cpp"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]
# Per-source additions.  Attention: matrix-core results in ordinary VGPRs -- the kernel
# works on its score and output accumulators with VALU ops every key tile, and
# accumulator-register results cost a copy each way (112 moves per tile).  The GEMMs keep
# the default (measured slower with it).
SOURCE_FLAGS = {"rs_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                "rs_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                "rs_attn_map.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
HOST_FLAGS = [
    "-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall",
    "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
    "-I" + os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link librs.so; returns its path.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    jobs = []
    objs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([hipcc] + HIP_FLAGS + SOURCE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["g++"] + HOST_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs +
         ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
