"""Build step: compiles the HIP kernels and the host library into librpa.so (gfx950).

Run ``python -m ragged_paged_attention_forward_amd.build`` (or call ``build()``).
hipcc cross-compiles for gfx950, so this works on machines without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "librpa.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

# Kernel translation units, one per head size (each may take its own
# register-allocation options).  MFMA accumulators live in the architectural
# VGPRs, where the softmax and rescaling code uses them without copies.
KERNEL_SOURCES = {
    "rpa_kernels_d64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "rpa_kernels_d128.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "rpa_kernels_d256.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "rpa_kernels_d512.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "rpa_probe.hip": [],
    "rpa_e4m3.hip": [],
    "rpa_noalloc.hip": [],
}
HOST_SOURCES = ["rpa_dispatch.cpp", "rpa_api.cpp", "rpa_plan.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU forms stay off: the compiler would otherwise emit them
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
        # the five leading kernel arguments (work items, page table, Q, K, V:
        # ten scalar registers) arrive preloaded in scalar registers
        "-mllvm", "-amdgpu-kernarg-preload-count=5",
    ]


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source (in parallel) and link librpa.so in the package directory."""
    from concurrent.futures import ThreadPoolExecutor
    cc = hipcc()
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    jobs = []
    for src, flags in KERNEL_SOURCES.items():
        obj = os.path.join(out_dir, src + ".o")
        jobs.append(([cc] + compile_flags() + flags + list(extra_flags) +
                     ["-c", os.path.join(CSRC, src), "-o", obj], obj))
    for src in HOST_SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        jobs.append(([cc, "-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC,
                      "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, src), "-o", obj], obj))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    objs = [o for _, o in jobs]
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    text = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{text}")
    if verbose and text.strip():
        print(text)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
