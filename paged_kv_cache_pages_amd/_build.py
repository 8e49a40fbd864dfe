"""Build libpagedkv.so in-tree for gfx950 with hipcc (host validator with g++).

Usage: ``python -m paged_kv_cache_pages_amd._build`` (also called by ``__graft_entry__.build``).
The library lands in ``paged_kv_cache_pages_amd/lib/libpagedkv.so``; objects in ``_build/``.
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
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libpagedkv.so")
# A plain C++ client of the C ABI (no Python, no PyTorch): test code, built beside its source for
# a GPU test, never part of the library.
CLIENT_SRC = os.path.join(ROOT, "tests", "host", "abi_client.cpp")
CLIENT_PATH = os.path.join(ROOT, "tests", "host", "pkv_abi_client")
# A stand-alone read-bandwidth probe for the decode kernels' access pattern (measurement only).
CEILING_SRC = os.path.join(ROOT, "tests", "host", "read_ceiling.hip")
CEILING_PATH = os.path.join(ROOT, "tests", "host", "pkv_read_ceiling")
ISSUE_SRC = os.path.join(ROOT, "tests", "host", "issue_rate.hip")
ISSUE_PATH = os.path.join(ROOT, "tests", "host", "pkv_issue_rate")
CU_READ_SRC = os.path.join(ROOT, "tests", "host", "cu_read_rate.hip")
CU_READ_PATH = os.path.join(ROOT, "tests", "host", "pkv_cu_read_rate")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_SOURCES = ["pagedkv_api.hip", "kv_append.hip", "paged_attention.hip", "rope_append.hip", "prefill.hip"]
CXX_SOURCES = ["validate.cpp", "page_allocator.cpp"]

# Per-file additions: keep MFMA accumulators in ordinary VGPRs, so the softmax rescale of the
# output tile does not copy it between register files every step.
FILE_FLAGS = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "paged_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form",
                                      # the decode kernels' 14 leading argument dwords go to SGPRs
                                      "-mllvm", "-amdgpu-kernarg-preload-count=14"]}

ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed FP32 instructions stay off: the compiler must not form v_pk_{add,mul,fma}_f32
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every source (always, even when a library exists) and link the shared library."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    hipcc = _hipcc()
    extra = list(extra_flags or [])
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OBJ_DIR, src + ".o")
        jobs.append([hipcc, *HIP_FLAGS, *FILE_FLAGS.get(src, []), *extra, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(OBJ_DIR, src + ".o")
        jobs.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [j[-1] for j in jobs]
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    if os.path.exists(CLIENT_SRC):  # a source tree shipped without tests/ has no client
        client_tmp = CLIENT_PATH + ".tmp"
        _run(["g++", "-O2", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
              "-I", INCLUDE, CLIENT_SRC, "-o", client_tmp, "-L", LIB_DIR, "-lpagedkv", "-L", os.path.join(ROCM, "lib"),
              "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../paged_kv_cache_pages_amd/lib",
              "-Wl,-rpath," + os.path.join(ROCM, "lib")], verbose)
        os.replace(client_tmp, CLIENT_PATH)
    if os.path.exists(CEILING_SRC):
        ceiling_tmp = CEILING_PATH + ".tmp"
        _run([hipcc, *HIP_FLAGS, CEILING_SRC, "-o", ceiling_tmp], verbose)
        os.replace(ceiling_tmp, CEILING_PATH)
    if os.path.exists(ISSUE_SRC):
        issue_tmp = ISSUE_PATH + ".tmp"
        _run([hipcc, *HIP_FLAGS, ISSUE_SRC, "-o", issue_tmp], verbose)
        os.replace(issue_tmp, ISSUE_PATH)
    if os.path.exists(CU_READ_SRC):
        cu_tmp = CU_READ_PATH + ".tmp"
        _run([hipcc, *HIP_FLAGS, CU_READ_SRC, "-o", cu_tmp], verbose)
        os.replace(cu_tmp, CU_READ_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
