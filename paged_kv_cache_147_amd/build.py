"""Build libpagedkv.so (host pool + gfx950 kernels) in-tree with hipcc.

Run as ``python paged_kv_cache_147_amd/build.py`` (no package import, so a stale
library is never loaded first) or through
``__graft_entry__.build()``.  Objects go to ``_build/`` at the repository
root; the shared library lands next to this file, where the binding loads it.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
# Memory-read ceilings for the benchmark: a separate library, not part of the decode path.
CEILING_LIB = os.path.join(PKG, "libpagedkv_ceiling.so")
CEILING_SOURCES = ["ceiling.hip"]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
# Device code: gfx950 only; packed float32 ops stay off (ordinary float code
# is compiled to unpacked VALU instructions).
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = ["status.cpp", "pool.cpp", "cache_ops.hip", "decode.hip", "decode_fp8.hip", "prefill.hip"]
# Per-source extras.  prefill: matrix-core accumulators in ordinary VGPRs, so
# the softmax can rescale them in place (in AGPRs every step would copy them
# out and back).
EXTRA = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"], "decode_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return exe


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, src + ".o")
    cmd = [hipcc(), *COMMON]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *HIP_FLAGS, *EXTRA.get(src, [])]
    cmd += ["-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag; drop that note
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return obj, err


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose=True, jobs=None):
    os.makedirs(OBJDIR, exist_ok=True)
    sources = SOURCES + CEILING_SOURCES
    jobs = jobs or min(len(sources), os.cpu_count() or 4)
    with ThreadPoolExecutor(jobs) as ex:
        results = dict(zip(sources, ex.map(_compile, sources)))
    for _, err in results.values():
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    _link([results[s][0] for s in SOURCES], LIB)
    _link([results[s][0] for s in CEILING_SOURCES], CEILING_LIB)
    if verbose:
        print(f"built {LIB} and {CEILING_LIB}")
    return LIB


if __name__ == "__main__":
    build()
