"""Build libhk.so and libhk_probe.so (HIP for gfx950) in-tree with hipcc.

    python hash_top_kv_amd/build.py        # or __graft_entry__.build()

Each translation unit compiles to hash_top_kv_amd/_build/*.o in parallel.  libhk.so (the
decode path, include/hk.h) and libhk_probe.so (the measurement aids of
include/hk_probe.h) are linked next to this file.  Packed-fp32 instructions are disabled
for all device code.
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
LIB = os.path.join(HERE, "libhk.so")
PROBE_LIB = os.path.join(HERE, "libhk_probe.so")
LIB_SOURCES = ["api.hip", "retrieve.hip", "attend.hip", "fused.hip", "encode.hip", "evict.hip",
               "exact.hip", "tiny.hip"]
PROBE_SOURCES = ["probe.hip"]
SOURCES = LIB_SOURCES + PROBE_SOURCES
ARCH = "gfx950"
# The attention kernels keep their matrix-core accumulators in ordinary VGPRs: the
# online-softmax rescale multiplies them in place, which with accumulation registers
# costs a copy out and back per tile and a larger register footprint.
EXTRA_FLAGS = {"attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "fused.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "tiny.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "encode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


# Kernel arguments preloaded into SGPRs at launch (up to 16 dwords), so a kernel's first
# memory requests need no scalar load of its arguments first.
def common_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-kernarg-preload-count=16",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Wall", "-Wno-unused-function", "-Wno-unused-result"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noisy = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noisy:
        sys.stderr.write("\n".join(noisy) + "\n")
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for {os.path.basename(out)}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    # the largest translation units first, so the parallel build ends sooner
    order = sorted(SOURCES, key=lambda f: -os.path.getsize(os.path.join(CSRC, f)))
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = dict(zip(order, ex.map(_compile, order)))
    _link([objs[f] for f in LIB_SOURCES], LIB)
    _link([objs[f] for f in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
