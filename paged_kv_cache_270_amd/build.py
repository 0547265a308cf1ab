"""Build libpkv.so (gfx950) in-tree with hipcc.

    python -m paged_kv_cache_270_amd.build

Compiles csrc/pkv_host.cpp and the kernels in csrc/*.hip into
paged_kv_cache_270_amd/libpkv.so.  Device code is built for gfx950 only, at -O3,
with packed fp32 instructions disabled (-packed-fp32-ops) and the default
correctly rounded fp32 division (no fast-math).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -amdgpu-mfma-vgpr-form: MFMA accumulators stay in ordinary VGPRs, so the
# softmax rescale works on them in place instead of copying through AGPRs.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-I", INCLUDE]


def build(verbose: bool = False) -> str:
    objs = []
    for src, dev in (("pkv_host.cpp", False), ("pkv_kernels.hip", True),
                     ("pkv_write.hip", True), ("pkv_prefill.hip", True),
                     ("pkv_swap.hip", True), ("pkv_probe.hip", True),
                     ("pkv_noalloc.hip", True)):
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + COMMON + (DEVICE_FLAGS + ["-x", "hip"] if dev else []) + \
              ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950"] + objs + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
