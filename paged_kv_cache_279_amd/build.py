"""Build libpkv.so in-tree with hipcc for gfx950.

``python -m paged_kv_cache_279_amd.build`` (or ``build()``) compiles the HIP
kernels and the host allocator into ``paged_kv_cache_279_amd/libpkv.so``.
It always recompiles.
"""

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
INCLUDE_DIR = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libpkv.so")
SOURCES = [os.path.join(CSRC, "pkv_device.hip"), os.path.join(CSRC, "pkv_host.cpp")]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # never let the compiler form packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the softmax rescales them with VALU ops
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc_path():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose=False, extra_flags=()):
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc_path()] + HIP_FLAGS + list(extra_flags) + ["-I", INCLUDE_DIR, "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    lines = [ln for ln in res.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, "\n".join(lines)))
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, extra_flags=[a for a in sys.argv[1:] if a != "-v"])
    print(LIB_PATH)
