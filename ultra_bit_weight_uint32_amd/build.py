"""Build libubw.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m ultra_bit_weight_uint32_amd.build [-v]
"""
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libubw.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("kernels.hip", "api.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off: hipcc would otherwise emit them from scalar code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # a wave-uniform atomic with a returned value would otherwise be rewritten into a wave
    # reduction that waits for the value at once (and for every load issued before it)
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + ["-o", tmp] + SOURCES
    t0 = time.time()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name and says so; that is noise
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
