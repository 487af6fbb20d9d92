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
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("kernels.hip", "rows4.hip", "mfma.hip", "fit.hip", "saliency.hip", "api.hip")]

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
    """Compile every source to an object in parallel (one hipcc per file), then link."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    tmp = LIB + ".tmp"
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    t0 = time.time()
    jobs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [hipcc] + compile_flags + ["-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    # hipcc's host pass does not know the packed-fp32 feature name and says so; that is noise
    noise = "is not a recognized feature for this target"
    failed, msgs = False, []
    for p in jobs:
        out, _ = p.communicate()
        msgs += [ln for ln in out.splitlines() if noise not in ln and ln.strip()]
        failed = failed or p.returncode != 0
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
