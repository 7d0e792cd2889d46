"""Compile the HIP sources under csrc/ into libmoe_hip.so (gfx950 only).

Run as ``python quantized_moe_transformer_amd/build.py`` (the package itself
needs the library to import).  hipcc cross-compiles
for gfx950 without a GPU present.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_hip.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # never emit packed fp32 arithmetic (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments arrive preloaded in registers (kernels
    # whose first argument is a struct are unaffected)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
