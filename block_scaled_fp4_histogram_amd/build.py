"""Builds the gfx950 library block_scaled_fp4_histogram_amd/libmoe_gfx950.so with hipcc."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_gfx950.so")
SOURCES = [os.path.join(CSRC, "moe_kernels.hip"), os.path.join(CSRC, "moe_decode.hip"),
           os.path.join(CSRC, "moe_prefill.hip"), os.path.join(CSRC, "moe_static.hip"),
           os.path.join(CSRC, "moe_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # an entry point that references a missing definition fails here, not at load time
    "-Wl,--no-undefined",
    "-munsafe-fp-atomics",
    # MFMA accumulators in VGPRs: in-place accumulation, no AGPR copies in pipelined loops
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    cmd = [HIPCC] + FLAGS + SOURCES + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err:
        print(err, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
