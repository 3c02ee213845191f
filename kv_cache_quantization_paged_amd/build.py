"""Build ``libkvfp4.so`` (the C-ABI library) for gfx950 with hipcc, in-tree.

Flags: -ffp-contract=off keeps every fp32 multiply and add separately rounded
(the codes depend on it); fp32 division stays IEEE-correct (hipcc's default);
packed-fp32 instructions are disabled.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libkvfp4.so")
SOURCES = ["abi.hip", "append.hip", "dequant.hip", "materialize.hip", "global_scale.hip", "codec.hip",
           "attention.hip", "table_checks.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the attention kernel rescales and
    # stores them with vector ALU work, which AGPRs would turn into copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    "-Wl,-rpath,/opt/rocm/lib",
]


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [HIPCC] + FLAGS + srcs + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
