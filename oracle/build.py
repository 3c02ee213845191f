"""Build the CPU oracle library (test infrastructure) with plain gcc.

-ffp-contract=off keeps every fp32 multiply and add a separate rounding; no
-ffast-math, so denormals and IEEE division are kept.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvfp4_oracle.c")
LIB = os.path.join(HERE, "libkvfp4_oracle.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    """Compile ``src`` (by default the oracle) into ``lib``."""
    cmd = [
        "gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
        "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra", "-Wno-unused-parameter",
        src, "-o", lib + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
