"""Builds the fp64 CPU oracle (oracle/liboracle.so) with gcc.

TEST INFRASTRUCTURE ONLY: the library this builds is loaded by the tests, the
smoke check and the benchmark's CPU-baseline leg, never by the product path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "resolvent_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")


def build_oracle(verbose: bool = False) -> str:
    """Compile the oracle; -ffp-contract=off keeps every multiply-add unfused."""
    cmd = [
        "gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        SOURCE, "-o", LIBRARY + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build_oracle(verbose=True))
