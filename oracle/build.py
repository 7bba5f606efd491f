"""Compile the CPU oracle (plain C, gcc) into oracle/libpa_ref.so.

Test infrastructure: the oracle is the fp64 checker for the GPU library, not part of it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libpa_ref.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "pa_ref.c")
    tmp = LIB + ".tmp"
    # -ffp-contract=off keeps every multiply and add separately rounded, so the paged and
    # dense routines (same operation order) agree bit for bit.
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-Wall",
           "-o", tmp, src, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
