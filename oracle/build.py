"""Build the fp64 CPU oracle (``liboracle.so``) with gcc + OpenMP.

Test infrastructure: the oracle is the reference the HIP library is tested
against; it is built beside it, never linked into it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sol_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
DIGEST = LIB + ".srcdigest"  # digest of the source and flags LIB was built from
FLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]


def source_digest() -> str:
    import hashlib
    with open(SRC, "rb") as fh:
        return hashlib.sha256(fh.read() + b"\0" + " ".join(FLAGS).encode()).hexdigest()


def built_digest():
    try:
        with open(DIGEST) as fh:
            return fh.read().strip()
    except OSError:
        return None


def build(verbose: bool = False) -> str:
    cmd = ["gcc"] + FLAGS + ["-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    with open(DIGEST + ".tmp", "w") as fh:
        fh.write(source_digest() + "\n")
    os.replace(DIGEST + ".tmp", DIGEST)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
