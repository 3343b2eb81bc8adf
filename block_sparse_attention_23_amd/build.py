"""Build libsol.so (HIP, gfx950) in-tree with hipcc.

``python -m block_sparse_attention_23_amd.build`` or ``build()`` from Python.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsol.so")
SOURCES = [os.path.join(CSRC, f) for f in
           ("sol_pool_route.hip", "sol_sweep.hip", "sol_f32.hip", "sol_api.hip")]
HEADERS = [os.path.join(CSRC, "sol_device.h"), os.path.join(CSRC, "sol_launch.h"),
           os.path.join(CSRC, "sol_tile.h"), os.path.join(INCLUDE, "sol.h")]
ARCH = "gfx950"
DIGEST = LIB + ".srcdigest"  # digest of the sources and flags LIB was built from

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 VALU forms in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def digest_flags(extra=()):
    """The compiler flags that enter the digest: all but the include paths,
    which depend on where the tree sits (the same tree is built in one place
    and loaded from another)."""
    return [f for f in HIPCC_FLAGS + list(extra) if not f.startswith("-I")]


def source_digest(extra=()) -> str:
    """sha256 over the library's sources, headers and compiler flags."""
    import hashlib
    h = hashlib.sha256()
    for f in SOURCES + HEADERS:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read() + b"\0")
    h.update(" ".join(digest_flags(extra)).encode())
    return h.hexdigest()


def built_digest():
    """The digest recorded when LIB was built (None if there is none)."""
    try:
        with open(DIGEST) as fh:
            return fh.read().strip()
    except OSError:
        return None


def check_current():
    """Raise unless LIB exists and was built from the sources as they are now."""
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: build it with "
                           "`python -m block_sparse_attention_23_amd.build` (hipcc, gfx950)")
    if built_digest() != source_digest():
        raise RuntimeError(f"{LIB} is stale: it was not built from the current sources "
                           "(rebuild with `python -m block_sparse_attention_23_amd.build`)")


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def build(verbose: bool = False, extra=()) -> str:
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra) + ["-o", LIB + ".tmp"] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    with open(DIGEST + ".tmp", "w") as fh:
        fh.write(source_digest(extra) + "\n")
    os.replace(DIGEST + ".tmp", DIGEST)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
