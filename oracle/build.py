"""Compile the fp64 CPU oracle (plain C, gcc) into oracle/liblforacle.so.

Test infrastructure: the oracle checks the HIP library; it is never part
of the product path.
"""
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lf_oracle.c")
LIB = os.path.join(HERE, "liblforacle.so")


def source_hash(src: str = SRC) -> str:
    """Hash of the oracle's source, written beside the library at build time
    (liblforacle.so.hash) so that a stale build is noticed."""
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def build(src: str = SRC, out: str = LIB, verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-pthread", src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    with open(out + ".hash", "w") as f:
        f.write(source_hash(src) + "\n")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
