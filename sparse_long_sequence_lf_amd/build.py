"""Build liblfattn.so (the C-ABI library) for gfx950 with hipcc, in-tree,
and libmfmapeak.so (the benchmark's MFMA-rate probe, not part of the library).

    python -m sparse_long_sequence_lf_amd.build
"""
import glob
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblfattn.so")
SOURCES = [os.path.join(CSRC, "lf_host.cpp"), os.path.join(CSRC, "lf_fwd_kernels.hip"),
           os.path.join(CSRC, "lf_bwd_kernels.hip"), os.path.join(CSRC, "lf_bwd_mfma.hip")]
PEAK_LIB = os.path.join(PKG, "libmfmapeak.so")


def hashed_files():
    """The files liblfattn.so is built from: its sources, the internal
    headers beside them and the public header."""
    return sorted(SOURCES + glob.glob(os.path.join(CSRC, "lf_*.h")) + [os.path.join(INCLUDE, "lf_attn.h")])


def source_hash() -> str:
    """Hash of the library's sources (names and contents); compiled into the
    library (lf_build_hash) so that a loader can refuse a stale build."""
    h = hashlib.sha256()
    for path in hashed_files():
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:16]
PEAK_SOURCE = os.path.join(CSRC, "mfma_peak.hip")

# gfx950 only; packed fp32 VALU ops are kept out of the generated code;
# MFMA accumulators live in ordinary VGPRs (no AGPR copies around the softmax
# rescale of O); machine sinking is off so the next stage's K/V loads stay
# ahead of the current stage's compute instead of being sunk next to their
# LDS stores (which would serialise load latency and compute).
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-disable-machine-sink",
             "-Wno-unused-command-line-argument"]


def build(out: str = LIB, defines=(), verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = []
    tmpdir = os.path.join(PKG, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    dflags = ["-D" + d for d in defines] + ['-DLF_SOURCE_HASH="%s"' % source_hash()]
    for src in SOURCES:
        obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc] + HIP_FLAGS + dflags + ["-I", INCLUDE, "-I", CSRC] + lang + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    return out


def build_peak_probe(out: str = PEAK_LIB, verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc] + HIP_FLAGS + ["-shared", PEAK_SOURCE, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    build_peak_probe(verbose=True)
    sys.exit(0)
