"""Build the C-ABI shared library (libsmla.so) for gfx950 with hipcc.

Run ``python -m sparse_mla_decode_top_amd.build`` (or ``__graft_entry__.build()``).
The library is written next to this file; the binding loads it from there.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsmla.so")
SOURCES = [os.path.join(CSRC, "smla_kernels.hip"), os.path.join(CSRC, "smla_prefill.hip"),
           os.path.join(CSRC, "smla_api.cpp")]
# the peak probe (bench.py's measured matrix-core rate), a library of its own
PEAK_LIB = os.path.join(HERE, "libsmla_peak.so")
PEAK_SOURCES = [os.path.join(CSRC, "smla_peak.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # preload the attention kernel's leading scalar arguments into SGPRs
    "-mllvm", "-amdgpu-kernarg-preload-count=8",
    "-Wall", "-Wno-unused-lambda-capture",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(sources, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-x", "hip"] + sources + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, lib)


def build(verbose=False):
    """Compile libsmla.so (the decode) and libsmla_peak.so (the peak probe); always recompiles."""
    _compile(SOURCES, LIB, verbose)
    _compile(PEAK_SOURCES, PEAK_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
