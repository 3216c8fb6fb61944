"""Build libmsa.so (all HIP kernels + the C ABI) in-tree for gfx950 with hipcc.

Self-contained on purpose: run it as a script, or load it by file path
(``load_builder()`` in ``__graft_entry__``), since importing the package itself
needs the library it builds."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmsa.so")
SOURCES = ["msa_api.hip", "index_topk.hip", "sparse_attn.hip", "decode.hip", "backward.hip"]


def hipcc_command(out: str = LIB, extra=(), sources=SOURCES) -> list[str]:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    return [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *extra, "-o", out, *[os.path.join(CSRC, s) for s in sources]]


# The benchmark's measured-peak kernels: a library of their own, not part of libmsa.
PEAKS_LIB = os.path.join(PKG, "libmsa_peaks.so")
PEAKS_SOURCES = ["peak_probe.hip"]


def build(verbose: bool = False) -> str:
    for out, srcs in ((LIB, SOURCES), (PEAKS_LIB, PEAKS_SOURCES)):
        tmp = out + ".tmp"
        cmd = hipcc_command(tmp, sources=srcs)
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
