"""Build libw4a16.so (gfx950) in-tree with hipcc.

    python -m w4a16_weight_only_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libw4a16.so")
SOURCES = ["api.cpp", "gemv.hip", "gemm_mfma.hip", "gemm_shared.hip", "gemm_tile.hip", "gemm_tall.hip", "repack.hip", "glue.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


# hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
_NOISE = "not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if _NOISE not in l)
    if verbose and out.strip():
        print(out)
    return res.returncode, out


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the library."""
    tag = ".tmp%d" % os.getpid()
    objs = [os.path.join(CSRC, s + tag + ".o") for s in SOURCES]
    cmds = [[HIPCC] + [f for f in FLAGS if f != "-shared"] + ["-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    tmp = LIB + tag
    try:
        with ThreadPoolExecutor(max_workers=min(len(cmds), max(1, (os.cpu_count() or 1)))) as ex:
            results = list(ex.map(lambda c: _run(c, verbose), cmds))
        for (rc, out), src in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (src, out))
        rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
        if rc != 0:
            raise RuntimeError("hipcc link failed:\n" + out)
        os.replace(tmp, LIB)
    finally:
        for f in objs + [tmp]:
            if os.path.exists(f):
                os.remove(f)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
