"""Build libint4gemv.so in-tree with hipcc for gfx950.

Flags:
  -O3 --offload-arch=gfx950          CDNA4 only
  -fhip-fp32-correctly-rounded-divide-sqrt, -fno-gpu-flush-denormals-to-zero
                                     IEEE division and subnormals: the quantizer
                                     is bit-exact and the dequant-dot relies on
                                     fp16 subnormals
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                     no packed-fp32 instructions in device code
No fast-math flag of any kind.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libint4gemv.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("kernels.hip", "slice.hip", "gemm.hip", "abi.hip",
                                                   "probe.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature and says so; that is harmless.
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError(f"hipcc failed with status {res.returncode}: {' '.join(cmd[-3:])}")
    if verbose and err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile each source to an object in parallel, then link the shared library."""
    import concurrent.futures
    import tempfile

    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    with tempfile.TemporaryDirectory(prefix="int4gemv_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        cmds = [[hipcc(), *HIPCC_FLAGS, *(extra_flags or []), *inc, "-c", src, "-o", obj]
                for src, obj in zip(SOURCES, objs)]
        with concurrent.futures.ThreadPoolExecutor(len(cmds)) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB_PATH + ".tmp"
        _run([hipcc(), *HIPCC_FLAGS, *(extra_flags or []), *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
