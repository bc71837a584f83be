"""Builds the HIP library libq8gemv.so in-tree for gfx950.

    python -m block_quantized_weight_02_amd.build   (or build() from Python)

hipcc cross-compiles; no GPU is needed to build.  Packed-FP32 instructions are
disabled for every device compile (-Xclang -target-feature -Xclang
-packed-fp32-ops), and fp32 division is correctly rounded (the quantizers
rely on it).
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libq8gemv.so")
SOURCES = ["q8_kernels.hip", "q8_mfma32.hip", "q8_tile16.hip", "q8_gemm.hip", "q8_measure.hip",
           "q8_noalloc.hip", "q8_api.cpp"]
# Per-source device flags.  The GEMM writes its MFMA results to VGPRs (by
# default the compiler routes them through one AGPR quad and serialises the
# matrix core behind its reads).
SOURCE_FLAGS = {"q8_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = os.environ.get("Q8_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    """Compiles every source to an object (in parallel), then links the
    shared library; returns its path."""
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Wall", "-Wno-unused-command-line-argument",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fhip-fp32-correctly-rounded-divide-sqrt",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC, *extra]
    with tempfile.TemporaryDirectory(prefix="q8build") as d:
        objs = [os.path.join(d, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[hipcc(), *flags, *SOURCE_FLAGS.get(s, []), "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = out + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True)
