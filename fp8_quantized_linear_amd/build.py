"""Build libfql.so (the gfx950 HIP library behind include/fql.h) in-tree, and
libfql_calib.so, the measurement aids bench.py loads (streaming-read and
MFMA-loop calibration kernels; not part of the layer).

Usage: python -m fp8_quantized_linear_amd.build   (or call build()).

Every HIP source is compiled for gfx950 only, with:
  * correctly rounded float32 division and kept denormals (the quantizer's
    codes and scales must equal an IEEE reference bit for bit);
  * packed-FP32 instructions disabled (-packed-fp32-ops);
  * no fast-math.
The sources that issue direct global->LDS loads are also compiled to
assembly, and the library is not linked if any of those loads reads an SGPR
sooner after its VALU write than the hardware allows (lds_dma_check).
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

try:
    from . import lds_dma_check
except ImportError:  # run as a script
    import lds_dma_check

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfql.so")
CALIB_LIB = os.path.join(HERE, "libfql_calib.so")
CALIB_SOURCES = ["calib.hip"]

SOURCES = ["fql_api.hip", "quant_nvfp4.hip", "pack_nvfp4.hip", "gemm_nvfp4.hip", "sc_quant.hip",
           "sc_gemm.hip", "transform_nvfp4.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src, obj, verbose):
    cmd = [_hipcc(), *HIPCC_FLAGS, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def lds_dma_violations(src):
    """Wait-state violations before the LDS-DMA loads of one source's kernels."""
    asm = lds_dma_check.device_asm(_hipcc(), HIPCC_FLAGS, CSRC, src,
                                   os.path.join(BUILD, src.replace(".hip", ".s")))
    bad, loads = lds_dma_check.hazards(asm)
    if loads == 0:
        bad.append(f"{src}: no LDS-DMA load found in the assembly")
    return [f"{src}: {b}" for b in bad]


def build(verbose=False):
    """Compile all sources and link libfql.so and libfql_calib.so. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in srcs]
    checked = lds_dma_check.sources_with_lds_dma(CSRC, SOURCES)
    with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        checks = [ex.submit(lds_dma_violations, s) for s in checked]
        list(ex.map(lambda so: _compile(so[0], so[1], verbose), zip(srcs, objs)))
        bad = [b for c in checks for b in c.result()]
    if bad:
        raise RuntimeError("LDS-DMA loads without their wait states (library not linked):\n" +
                           "\n".join(bad[:20]))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], CALIB_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
