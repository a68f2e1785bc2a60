"""CPU oracle for the NVFP4 W4A4 quantized linear layer and its sibling formats.

This package is TEST INFRASTRUCTURE. It is a plain, slow, obviously correct
reference of what the GPU path computes: every floating-point step that the
GPU path must reproduce bit for bit is written out in explicit numpy float32,
and the GEMM is an fp64 matmul of exactly decoded operands.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The product package (``fp8_quantized_linear_amd``)
never imports it, and it imports nothing from the product package: the two
share no code. Inputs for both come from the ``synthetic`` package, which holds
random draws only.

Sources. The method is described by three vLLM pull-request write-ups:
"TorchNvFp4LinearKernel" (torch._scaled_mm NVFP4 backend), "QUTLASS NVFP4
online transforms" and "B12X CuTe-DSL linear backends". Those pages fix the
sequence quantize -> block-scaled GEMM -> alpha -> bias, two FP4 values per
byte, the Hadamard block sizes {16, 32, 64, 128} and the 1/sqrt(n)
normalisation. The element formats (E2M1, E4M3, E8M0), the 16-element NVFP4
block and the global scale 448*6/amax are not printed on the pages; they come
from the OCP Microscaling v1.0 / NVFP4 definitions, and each reading taken
where the pages are silent is listed in the design notes.

Parity status per function is stated in each module header.
"""

from .formats import (  # noqa: F401
    E2M1_MAGNITUDES,
    bf16_bits_to_f64,
    bf16_round_bits,
    e2m1_decode,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
    e8m0_decode,
)
from .hadamard import fwht_fp32, hadamard_scale_fp32, sylvester  # noqa: F401
from .nvfp4 import (  # noqa: F401
    amax_for_calibration,
    dequant_nvfp4,
    global_scale_from_amax,
    linear_nvfp4,
    pack_nibbles,
    quant_nvfp4,
    unpack_nibbles,
)
