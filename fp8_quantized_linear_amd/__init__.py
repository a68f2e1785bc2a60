"""NVFP4 W4A4 quantized linear layer for AMD MI355X (gfx950).

Thin Python binding over the C ABI in include/fql.h (libfql.so, built
in-tree by fp8_quantized_linear_amd.build). This module only marshals
arguments: every step of the layer runs in the library's HIP kernels.
PyTorch provides device memory and the current stream.

Typical use (weights quantized and packed once, activations per call):

    w = NVFP4Weight.from_float(w_fp32_cuda, input_global_scale=g_x)
    y = linear_nvfp4(x_bf16_cuda, w, bias=b)

The layer follows the vLLM write-ups' NVFP4 linear path ("TorchNvFp4LinearKernel",
"B12X CuTe-DSL linear backends"): quantize x with the layer's input global
scale, block-scaled GEMM with the packed weight, multiply by alpha (the
product of the two global dequant scales), add the bias, keep the input dtype
and the shape [*x.shape[:-1], N].
"""

import ctypes
import os
import threading

import torch

__all__ = [
    "FQLError",
    "lib",
    "is_supported",
    "can_implement",
    "amax",
    "global_scale_from_amax",
    "quant_nvfp4",
    "quant_nvfp4_weight",
    "packed_nvfp4_bytes",
    "pack_weight_nvfp4",
    "unpack_weight_nvfp4",
    "linear_workspace_bytes",
    "linear_plan",
    "new_workspace",
    "linear_nvfp4",
    "NVFP4Weight",
    "HADAMARD_BLOCKS",
    "quant_mxfp4",
    "quant_mxfp4_weight",
    "packed_mxfp4_bytes",
    "pack_weight_mxfp4",
    "linear_mxfp4_workspace_bytes",
    "linear_mxfp4_plan",
    "linear_mxfp4",
    "MXFP4Weight",
    "quant_mxfp8",
    "quant_mxfp8_weight",
    "pack_weight_mxfp8",
    "linear_mxfp8",
    "MXFP8Weight",
    "quant_fp8",
    "quant_fp8_weight",
    "pack_weight_fp8",
    "linear_fp8",
    "FP8Weight",
    "quant_fp8_block",
    "quant_fp8_block_weight",
    "pack_weight_fp8_block",
    "linear_fp8_block",
    "FP8BlockWeight",
    "fp8_scale_from_amax",
    "linear_sc_plan",
    "linear_sc_workspace_bytes",
    "warmup",
    "token_counts_for_warmup",
    "transform_bf16",
    "quant_nvfp4_transform",
    "quant_nvfp4_dynamic",
    "nvfp4_alpha",
    "fp8_output_scale",
    "set_plan_override",
    "plan_override",
    "linear_nvfp4_quantize",
    "linear_nvfp4_gemm",
    "linear_nvfp4_noalloc",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfql.so")
HADAMARD_BLOCKS = (0, 16, 32, 64, 128)
FMT_NVFP4 = 1
FMT_MXFP4 = 2
FMT_MXFP8 = 3
FMT_FP8 = 4
FMT_FP8_BLOCK = 5

_c_int, _c_i64, _c_f32, _c_vp, _c_sz = (ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                         ctypes.c_void_p, ctypes.c_size_t)

# name -> (restype, argtypes); must match include/fql.h
SIGNATURES = {
    "fql_version": (_c_int, []),
    "fql_last_error": (ctypes.c_char_p, []),
    "fql_is_supported": (_c_int, [_c_int, ctypes.c_char_p, _c_sz]),
    "fql_can_implement": (_c_int, [_c_int, _c_i64, _c_i64, _c_int, ctypes.c_char_p, _c_sz]),
    "fql_amax_bf16": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_vp]),
    "fql_amax_f32": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_vp]),
    "fql_quant_nvfp4": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_f32, _c_int, _c_vp, _c_vp, _c_vp]),
    "fql_quant_nvfp4_f32": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_f32, _c_int, _c_vp, _c_vp, _c_vp]),
    "fql_packed_nvfp4_bytes": (_c_int, [_c_i64, _c_i64, ctypes.POINTER(_c_sz)]),
    "fql_pack_weight_nvfp4": (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fql_unpack_weight_nvfp4": (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "fql_linear_nvfp4_workspace_bytes": (_c_int, [_c_i64, _c_i64, _c_i64, ctypes.POINTER(_c_sz)]),
    "fql_linear_nvfp4_describe": (_c_int, [_c_i64, _c_i64, _c_i64, _c_int, ctypes.c_char_p, _c_sz]),
    "fql_linear_nvfp4": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_f32, _c_int, _c_vp, _c_i64,
                                  _c_f32, _c_vp, _c_vp, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fql_quant_mxfp8": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "fql_quant_mxfp8_f32": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "fql_packed_mxfp8_bytes": (_c_int, [_c_i64, _c_i64, ctypes.POINTER(_c_sz)]),
    "fql_pack_weight_mxfp8": (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fql_linear_mxfp8_workspace_bytes": (_c_int, [_c_i64, _c_i64, _c_i64, ctypes.POINTER(_c_sz)]),
    "fql_linear_mxfp8_describe": (_c_int, [_c_i64, _c_i64, _c_i64, ctypes.c_char_p, _c_sz]),
    "fql_linear_mxfp8": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_f32, _c_vp,
                                  _c_vp, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fql_quant_fp8": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_f32, _c_vp, _c_vp]),
    "fql_quant_fp8_f32": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_f32, _c_vp, _c_vp]),
    "fql_packed_fp8_bytes": (_c_int, [_c_i64, _c_i64, ctypes.POINTER(_c_sz)]),
    "fql_pack_weight_fp8": (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fql_linear_fp8_workspace_bytes": (_c_int, [_c_i64, _c_i64, _c_i64, ctypes.POINTER(_c_sz)]),
    "fql_linear_fp8_describe": (_c_int, [_c_i64, _c_i64, _c_i64, ctypes.c_char_p, _c_sz]),
    "fql_linear_fp8": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_f32, _c_vp, _c_i64, _c_f32,
                                _c_vp, _c_vp, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fql_quant_fp8_block": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "fql_quant_fp8_block_weight_f32": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "fql_packed_fp8_block_bytes": (_c_int, [_c_i64, _c_i64, ctypes.POINTER(_c_sz)]),
    "fql_pack_weight_fp8_block": (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fql_linear_fp8_block_workspace_bytes": (_c_int, [_c_i64, _c_i64, _c_i64, ctypes.POINTER(_c_sz)]),
    "fql_linear_fp8_block_describe": (_c_int, [_c_i64, _c_i64, _c_i64, ctypes.c_char_p, _c_sz]),
    "fql_linear_fp8_block": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_f32, _c_vp,
                                      _c_vp, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fql_transform_bf16": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_int, _c_vp, _c_i64,
                                    _c_vp]),
    "fql_quant_nvfp4_transform": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_f32, _c_vp, _c_int,
                                           _c_vp, _c_vp, _c_vp]),
    "fql_quant_nvfp4_dynamic": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_int, _c_vp,
                                         _c_vp, _c_vp, _c_vp]),
    "fql_linear_nvfp4_transform": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_f32, _c_vp, _c_int,
                                            _c_vp, _c_i64, _c_f32, _c_vp, _c_vp, _c_i64, _c_vp,
                                            _c_sz, _c_vp]),
    "fql_linear_nvfp4_dynamic": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_int, _c_vp,
                                          _c_i64, _c_f32, _c_vp, _c_vp, _c_i64, _c_vp, _c_sz,
                                          _c_vp]),
    "fql_quant_mxfp4": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "fql_quant_mxfp4_f32": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "fql_packed_mxfp4_bytes": (_c_int, [_c_i64, _c_i64, ctypes.POINTER(_c_sz)]),
    "fql_pack_weight_mxfp4": (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fql_linear_mxfp4_workspace_bytes": (_c_int, [_c_i64, _c_i64, _c_i64, ctypes.POINTER(_c_sz)]),
    "fql_linear_mxfp4_describe": (_c_int, [_c_i64, _c_i64, _c_i64, ctypes.c_char_p, _c_sz]),
    "fql_linear_mxfp4": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_f32, _c_vp,
                                  _c_vp, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fql_linear_nvfp4_dev_alpha": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_f32, _c_int, _c_vp,
                                            _c_i64, _c_vp, _c_vp, _c_vp, _c_i64, _c_vp, _c_sz,
                                            _c_vp]),
    "fql_linear_fp8_dev_alpha": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_f32, _c_vp, _c_i64,
                                          _c_vp, _c_vp, _c_vp, _c_i64, _c_vp, _c_sz, _c_vp]),
    "fql_linear_nvfp4_quantize": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_f32, _c_int, _c_i64,
                                           _c_vp, _c_sz, _c_vp]),
    "fql_linear_nvfp4_gemm": (_c_int, [_c_i64, _c_i64, _c_int, _c_vp, _c_i64, _c_f32, _c_vp, _c_vp,
                                       _c_i64, _c_vp, _c_sz, _c_vp]),
    "fql_nvfp4_global_scale": (_c_int, [_c_f32, ctypes.POINTER(_c_f32)]),
    "fql_nvfp4_alpha": (_c_int, [_c_f32, _c_f32, ctypes.POINTER(_c_f32)]),
    "fql_fp8_scale": (_c_int, [_c_f32, ctypes.POINTER(_c_f32)]),
    "fql_fp8_output_scale": (_c_int, [_c_f32, _c_f32, ctypes.POINTER(_c_f32)]),
    "fql_set_plan_override": (_c_int, [_c_int, ctypes.c_char_p]),
    "fql_linear_nvfp4_noalloc": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_f32, _c_int, _c_vp,
                                          _c_i64, _c_f32, _c_vp, _c_vp, _c_i64, _c_vp]),
}

PLAN_OVERRIDES = {"nvfp4": 0, "sc_gemm": 1, "sc_gemv": 2}  # FQL_PLAN_NVFP4, _SC_GEMM, _SC_GEMV


class FQLError(RuntimeError):
    """An error status returned by the library (message from fql_last_error)."""


_lib = None
_lib_lock = threading.Lock()


def lib():
    """The loaded libfql.so (built in-tree on first use if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                from . import build as _build

                _build.build()
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def _check(status):
    if status < 0:
        raise FQLError(f"fql error {status}: {lib().fql_last_error().decode()}")
    return status


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _require_cuda(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise FQLError(f"{name} must be a CUDA (HIP) tensor")


def _rows_view(x, name):
    """(2-D view [M, K], row stride) of x [..., K] without copying."""
    if x.dim() < 1:
        raise FQLError(f"{name} must have at least one dimension")
    if x.stride(-1) != 1:
        raise FQLError(f"{name} must have unit stride in its last dimension")
    K = x.shape[-1]
    if x.dim() == 1:
        return x.view(1, K), K
    try:
        x2 = x.view(-1, K) if x.dim() > 2 else x
    except RuntimeError as e:
        raise FQLError(f"{name}: leading dimensions cannot be flattened without a copy") from e
    ld = x2.stride(0) if x2.shape[0] > 1 else max(K, x2.stride(0))
    return x2, ld


# ---------------------------------------------------------------------------
# availability
# ---------------------------------------------------------------------------

def is_supported(device=0):
    buf = ctypes.create_string_buffer(256)
    r = _check(lib().fql_is_supported(int(device), buf, 256))
    return bool(r), buf.value.decode()


def can_implement(N, K, hadamard_block=0, fmt=FMT_NVFP4):
    buf = ctypes.create_string_buffer(256)
    r = _check(lib().fql_can_implement(int(fmt), int(N), int(K), int(hadamard_block), buf, 256))
    return bool(r), buf.value.decode()


# ---------------------------------------------------------------------------
# quantizer
# ---------------------------------------------------------------------------

def amax(x, hadamard_block=0):
    """max |v| of x (bf16 or float32, [..., K]) after the optional rotation; 0-d float32 tensor."""
    _require_cuda(x, "x")
    x2, ld = _rows_view(x, "x")
    M, K = x2.shape
    out = torch.empty((), dtype=torch.float32, device=x.device)
    if x.dtype == torch.bfloat16:
        fn = lib().fql_amax_bf16
    elif x.dtype == torch.float32:
        fn = lib().fql_amax_f32
    else:
        raise FQLError("amax supports bfloat16 and float32 inputs")
    _check(fn(_ptr(x2), M, K, ld, int(hadamard_block), _ptr(out), _stream(x.device)))
    return out


def _host_scalar(name, *args):
    out = _c_f32()
    _check(getattr(lib(), name)(*[_c_f32(float(a)) for a in args], ctypes.byref(out)))
    return out.value


def global_scale_from_amax(amax_value):
    """The NVFP4 global scale g = fl32(448 * 6 / amax) of a calibration amax
    (1 when amax is 0, at most 2^118), from the library (host-side)."""
    return _host_scalar("fql_nvfp4_global_scale", amax_value)


def nvfp4_alpha(input_global_scale, weight_global_scale):
    """alpha = fl32((1/g_x) * (1/g_w)), the product of the two global dequant scales."""
    return _host_scalar("fql_nvfp4_alpha", input_global_scale, weight_global_scale)


def fp8_output_scale(input_scale, weight_scale):
    """The per-tensor FP8 output scale fl32(s_x * s_w)."""
    return _host_scalar("fql_fp8_output_scale", input_scale, weight_scale)


def set_plan_override(spec, which="nvfp4"):
    """Replace a launch-plan override (benchmarking and tests): `which` is "nvfp4"
    (FQL_PLAN syntax), "sc_gemm" (FQL_SC_PLAN) or "sc_gemv" (FQL_SC_GEMV); None
    or "" removes it. Results change at most in the float32 summation order."""
    _check(lib().fql_set_plan_override(PLAN_OVERRIDES[which],
                                       None if not spec else str(spec).encode()))


class plan_override:
    """Context manager: `with plan_override("kind=3,mt=4,nt=2,st=3"): ...` sets the
    override on entry and removes it on exit."""

    def __init__(self, spec, which="nvfp4"):
        self.spec, self.which = spec, which

    def __enter__(self):
        set_plan_override(self.spec, self.which)
        return self

    def __exit__(self, *exc):
        set_plan_override(None, self.which)
        return False


def quant_nvfp4(x, global_scale, hadamard_block=0, codes=None, scales=None):
    """Quantize bf16 x [..., K] to NVFP4: (codes uint8 [..., K/2], scales uint8 [..., K/16])."""
    _require_cuda(x, "x")
    if x.dtype != torch.bfloat16:
        raise FQLError("quant_nvfp4 takes bfloat16 activations")
    x2, ld = _rows_view(x, "x")
    M, K = x2.shape
    lead = tuple(x.shape[:-1])
    if codes is None:
        codes = torch.empty(lead + (K // 2,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(lead + (K // 16,), dtype=torch.uint8, device=x.device)
    _check(lib().fql_quant_nvfp4(_ptr(x2), M, K, ld, float(global_scale), int(hadamard_block),
                                 _ptr(codes), _ptr(scales), _stream(x.device)))
    return codes, scales


def quant_nvfp4_weight(w, global_scale, hadamard_block=0):
    """Quantize float32 weights w [N, K] (rows rotated if hadamard_block > 0)."""
    _require_cuda(w, "w")
    if w.dtype != torch.float32:
        raise FQLError("quant_nvfp4_weight takes float32 weights")
    w2, ld = _rows_view(w, "w")
    N, K = w2.shape
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, K // 16), dtype=torch.uint8, device=w.device)
    _check(lib().fql_quant_nvfp4_f32(_ptr(w2), N, K, ld, float(global_scale), int(hadamard_block),
                                     _ptr(codes), _ptr(scales), _stream(w.device)))
    return codes, scales


# ---------------------------------------------------------------------------
# packer
# ---------------------------------------------------------------------------

def packed_nvfp4_bytes(N, K):
    n = ctypes.c_size_t()
    _check(lib().fql_packed_nvfp4_bytes(int(N), int(K), ctypes.byref(n)))
    return n.value


def pack_weight_nvfp4(codes, scales, out=None):
    """Re-lay canonical NVFP4 weight (codes [N, K/2], scales [N, K/16]) for the GEMM."""
    _require_cuda(codes, "codes")
    N, K = codes.shape[0], codes.shape[1] * 2
    if not (codes.is_contiguous() and scales.is_contiguous()):
        raise FQLError("codes and scales must be contiguous")
    if tuple(scales.shape) != (N, K // 16):
        raise FQLError("scales must be [N, K/16]")
    nbytes = packed_nvfp4_bytes(N, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    _check(lib().fql_pack_weight_nvfp4(_ptr(codes), _ptr(scales), N, K, _ptr(out), out.numel(),
                                       _stream(codes.device)))
    return out


def unpack_weight_nvfp4(packed, N, K):
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=packed.device)
    scales = torch.empty((N, K // 16), dtype=torch.uint8, device=packed.device)
    _check(lib().fql_unpack_weight_nvfp4(_ptr(packed), int(N), int(K), _ptr(codes), _ptr(scales),
                                         _stream(packed.device)))
    return codes, scales


class NVFP4Weight:
    """A packed NVFP4 weight and the layer constants the linear call needs.

    packed: uint8 device buffer from pack_weight_nvfp4; N, K: logical shape;
    input_global_scale: the activation encode scale g_x (static calibration);
    weight_global_scale: g_w; hadamard_block: rotation block (0 = none).
    alpha = 1 / (g_x * g_w) rounded once to float32.
    transform: optional bf16 [b, b] device matrix T (b in {16, 32, 64, 128}),
    a general block-diagonal transform applied to the activation in place of
    the Hadamard rotation (the weight must have been transformed alike
    offline). dynamic_input_scale: g_x is computed from each call's
    activation (448 * 6 / amax) on the device instead of the static scale.
    alpha_dev: alpha as a float32 device scalar, which linear_nvfp4 reads
    when no alpha is passed, so repack_ with a new weight global scale keeps
    captured graphs valid.
    """

    def __init__(self, packed, N, K, input_global_scale, weight_global_scale, hadamard_block=0,
                 transform=None, dynamic_input_scale=False):
        self.packed = packed
        self.N, self.K = int(N), int(K)
        self.input_global_scale = float(input_global_scale)
        self.weight_global_scale = float(weight_global_scale)
        self.hadamard_block = int(hadamard_block)
        if transform is not None:
            _transform_matrix(transform)
            if self.hadamard_block:
                raise FQLError("a weight takes either a Hadamard block or a transform matrix")
        self.transform = transform
        self.dynamic_input_scale = bool(dynamic_input_scale)
        self.alpha = nvfp4_alpha(self.input_global_scale, self.weight_global_scale)
        self.alpha_dev = torch.full((1,), self.alpha, dtype=torch.float32, device=packed.device)

    @classmethod
    def from_float(cls, w, input_global_scale, hadamard_block=0, weight_global_scale=None,
                   transform=None, dynamic_input_scale=False):
        """Quantize and pack a float32 weight [N, K] on the GPU (already
        transformed when `transform` is given)."""
        if weight_global_scale is None:
            weight_global_scale = global_scale_from_amax(amax(w, hadamard_block).item())
        codes, scales = quant_nvfp4_weight(w, weight_global_scale, hadamard_block)
        packed = pack_weight_nvfp4(codes, scales)
        return cls(packed, w.shape[0], w.shape[1], input_global_scale, weight_global_scale,
                   hadamard_block, transform=transform, dynamic_input_scale=dynamic_input_scale)

    def repack_(self, codes, scales, weight_global_scale=None):
        """Re-pack new canonical weights into the same storage (address kept).

        weight_global_scale: the new weight's g_w when it differs from the old
        one; alpha is then recomputed and written to alpha_dev in stream order,
        so graphs captured on calls without an explicit alpha replay with it.
        Weights with a transform or a dynamic input scale pass g_w to the
        library by value and reject a changed scale.
        """
        pack_weight_nvfp4(codes, scales, out=self.packed)
        if weight_global_scale is not None and float(weight_global_scale) != self.weight_global_scale:
            if self.transform is not None or self.dynamic_input_scale:
                raise FQLError("a weight with a transform or a dynamic input scale keeps its "
                               "weight global scale across repack_")
            alpha = nvfp4_alpha(self.input_global_scale, weight_global_scale)
            self.weight_global_scale = float(weight_global_scale)
            self.alpha = alpha
            self.alpha_dev.fill_(alpha)
        return self


# ---------------------------------------------------------------------------
# linear
# ---------------------------------------------------------------------------

def linear_workspace_bytes(M, N, K):
    n = ctypes.c_size_t()
    _check(lib().fql_linear_nvfp4_workspace_bytes(int(M), int(N), int(K), ctypes.byref(n)))
    return n.value


def linear_plan(M, N, K, aligned=True, transform=False, hadamard_block=0):
    """One-line description of the kernel/launch plan a linear call of this shape uses
    (`transform`: the plan of a call with a general transform matrix; `hadamard_block`:
    that of a call with this block Hadamard rotation, 0 for none)."""
    buf = ctypes.create_string_buffer(256)
    flags = int(bool(aligned)) | (2 if transform else 0) | (4 if hadamard_block else 0)
    _check(lib().fql_linear_nvfp4_describe(int(M), int(N), int(K), flags, buf, 256))
    return buf.value.decode()


_workspaces = {}


def new_workspace(nbytes, device):
    """A zero-filled workspace buffer (its leading arrival counters must start at zero;
    every linear call leaves them zero again). One workspace per stream at a time."""
    return torch.zeros(max(int(nbytes), 1 << 20), dtype=torch.uint8, device=device)


def _workspace(device, nbytes):
    key = (device.type, device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = new_workspace(nbytes, device)
        _workspaces[key] = ws
    return ws


def linear_nvfp4(x, weight, alpha=None, bias=None, out=None, workspace=None):
    """y = bf16(alpha * quant(x) @ W^T + bias) for bf16 x [..., K]; returns [..., N]."""
    _require_cuda(x, "x")
    if x.dtype != torch.bfloat16:
        raise FQLError("linear_nvfp4 takes bfloat16 activations")
    if x.shape[-1] != weight.K:
        raise FQLError(f"x has K={x.shape[-1]}, weight has K={weight.K}")
    x2, ld = _rows_view(x, "x")
    M, K = x2.shape
    N = weight.N
    alpha_dev = getattr(weight, "alpha_dev", None) if alpha is None else None
    if alpha is None:
        alpha = weight.alpha
    if bias is not None:
        _require_cuda(bias, "bias")
        if bias.dtype != torch.bfloat16 or bias.numel() != N or not bias.is_contiguous():
            raise FQLError("bias must be a contiguous bf16 tensor of N elements")
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (N,), dtype=torch.bfloat16, device=x.device)
    y2, ldy = _rows_view(out, "out")
    need = linear_workspace_bytes(M, N, K)
    if workspace is None:
        workspace = _workspace(x.device, need)
    T = getattr(weight, "transform", None)
    if getattr(weight, "dynamic_input_scale", False):
        b = T.shape[0] if T is not None else weight.hadamard_block
        _check(lib().fql_linear_nvfp4_dynamic(_ptr(x2), M, K, ld, _ptr(T), b, _ptr(weight.packed), N,
                                              weight.weight_global_scale, _ptr(bias), _ptr(y2), ldy,
                                              _ptr(workspace), workspace.numel(), _stream(x.device)))
    elif T is not None:
        _check(lib().fql_linear_nvfp4_transform(_ptr(x2), M, K, ld, weight.input_global_scale,
                                                _ptr(T), T.shape[0], _ptr(weight.packed), N,
                                                float(alpha), _ptr(bias), _ptr(y2), ldy,
                                                _ptr(workspace), workspace.numel(),
                                                _stream(x.device)))
    elif alpha_dev is not None:
        _check(lib().fql_linear_nvfp4_dev_alpha(_ptr(x2), M, K, ld, weight.input_global_scale,
                                                weight.hadamard_block, _ptr(weight.packed), N,
                                                _ptr(alpha_dev), _ptr(bias), _ptr(y2), ldy,
                                                _ptr(workspace), workspace.numel(),
                                                _stream(x.device)))
    else:
        _check(lib().fql_linear_nvfp4(_ptr(x2), M, K, ld, weight.input_global_scale,
                                      weight.hadamard_block, _ptr(weight.packed), N, float(alpha),
                                      _ptr(bias), _ptr(y2), ldy, _ptr(workspace), workspace.numel(),
                                      _stream(x.device)))
    return out


def linear_nvfp4_noalloc(x, weight, out, alpha=None, bias=None):
    """linear_nvfp4 for callers that cannot allocate: no workspace, the library's
    static per-device scratch instead (FQL_NOALLOC_SCRATCH_BYTES; larger calls
    raise). `out` (bf16 [..., N]) must be given; calls that overlap in time on
    one device race on the shared scratch."""
    _require_cuda(x, "x")
    if x.dtype != torch.bfloat16:
        raise FQLError("linear_nvfp4_noalloc takes bfloat16 activations")
    if x.shape[-1] != weight.K:
        raise FQLError(f"x has K={x.shape[-1]}, weight has K={weight.K}")
    if getattr(weight, "transform", None) is not None or getattr(weight, "dynamic_input_scale", False):
        raise FQLError("linear_nvfp4_noalloc takes plain (optionally Hadamard-rotated) weights")
    x2, ld = _rows_view(x, "x")
    M, K = x2.shape
    if bias is not None:
        _require_cuda(bias, "bias")
        if bias.dtype != torch.bfloat16 or bias.numel() != weight.N or not bias.is_contiguous():
            raise FQLError("bias must be a contiguous bf16 tensor of N elements")
    y2, ldy = _rows_view(out, "out")
    a = weight.alpha if alpha is None else alpha
    _check(lib().fql_linear_nvfp4_noalloc(_ptr(x2), M, K, ld, weight.input_global_scale,
                                          weight.hadamard_block, _ptr(weight.packed), weight.N,
                                          float(a), _ptr(bias), _ptr(y2), ldy, _stream(x.device)))
    return out


def linear_nvfp4_quantize(x, weight, workspace):
    """Diagnostics: the quantizer half of linear_nvfp4 (plain weights only): writes
    the GEMM's activation operand into `workspace` exactly as the linear call does."""
    _require_cuda(x, "x")
    x2, ld = _rows_view(x, "x")
    M, K = x2.shape
    _check(lib().fql_linear_nvfp4_quantize(_ptr(x2), M, K, ld, weight.input_global_scale,
                                           weight.hadamard_block, weight.N, _ptr(workspace),
                                           workspace.numel(), _stream(x.device)))
    return workspace


def linear_nvfp4_gemm(M, weight, workspace, alpha, x_aligned=True, bias=None, out=None):
    """Diagnostics: the GEMM half of linear_nvfp4 on the operand linear_nvfp4_quantize
    left in `workspace`; returns y bf16 [M, N]."""
    N = weight.N
    if out is None:
        out = torch.empty((int(M), N), dtype=torch.bfloat16, device=workspace.device)
    y2, ldy = _rows_view(out, "out")
    _check(lib().fql_linear_nvfp4_gemm(int(M), weight.K, int(bool(x_aligned)), _ptr(weight.packed), N,
                                       float(alpha), _ptr(bias), _ptr(y2), ldy, _ptr(workspace),
                                       workspace.numel(), _stream(workspace.device)))
    return out


# ---------------------------------------------------------------------------
# general block-diagonal transform, dynamic global scale
# ---------------------------------------------------------------------------

def _transform_matrix(T):
    _require_cuda(T, "transform")
    if (T.dtype != torch.bfloat16 or T.dim() != 2 or T.shape[0] != T.shape[1]
            or T.shape[0] not in (16, 32, 64, 128) or not T.is_contiguous()
            or T.data_ptr() % 16 != 0):
        raise FQLError("transform must be a contiguous, 16-byte aligned bf16 [b, b] matrix, "
                       "b in {16, 32, 64, 128}")
    return T.shape[0]


def transform_bf16(x, T):
    """v = per-chunk T @ x (float32 [..., K]) for bf16 x [..., K]: the block-diagonal
    transform alone, as the quantizer applies it."""
    _require_cuda(x, "x")
    if x.dtype != torch.bfloat16:
        raise FQLError("transform_bf16 takes bfloat16 activations")
    b = _transform_matrix(T)
    x2, ld = _rows_view(x, "x")
    M, K = x2.shape
    v = torch.empty(tuple(x.shape[:-1]) + (K,), dtype=torch.float32, device=x.device)
    _check(lib().fql_transform_bf16(_ptr(x2), M, K, ld, _ptr(T), b, _ptr(v), K, _stream(x.device)))
    return v


def quant_nvfp4_transform(x, T, global_scale, codes=None, scales=None):
    """NVFP4-quantize per-chunk T @ x: (codes uint8 [..., K/2], scales uint8 [..., K/16])."""
    _require_cuda(x, "x")
    if x.dtype != torch.bfloat16:
        raise FQLError("quant_nvfp4_transform takes bfloat16 activations")
    b = _transform_matrix(T)
    x2, ld = _rows_view(x, "x")
    M, K = x2.shape
    lead = tuple(x.shape[:-1])
    if codes is None:
        codes = torch.empty(lead + (K // 2,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(lead + (K // 16,), dtype=torch.uint8, device=x.device)
    _check(lib().fql_quant_nvfp4_transform(_ptr(x2), M, K, ld, float(global_scale), _ptr(T), b,
                                           _ptr(codes), _ptr(scales), _stream(x.device)))
    return codes, scales


DYNAMIC_SCALARS = 68  # FQL_DYNAMIC_SCALARS: 64 partial maxima, amax, g


def quant_nvfp4_dynamic(x, T=None, hadamard_block=0):
    """NVFP4-quantize x with g = 448 * 6 / amax computed on the device from this
    activation (after the transform T, or the Hadamard rotation, if any).
    Returns (codes, scales, scalars): scalars float32 [2] on the device,
    [0] = amax, [1] = g."""
    _require_cuda(x, "x")
    if x.dtype != torch.bfloat16:
        raise FQLError("quant_nvfp4_dynamic takes bfloat16 activations")
    b = _transform_matrix(T) if T is not None else int(hadamard_block)
    x2, ld = _rows_view(x, "x")
    M, K = x2.shape
    lead = tuple(x.shape[:-1])
    codes = torch.empty(lead + (K // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(lead + (K // 16,), dtype=torch.uint8, device=x.device)
    buf = torch.empty(DYNAMIC_SCALARS, dtype=torch.float32, device=x.device)
    _check(lib().fql_quant_nvfp4_dynamic(_ptr(x2), M, K, ld, _ptr(T), b, _ptr(buf), _ptr(codes),
                                         _ptr(scales), _stream(x.device)))
    return codes, scales, buf[64:66]


# ---------------------------------------------------------------------------
# scaled-MFMA formats: MXFP4, MXFP8 (E8M0 per 32), per-tensor FP8, block FP8
# ---------------------------------------------------------------------------

_SC = {"mxfp4": "mxfp4", "mxfp8": "mxfp8", "fp8": "fp8", "fp8_block": "fp8_block"}


def _fn(name):
    return getattr(lib(), name)


def _size_query(name, *args):
    n = ctypes.c_size_t()
    _check(_fn(name)(*[int(a) for a in args], ctypes.byref(n)))
    return n.value


def _sc_codes_shape(fmt, lead, K):
    return lead + ((K // 2,) if fmt == "mxfp4" else (K,))


def _quant_sc(fmt, x, name, dtype, fn, scale=None, weight_tiles=False):
    _require_cuda(x, name)
    if x.dtype != dtype:
        raise FQLError(f"{name} must be {dtype}")
    x2, ld = _rows_view(x, name)
    M, K = x2.shape
    lead = tuple(x.shape[:-1])
    codes = torch.empty(_sc_codes_shape(fmt, lead, K), dtype=torch.uint8, device=x.device)
    if fmt in ("mxfp4", "mxfp8"):
        scales = torch.empty(lead + (K // 32,), dtype=torch.uint8, device=x.device)
    elif fmt == "fp8_block":
        shape = (M // 128, K // 128) if weight_tiles else lead + (K // 128,)
        scales = torch.empty(shape, dtype=torch.float32, device=x.device)
    else:
        scales = None
    if fmt == "fp8":
        _check(fn(_ptr(x2), M, K, ld, float(scale), _ptr(codes), _stream(x.device)))
        return codes
    _check(fn(_ptr(x2), M, K, ld, _ptr(codes), _ptr(scales), _stream(x.device)))
    return codes, scales


def quant_mxfp4(x):
    """Quantize bf16 x [..., K] to MXFP4: (codes uint8 [..., K/2], scales uint8 [..., K/32])."""
    return _quant_sc("mxfp4", x, "x", torch.bfloat16, _fn("fql_quant_mxfp4"))


def quant_mxfp4_weight(w):
    """Quantize float32 weights w [N, K] to MXFP4 (codes, scales)."""
    return _quant_sc("mxfp4", w, "w", torch.float32, _fn("fql_quant_mxfp4_f32"))


def quant_mxfp8(x):
    """Quantize bf16 x [..., K] to MXFP8: (codes uint8 [..., K], scales uint8 [..., K/32])."""
    return _quant_sc("mxfp8", x, "x", torch.bfloat16, _fn("fql_quant_mxfp8"))


def quant_mxfp8_weight(w):
    return _quant_sc("mxfp8", w, "w", torch.float32, _fn("fql_quant_mxfp8_f32"))


def quant_fp8(x, scale):
    """Per-tensor FP8 codes uint8 [..., K] of bf16 x with the float32 scale s (q = E4M3(x * fl32(1/s)))."""
    return _quant_sc("fp8", x, "x", torch.bfloat16, _fn("fql_quant_fp8"), scale=scale)


def quant_fp8_weight(w, scale):
    return _quant_sc("fp8", w, "w", torch.float32, _fn("fql_quant_fp8_f32"), scale=scale)


def quant_fp8_block(x):
    """Block FP8 of bf16 x [..., K]: (codes uint8 [..., K], scales float32 [..., K/128])."""
    return _quant_sc("fp8_block", x, "x", torch.bfloat16, _fn("fql_quant_fp8_block"))


def quant_fp8_block_weight(w):
    """Block FP8 of float32 w [N, K] over 128 x 128 tiles: (codes [N, K], scales [N/128, K/128])."""
    return _quant_sc("fp8_block", w, "w", torch.float32, _fn("fql_quant_fp8_block_weight_f32"),
                     weight_tiles=True)


def fp8_scale_from_amax(amax_value):
    """The per-tensor FP8 calibration scale fl32(amax / 448) (1 when that is 0), from
    the library (host-side)."""
    return _host_scalar("fql_fp8_scale", amax_value)


def packed_mxfp4_bytes(N, K):
    return _size_query("fql_packed_mxfp4_bytes", N, K)


def _pack_sc(fmt, codes, scales, out):
    _require_cuda(codes, "codes")
    N = codes.shape[0]
    K = codes.shape[1] * (2 if fmt == "mxfp4" else 1)
    if not codes.is_contiguous() or (scales is not None and not scales.is_contiguous()):
        raise FQLError("codes and scales must be contiguous")
    if fmt in ("mxfp4", "mxfp8") and tuple(scales.shape) != (N, K // 32):
        raise FQLError("scales must be [N, K/32]")
    if fmt == "fp8_block" and (tuple(scales.shape) != (N // 128, K // 128) or scales.dtype != torch.float32):
        raise FQLError("scales must be float32 [N/128, K/128]")
    nbytes = _size_query(f"fql_packed_{fmt}_bytes", N, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    if fmt == "fp8":
        _check(_fn("fql_pack_weight_fp8")(_ptr(codes), N, K, _ptr(out), out.numel(),
                                          _stream(codes.device)))
    else:
        _check(_fn(f"fql_pack_weight_{fmt}")(_ptr(codes), _ptr(scales), N, K, _ptr(out), out.numel(),
                                             _stream(codes.device)))
    return out, N, K


def pack_weight_mxfp4(codes, scales, out=None):
    """Re-lay canonical MXFP4 weight (codes [N, K/2], scales [N, K/32]) for the GEMM."""
    return _pack_sc("mxfp4", codes, scales, out)[0]


def pack_weight_mxfp8(codes, scales, out=None):
    """Re-lay canonical MXFP8 weight (codes [N, K], scales [N, K/32]) for the GEMM."""
    return _pack_sc("mxfp8", codes, scales, out)[0]


def pack_weight_fp8(codes, out=None):
    """Re-lay per-tensor FP8 weight codes [N, K] for the GEMM."""
    return _pack_sc("fp8", codes, None, out)[0]


def pack_weight_fp8_block(codes, scales, out=None):
    """Re-lay block FP8 weight (codes [N, K], float32 scales [N/128, K/128]) for the GEMM."""
    return _pack_sc("fp8_block", codes, scales, out)[0]


class _ScWeight:
    fmt = None

    def __init__(self, packed, N, K):
        self.packed = packed
        self.N, self.K = int(N), int(K)

    def repack_(self, codes, scales=None):
        """Re-pack new canonical weights into the same storage (address kept)."""
        _pack_sc(self.fmt, codes, scales, self.packed)
        return self


class MXFP4Weight(_ScWeight):
    """A packed MXFP4 weight [N, K] (uint8 device buffer from pack_weight_mxfp4)."""
    fmt = "mxfp4"

    @classmethod
    def from_float(cls, w):
        codes, scales = quant_mxfp4_weight(w)
        return cls(pack_weight_mxfp4(codes, scales), w.shape[0], w.shape[1])


class MXFP8Weight(_ScWeight):
    """A packed MXFP8 weight [N, K]."""
    fmt = "mxfp8"

    @classmethod
    def from_float(cls, w):
        codes, scales = quant_mxfp8_weight(w)
        return cls(pack_weight_mxfp8(codes, scales), w.shape[0], w.shape[1])


class FP8BlockWeight(_ScWeight):
    """A packed block-FP8 weight [N, K] (scales of 128 x 128 tiles inside the blob)."""
    fmt = "fp8_block"

    @classmethod
    def from_float(cls, w):
        codes, scales = quant_fp8_block_weight(w)
        return cls(pack_weight_fp8_block(codes, scales), w.shape[0], w.shape[1])


class FP8Weight(_ScWeight):
    """A packed per-tensor FP8 weight [N, K] with its weight scale and the layer's
    static input scale; alpha = fl32(input_scale * weight_scale), also kept as a
    float32 device scalar (alpha_dev) that linear_fp8 reads when no alpha is
    passed, so repack_ with a new weight scale keeps captured graphs valid."""
    fmt = "fp8"

    def __init__(self, packed, N, K, weight_scale, input_scale):
        super().__init__(packed, N, K)
        self.weight_scale = _c_f32(float(weight_scale)).value
        self.input_scale = _c_f32(float(input_scale)).value
        self.alpha = fp8_output_scale(self.input_scale, self.weight_scale)
        self.alpha_dev = torch.full((1,), self.alpha, dtype=torch.float32, device=packed.device)

    def repack_(self, codes, scales=None, weight_scale=None):
        """Re-pack new FP8 weight codes into the same storage; a new weight_scale
        updates alpha and alpha_dev (in stream order)."""
        _pack_sc(self.fmt, codes, scales, self.packed)
        if weight_scale is not None:
            self.weight_scale = _c_f32(float(weight_scale)).value
            self.alpha = fp8_output_scale(self.input_scale, self.weight_scale)
            self.alpha_dev.fill_(self.alpha)
        return self

    @classmethod
    def from_float(cls, w, input_scale, weight_scale=None):
        if weight_scale is None:
            weight_scale = fp8_scale_from_amax(amax(w).item())
        return cls(pack_weight_fp8(quant_fp8_weight(w, weight_scale)), w.shape[0], w.shape[1],
                   weight_scale, input_scale)


def linear_sc_workspace_bytes(fmt, M, N, K):
    return _size_query(f"fql_linear_{_SC[fmt]}_workspace_bytes", M, N, K)


def linear_sc_plan(fmt, M, N, K):
    buf = ctypes.create_string_buffer(256)
    _check(_fn(f"fql_linear_{_SC[fmt]}_describe")(int(M), int(N), int(K), buf, 256))
    return buf.value.decode()


def linear_mxfp4_workspace_bytes(M, N, K):
    return linear_sc_workspace_bytes("mxfp4", M, N, K)


def linear_mxfp4_plan(M, N, K):
    """One-line description of the MXFP4 launch plan for this shape."""
    return linear_sc_plan("mxfp4", M, N, K)


def _linear_sc(fmt, x, weight, alpha, bias, out, workspace):
    _require_cuda(x, "x")
    if x.dtype != torch.bfloat16:
        raise FQLError(f"linear_{fmt} takes bfloat16 activations")
    if weight.fmt != fmt:
        raise FQLError(f"weight is {weight.fmt}, not {fmt}")
    if x.shape[-1] != weight.K:
        raise FQLError(f"x has K={x.shape[-1]}, weight has K={weight.K}")
    x2, ld = _rows_view(x, "x")
    M, K = x2.shape
    N = weight.N
    if bias is not None:
        _require_cuda(bias, "bias")
        if bias.dtype != torch.bfloat16 or bias.numel() != N or not bias.is_contiguous():
            raise FQLError("bias must be a contiguous bf16 tensor of N elements")
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (N,), dtype=torch.bfloat16, device=x.device)
    y2, ldy = _rows_view(out, "out")
    if workspace is None:
        workspace = _workspace(x.device, linear_sc_workspace_bytes(fmt, M, N, K))
    st = _stream(x.device)
    if fmt == "fp8" and alpha is None:
        _check(_fn("fql_linear_fp8_dev_alpha")(_ptr(x2), M, K, ld, weight.input_scale,
                                               _ptr(weight.packed), N, _ptr(weight.alpha_dev),
                                               _ptr(bias), _ptr(y2), ldy, _ptr(workspace),
                                               workspace.numel(), st))
    elif fmt == "fp8":
        _check(_fn("fql_linear_fp8")(_ptr(x2), M, K, ld, weight.input_scale, _ptr(weight.packed), N,
                                     float(alpha), _ptr(bias), _ptr(y2), ldy, _ptr(workspace),
                                     workspace.numel(), st))
    else:
        a = 1.0 if alpha is None else alpha
        _check(_fn(f"fql_linear_{fmt}")(_ptr(x2), M, K, ld, _ptr(weight.packed), N, float(a),
                                        _ptr(bias), _ptr(y2), ldy, _ptr(workspace), workspace.numel(),
                                        st))
    return out


def linear_mxfp4(x, weight, alpha=1.0, bias=None, out=None, workspace=None):
    """y = bf16(alpha * mxfp4(x) @ W^T + bias) for bf16 x [..., K]; returns [..., N]."""
    return _linear_sc("mxfp4", x, weight, alpha, bias, out, workspace)


def linear_mxfp8(x, weight, alpha=1.0, bias=None, out=None, workspace=None):
    """y = bf16(alpha * mxfp8(x) @ W^T + bias)."""
    return _linear_sc("mxfp8", x, weight, alpha, bias, out, workspace)


def linear_fp8(x, weight, alpha=None, bias=None, out=None, workspace=None):
    """y = bf16(alpha * fp8(x; input_scale) @ W_q^T + bias), alpha = input_scale * weight_scale."""
    return _linear_sc("fp8", x, weight, alpha, bias, out, workspace)


def linear_fp8_block(x, weight, alpha=1.0, bias=None, out=None, workspace=None):
    """y = bf16(sum over 128-groups of s_x s_w (x_q @ W_q^T) + bias)."""
    return _linear_sc("fp8_block", x, weight, alpha, bias, out, workspace)


# ---------------------------------------------------------------------------
# warmup
# ---------------------------------------------------------------------------

def token_counts_for_warmup(max_tokens, graph_sizes=()):
    """The row counts M a serving engine warms each layer at: 1 (a decode
    step), every positive graph-capture size, and the largest batch
    (B12X write-up, Implementation: the warmup token set)."""
    return sorted({1, int(max_tokens), *[int(g) for g in graph_sizes if int(g) > 0]})


def warmup(layers, token_counts, device=None):
    """Run every distinct (format, N, K, M) linear call once on zeros.

    `layers` holds packed weights (NVFP4Weight, MXFP4Weight, MXFP8Weight,
    FP8Weight, FP8BlockWeight); layers with the same format and shape are
    warmed once (the B12X write-up dedupes warmup layers by signature). This loads
    the kernels' code objects and leaves the per-stream workspace sized for
    the largest call, so later calls (and graph captures) allocate nothing.
    Returns the number of calls made.
    """
    seen = set()
    calls = 0
    for w in layers:
        fmt = "nvfp4" if isinstance(w, NVFP4Weight) else w.fmt
        for M in token_counts:
            key = (fmt, w.N, w.K, int(M))
            if key in seen:
                continue
            seen.add(key)
            dev = device or w.packed.device
            x = torch.zeros((int(M), w.K), dtype=torch.bfloat16, device=dev)
            fn = {"nvfp4": linear_nvfp4, "mxfp4": linear_mxfp4, "mxfp8": linear_mxfp8,
                  "fp8": linear_fp8, "fp8_block": linear_fp8_block}[fmt]
            fn(x, w)
            calls += 1
    return calls
