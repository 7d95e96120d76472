"""Python binding of libfp4mi.so, the gfx950 block-scaled FP4 codec.

Argument marshalling only: every step of the codec runs in the library's
HIP kernels.  Tensors are torch tensors on the GPU (PyTorch supplies device
memory and the current stream); outputs that are not passed in are
allocated with torch.empty.  A non-zero status from the library raises
Fp4Error.  If the shared library has not been built this module raises at
import: there is no CPU fallback.

Entry points (same names as the C ABI in include/fp4mi.h):
  fp4_quantize, fp4_dequantize, fp4quant_encode, fp4quant_decode,
  fp4_errfeedback_qdq, mxfp4_row_to_fp8_col, mxfp4_row_to_fp8_col_tokblk,
  mxfp4_row_to_fp8_row
plus ErrorFeedback, a name-keyed holder of residual buffers in the style of
the fp4-train page's ErrorFeedback.qdq(name, x, step).
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4mi.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python __graft_entry__.py` or `python block_scaled_fp4_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

# ---- constants (mirror include/fp4mi.h)
FP4_OK, FP4_EINVAL, FP4_ESHAPE, FP4_EALIGN, FP4_EDTYPE, FP4_EHIP, FP4_EOVERLAP = range(7)
DTYPE = {torch.float32: 0, torch.bfloat16: 1}
FMT = {"nvfp4": 0, "mxfp4": 1}
ROUND = {"rtn": 0, "sr": 1}
TSCALE = {"compute": 0, "given": 1}

_p, _i, _i32, _i64, _u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
_SIGS = {
    "fp4_quantize": [_p, _i, _i64, _i64, _i, _i, _u64, _u64, _i, _p, _p, _p, _p],
    "fp4_dequantize": [_p, _p, _p, _i64, _i64, _i, _p, _i, _p],
    "fp4quant_encode": [_p, _i, _i64, _i64, _i32, _p, _p, _p, _p],
    "fp4quant_encode_ex": [_p, _i, _i64, _i64, _i32, _i, _u64, _u64, _p, _p, _p, _p],
    "fp4quant_decode": [_p, _p, _p, _i64, _i64, _i32, _p, _i, _p],
    "fp4_errfeedback_qdq": [_p, _i, _i64, _i64, _p, _p, _i, _i, _u64, _u64, _i, _p, _p, _p, _p],
    "mxfp4_row_to_fp8_col": [_p, _p, _p, _i32, _i64, _i64, _p, _p, _p],
    "mxfp4_row_to_fp8_col_tokblk": [_p, _p, _p, _i32, _i64, _i64, _p, _p, _p],
    "mxfp4_row_to_fp8_row": [_p, _p, _i64, _i64, _p, _p, _p],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int
_lib.fp4_status_string.argtypes = [ctypes.c_int]
_lib.fp4_status_string.restype = ctypes.c_char_p
_lib.fp4_abi_version.argtypes = []
_lib.fp4_abi_version.restype = ctypes.c_int


class Fp4Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {_lib.fp4_status_string(status).decode()} (status {status})")


def raw():
    """The ctypes handle of the library (for ABI-level tests)."""
    return _lib


def status_string(status):
    return _lib.fp4_status_string(status).decode()


def abi_version():
    return _lib.fp4_abi_version()


def _check(fn, status):
    if status != FP4_OK:
        raise Fp4Error(fn, status)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _dtype_code(dt):
    return DTYPE.get(dt, 99)


def _dev(x):
    if not x.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not x.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return x


def _arg(t, name, dtype, numel, device, optional=False):
    """Checks a tensor argument the C ABI only sees as a pointer: same GPU as
    the main input, contiguous, of `dtype`, with at least `numel` elements
    (the library writes or reads exactly that many)."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} are needed")
    return t


def fp4_quantize(x, fmt="nvfp4", rounding="rtn", seed=0, step=0, tscale="compute",
                 tensor_scale=None, packed=None, scales=None, stream=None):
    """Quantize x [.., cols] -> (packed uint8 [rows, cols/2], scales uint8, tensor_scale).
    tensor_scale is a 1-element fp32 device tensor (NVFP4; None for MXFP4)."""
    _dev(x)
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    blk = 32 if fmt == "mxfp4" else 16
    if packed is None:
        packed = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // blk), dtype=torch.uint8, device=x.device)
    if fmt == "nvfp4" and tensor_scale is None:
        tensor_scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _arg(packed, "packed", torch.uint8, rows * cols // 2, x.device)
    _arg(scales, "scales", torch.uint8, rows * cols // blk, x.device)
    _arg(tensor_scale, "tensor_scale", torch.float32, 1, x.device, optional=fmt == "mxfp4")
    _check("fp4_quantize", _lib.fp4_quantize(
        _ptr(x), _dtype_code(x.dtype), rows, cols, FMT[fmt], ROUND[rounding], seed, step,
        TSCALE[tscale], _ptr(tensor_scale), _ptr(packed), _ptr(scales), _stream(stream)))
    return packed, scales, tensor_scale


def fp4_dequantize(packed, scales, rows, cols, fmt="nvfp4", tensor_scale=None,
                   out_dtype=torch.bfloat16, y=None, stream=None):
    """Receiver: (packed, scales[, tensor_scale]) -> y [rows, cols] in out_dtype."""
    _dev(packed)
    if y is None:
        y = torch.empty((rows, cols), dtype=out_dtype, device=packed.device)
    blk = 32 if fmt == "mxfp4" else 16
    _arg(packed, "packed", torch.uint8, rows * cols // 2, packed.device)
    _arg(scales, "scales", torch.uint8, rows * cols // blk, packed.device)
    _arg(tensor_scale, "tensor_scale", torch.float32, 1, packed.device, optional=fmt == "mxfp4")
    _arg(y, "y", y.dtype, rows * cols, packed.device)
    _check("fp4_dequantize", _lib.fp4_dequantize(
        _ptr(packed), _ptr(scales), _ptr(tensor_scale), rows, cols, FMT[fmt], _ptr(y),
        _dtype_code(y.dtype), _stream(stream)))
    return y


def fp4quant_encode(x, group, packed=None, s_rms=None, s_abs=None, stream=None):
    """FP4Quant encode -> (packed [rows, cols/2], s_rms [rows, cols/G], s_abs [rows, cols/G])."""
    return _fq_encode("fp4quant_encode", x, group, None, 0, 0, packed, s_rms, s_abs, stream)


def fp4quant_encode_ex(x, group, rounding="sr", seed=0, step=0, packed=None, s_rms=None, s_abs=None,
                       stream=None):
    """FP4Quant encode with RTN or stochastic rounding keyed by (seed, step,
    element index) -> (packed, s_rms, s_abs) as fp4quant_encode."""
    return _fq_encode("fp4quant_encode_ex", x, group, rounding, seed, step, packed, s_rms, s_abs,
                      stream)


def _fq_encode(fn, x, group, rounding, seed, step, packed, s_rms, s_abs, stream):
    _dev(x)
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    if packed is None:
        packed = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    ng = cols // group if group > 0 else 0
    if s_rms is None:
        s_rms = torch.empty((rows, ng), dtype=torch.float32, device=x.device)
    if s_abs is None:
        s_abs = torch.empty((rows, ng), dtype=torch.float32, device=x.device)
    _arg(packed, "packed", torch.uint8, rows * cols // 2, x.device)
    _arg(s_rms, "s_rms", torch.float32, rows * ng, x.device)
    _arg(s_abs, "s_abs", torch.float32, rows * ng, x.device)
    if rounding is None:
        status = _lib.fp4quant_encode(_ptr(x), _dtype_code(x.dtype), rows, cols, group, _ptr(packed),
                                      _ptr(s_rms), _ptr(s_abs), _stream(stream))
    else:
        status = _lib.fp4quant_encode_ex(_ptr(x), _dtype_code(x.dtype), rows, cols, group,
                                         ROUND.get(rounding, 99), seed, step, _ptr(packed), _ptr(s_rms),
                                         _ptr(s_abs), _stream(stream))
    _check(fn, status)
    return packed, s_rms, s_abs


def fp4quant_decode(packed, s_rms, s_abs, rows, cols, group, out_dtype=torch.bfloat16, y=None,
                    stream=None):
    """FP4Quant receiver -> y [rows, cols]."""
    _dev(packed)
    if y is None:
        y = torch.empty((rows, cols), dtype=out_dtype, device=packed.device)
    ng = cols // group if group > 0 else 0
    _arg(packed, "packed", torch.uint8, rows * cols // 2, packed.device)
    _arg(s_rms, "s_rms", torch.float32, rows * ng, packed.device)
    _arg(s_abs, "s_abs", torch.float32, rows * ng, packed.device)
    _arg(y, "y", y.dtype, rows * cols, packed.device)
    _check("fp4quant_decode", _lib.fp4quant_decode(
        _ptr(packed), _ptr(s_rms), _ptr(s_abs), rows, cols, group, _ptr(y), _dtype_code(y.dtype),
        _stream(stream)))
    return y


def fp4_errfeedback_qdq(x, residual=None, y=None, out_dtype=None, rounding="sr", seed=0, step=0,
                        tscale="compute", tensor_scale=None, packed=None, scales=None,
                        stream=None):
    """NVFP4 qdq with an fp32 error-feedback residual (updated in place).
    Returns (y, tensor_scale).  y may be x for an in-place update."""
    _dev(x)
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    if y is None:
        y = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    if tensor_scale is None:
        tensor_scale = torch.empty(1, dtype=torch.float32, device=x.device)
    n = rows * cols
    _arg(residual, "residual", torch.float32, n, x.device, optional=True)
    _arg(y, "y", y.dtype, n, x.device)
    _arg(tensor_scale, "tensor_scale", torch.float32, 1, x.device)
    _arg(packed, "packed", torch.uint8, n // 2, x.device, optional=True)
    _arg(scales, "scales", torch.uint8, n // 16, x.device, optional=True)
    _check("fp4_errfeedback_qdq", _lib.fp4_errfeedback_qdq(
        _ptr(x), _dtype_code(x.dtype), rows, cols, _ptr(residual), _ptr(y), _dtype_code(y.dtype),
        ROUND[rounding], seed, step, TSCALE[tscale], _ptr(tensor_scale), _ptr(packed),
        _ptr(scales), _stream(stream)))
    return y, tensor_scale


def mxfp4_row_to_fp8_col(packed, scales_e8m0, token_offsets, hidden, fp8_out=None,
                         fp8_scales=None, stream=None):
    """Ragged MXFP4 rows [T, H/2] (+ UE8M0 [T, H/32]) -> per-expert FP8 E4M3
    columns (flat uint8 [T*H]) and fp32 block scales (flat [T*H/128])."""
    _dev(packed)
    T = packed.shape[0]
    E = token_offsets.numel() - 1
    if fp8_out is None:
        fp8_out = torch.empty(T * hidden, dtype=torch.uint8, device=packed.device)
    if fp8_scales is None:
        fp8_scales = torch.empty(T * hidden // 128, dtype=torch.float32, device=packed.device)
    _arg(packed, "packed", torch.uint8, T * hidden // 2, packed.device)
    _arg(scales_e8m0, "scales_e8m0", torch.uint8, T * hidden // 32, packed.device)
    _arg(token_offsets, "token_offsets", torch.int64, 1, packed.device)
    _arg(fp8_out, "fp8_out", torch.uint8, T * hidden, packed.device)
    _arg(fp8_scales, "fp8_scales", torch.float32, T * hidden // 128, packed.device)
    _check("mxfp4_row_to_fp8_col", _lib.mxfp4_row_to_fp8_col(
        _ptr(packed), _ptr(scales_e8m0), _ptr(token_offsets), E, T, hidden, _ptr(fp8_out),
        _ptr(fp8_scales), _stream(stream)))
    return fp8_out, fp8_scales


def tokblk_scale_count(total_tokens, num_experts, hidden):
    """fp32 elements of the token-block scale buffer: H (ceil(T / 128) + E)."""
    return hidden * ((total_tokens + 127) // 128 + num_experts)


def mxfp4_row_to_fp8_col_tokblk(packed, scales_e8m0, token_offsets, hidden, fp8_out=None,
                                fp8_scales=None, stream=None):
    """Ragged MXFP4 rows [T, H/2] (+ UE8M0 [T, H/32]) -> per-expert FP8 E4M3
    columns (flat uint8 [T*H]) with FP8 blocks of 128 tokens per channel, and
    fp32 scales (flat [H (ceil(T/128) + E)]; expert e's [H, ceil(n_e/128)]
    matrix at element H (ceil(off_e/128) + e))."""
    _dev(packed)
    T = packed.shape[0]
    E = token_offsets.numel() - 1
    nsc = tokblk_scale_count(T, E, hidden)
    if fp8_out is None:
        fp8_out = torch.empty(T * hidden, dtype=torch.uint8, device=packed.device)
    if fp8_scales is None:
        fp8_scales = torch.empty(nsc, dtype=torch.float32, device=packed.device)
    _arg(packed, "packed", torch.uint8, T * hidden // 2, packed.device)
    _arg(scales_e8m0, "scales_e8m0", torch.uint8, T * hidden // 32, packed.device)
    _arg(token_offsets, "token_offsets", torch.int64, 1, packed.device)
    _arg(fp8_out, "fp8_out", torch.uint8, T * hidden, packed.device)
    _arg(fp8_scales, "fp8_scales", torch.float32, nsc, packed.device)
    _check("mxfp4_row_to_fp8_col_tokblk", _lib.mxfp4_row_to_fp8_col_tokblk(
        _ptr(packed), _ptr(scales_e8m0), _ptr(token_offsets), E, T, hidden, _ptr(fp8_out),
        _ptr(fp8_scales), _stream(stream)))
    return fp8_out, fp8_scales


def mxfp4_row_to_fp8_row(packed, scales_e8m0, hidden, fp8_out=None, fp8_scales=None,
                         stream=None):
    """MXFP4 rows [T, H/2] (+ UE8M0 [T, H/32]) -> FP8 E4M3 rows [T, H] and
    fp32 block scales [T, H/128] (no transpose)."""
    _dev(packed)
    T = packed.shape[0]
    if fp8_out is None:
        fp8_out = torch.empty((T, hidden), dtype=torch.uint8, device=packed.device)
    if fp8_scales is None:
        fp8_scales = torch.empty((T, hidden // 128), dtype=torch.float32, device=packed.device)
    _arg(packed, "packed", torch.uint8, T * hidden // 2, packed.device)
    _arg(scales_e8m0, "scales_e8m0", torch.uint8, T * hidden // 32, packed.device)
    _arg(fp8_out, "fp8_out", torch.uint8, T * hidden, packed.device)
    _arg(fp8_scales, "fp8_scales", torch.float32, T * hidden // 128, packed.device)
    _check("mxfp4_row_to_fp8_row", _lib.mxfp4_row_to_fp8_row(
        _ptr(packed), _ptr(scales_e8m0), T, hidden, _ptr(fp8_out), _ptr(fp8_scales),
        _stream(stream)))
    return fp8_out, fp8_scales


class ErrorFeedback:
    """Residual holder keyed by tensor name (fp4-train, "Usage").

    qdq(name, x, step) runs fp4_errfeedback_qdq with the residual kept for
    `name` (created as zeros on first use) and returns the new bf16/fp32
    tensor in x's dtype."""

    def __init__(self, stochastic=False, seed=0):
        self.rounding = "sr" if stochastic else "rtn"
        self.seed = seed
        self.residuals = {}

    def qdq(self, name, x, step, out=None):
        r = self.residuals.get(name)
        if r is None or r.shape != x.shape:
            r = torch.zeros(x.shape, dtype=torch.float32, device=x.device)
            self.residuals[name] = r
        y, _ = fp4_errfeedback_qdq(x, residual=r, y=out, rounding=self.rounding, seed=self.seed,
                                   step=step)
        return y
