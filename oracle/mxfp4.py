"""MXFP4 quantize / dequantize (oracle; test infrastructure only).

"weight precision part 2", "Block scaling": MXFP4 gives each block of 32
values one 8-bit scale that has to be a power of two (4.25 bits per value).
The MoE report ("方法概述", method overview) uses MXFP4 (E2M1, 32 elements
sharing one UE8M0 scale) for the dispatched activations ("BF16ToFP4Row").
"""
import numpy as np

from . import formats as F
from .philox import sr_uniform

BLOCK = 32


def scale_byte(absmax):
    """UE8M0 scale byte of a block.

    [reading] The pages fix only "8-bit, power of two".  The OCP MX shared
    exponent rule is taken [external]: e = floor(log2(absmax)) - 2 (2 is the
    exponent of E2M1's largest value, 6 = 1.5 * 2**2), clamped to
    [-127, 127], stored as e + 127.  absmax == 0 gives byte 0.  floor(log2)
    is read exactly from frexp."""
    a = np.asarray(absmax, dtype=np.float64)
    _, ex = np.frexp(a)                 # a = m * 2**ex, m in [0.5, 1)
    e = ex.astype(np.int64) - 1 - 2
    b = np.clip(e + 127, 0, 254)
    return np.where(a == 0, 0, b).astype(np.uint8)


def quantize(x, rounding="rtn", seed=0, step=0, row_ids=None):
    """x: float32 [R, C], C % 32 == 0 -> (codes [R, C], scale bytes [R, C/32]).

    q = x * 2**-e exactly (float64), then E2M1 RTN (saturating at 6), or
    stochastic rounding with the same (seed, step, global index) stream as
    NVFP4 ("fp4-train", "How it works" describes it for NVFP4; [reading] it
    applies unchanged to the power-of-two scaled value)."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    assert C % BLOCK == 0
    xb = x.reshape(R, C // BLOCK, BLOCK).astype(np.float64)
    sb = scale_byte(np.max(np.abs(xb), axis=-1))
    e = sb.astype(np.int64) - 127
    q = np.ldexp(xb, -e[..., None])
    if rounding == "rtn":
        codes = F.e2m1_rtn(q)
    else:
        rows = np.arange(R, dtype=np.int64) if row_ids is None else np.asarray(row_ids, np.int64)
        index = (rows[:, None] * C + np.arange(C, dtype=np.int64)[None, :]).reshape(R, C // BLOCK, BLOCK)
        codes = F.e2m1_sr(q, sr_uniform(index, seed, step))
    return codes.reshape(R, C), sb


def quantize_packed(x, rounding="rtn", seed=0, step=0, row_ids=None):
    codes, sb = quantize(x, rounding, seed, step, row_ids)
    return F.pack_codes(codes), sb


def dequantize_f32(codes, scale_bytes):
    """y = e2m1(code) * 2**(b-127), as float32 (exact unless it overflows;
    scale byte 0xFF is NaN)."""
    codes = np.asarray(codes)
    R, C = codes.shape
    s = F.e8m0_decode(scale_bytes).reshape(R, C // BLOCK, 1)
    v = F.e2m1_decode(codes).reshape(R, C // BLOCK, BLOCK)
    with np.errstate(over="ignore", invalid="ignore"):
        return (v * s).astype(np.float32).reshape(R, C)


def dequantize(packed, scale_bytes, out="bf16"):
    y = dequantize_f32(F.unpack_codes(packed), scale_bytes)
    return F.f32_to_bf16_bits(y) if out == "bf16" else y
