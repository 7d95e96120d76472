"""NVFP4 quantize / dequantize / error-feedback qdq (oracle; test
infrastructure only).

Follows "fp4-train": "How it works" (16-element blocks, scale block_absmax/6
encoded to e4m3, each element divided by the decoded scale and rounded to the
e2m1 grid by RTN or by counter-based stochastic rounding; per-element error
feedback residual; two codes per byte) and "Usage" (quantize -> (packed,
scale), dequantize(packed, scale, rows, cols), ErrorFeedback.qdq), and
"weight precision part 2", "Block scaling" (NVFP4: 16-element blocks with an
FP8 scale plus one 32-bit scale for the whole matrix).

All scalar arithmetic is IEEE float32, as a GPU implementation of the pages'
description performs it; numpy float32 operations are correctly rounded.
"""
import numpy as np

from . import formats as F
from .philox import sr_uniform

BLOCK = 16
E4M3_MAX = np.float32(448.0)
E2M1_MAX = np.float32(6.0)


def tensor_scale(v):
    """Per-tensor fp32 scale S_t.

    [reading] "weight precision part 2" only says NVFP4 carries one 32-bit
    scale per matrix.  It is taken as the scale that maps the tensor's
    absmax onto the largest block scale times the largest element:
    S_t = fl32(max|v| / (6 * 448)).  If that is 0 (all-zero tensor or an
    underflowing absmax) S_t = 1."""
    v = np.asarray(v, dtype=np.float32)
    a = np.float32(np.max(np.abs(v))) if v.size else np.float32(0)
    st = np.float32(a / np.float32(E2M1_MAX * E4M3_MAX))
    return np.float32(1.0) if st == 0 else st


def block_scale_codes(absmax, st):
    """Block scale byte: e4m3( fl32( fl32(absmax / 6) / S_t ) ).

    "fp4-train", "How it works": scale = block_absmax / 6, encoded to e4m3.
    [reading] with a per-tensor scale the encoded quantity is that value
    divided by S_t; RNE with saturation at 448 (formats.e4m3_encode)."""
    absmax = np.asarray(absmax, dtype=np.float32)
    r = (absmax / np.float32(6.0)).astype(np.float32)
    with np.errstate(over="ignore"):            # fp32 overflow gives inf, which saturates to 448
        r = (r / np.float32(st)).astype(np.float32)
    return F.e4m3_encode(r)


def decoded_scale(codes, st):
    """s_dec = fl32(e4m3_value * S_t)."""
    return (F.e4m3_decode(codes).astype(np.float32) * np.float32(st)).astype(np.float32)


def _codes_from_q(x, s_dec, rounding, seed, step, index):
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = (x / s_dec).astype(np.float32)          # correctly rounded fp32 division
    zero_scale = s_dec == 0
    q = np.where(zero_scale, np.copysign(np.float32(0), x), q)  # [reading] code = sign only
    if rounding == "rtn":
        return F.e2m1_rtn(q)
    u = sr_uniform(index, seed, step)
    return F.e2m1_sr(q, u)


def global_index(R, C, row_ids=None):
    """Global row-major element index of an [R, C] tile whose rows are rows
    `row_ids` (default 0..R-1) of a tensor with C columns ("fp4-train",
    "How it works": the SR stream is keyed by the global index)."""
    rows = np.arange(R, dtype=np.int64) if row_ids is None else np.asarray(row_ids, np.int64)
    return rows[:, None] * C + np.arange(C, dtype=np.int64)[None, :]


def quantize(x, st, rounding="rtn", seed=0, step=0, row_ids=None):
    """x: float32 [R, C] (C % 16 == 0); st: the tensor scale S_t.

    Returns (codes uint8 [R, C], scale bytes uint8 [R, C/16]).  SR draws
    u from Philox keyed by (seed, step, global row-major index); row_ids
    names the tensor rows that x holds when it is a sample of them."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    assert C % BLOCK == 0
    xb = x.reshape(R, C // BLOCK, BLOCK)
    absmax = np.max(np.abs(xb), axis=-1)
    sc = block_scale_codes(absmax, st)
    s_dec = decoded_scale(sc, st)[..., None]
    index = global_index(R, C, row_ids).reshape(R, C // BLOCK, BLOCK)
    codes = _codes_from_q(xb, s_dec, rounding, seed, step, index)
    return codes.reshape(R, C), sc


def dequantize_f32(codes, scale_bytes, st):
    """y = fl32(e2m1(code) * s_dec), float32 [R, C]."""
    codes = np.asarray(codes)
    R, C = codes.shape
    s_dec = decoded_scale(scale_bytes, st).reshape(R, C // BLOCK, 1)
    v = F.e2m1_decode(codes).astype(np.float32).reshape(R, C // BLOCK, BLOCK)
    with np.errstate(invalid="ignore", over="ignore"):
        return (v * s_dec).astype(np.float32).reshape(R, C)


def dequantize(packed, scale_bytes, st, out="bf16"):
    """Receiver: unpack, rescale; bf16 output is RNE of the fp32 product."""
    y = dequantize_f32(F.unpack_codes(packed), scale_bytes, st)
    return F.f32_to_bf16_bits(y) if out == "bf16" else y


def quantize_packed(x, st, rounding="rtn", seed=0, step=0, row_ids=None):
    codes, sc = quantize(x, st, rounding, seed, step, row_ids)
    return F.pack_codes(codes), sc


def errfeedback_qdq(x, r, st=None, rounding="sr", seed=0, step=0, out="bf16", row_ids=None):
    """One error-feedback quantize-dequantize step.

    "fp4-train", "How it works" and "Usage": the per-element residual
    x - dequant(quantize(x)) is carried and added into the next
    quantization.  Steps: v = fl32(x + r); S_t from max|v| unless given;
    quantize v (RTN or SR); y = fl32(e2m1 * s_dec); out = y in the output
    dtype (bf16 RNE); [reading] r_new = fl32(v - out), the residual against
    the value actually returned.  r = None means a plain qdq with no
    residual.  Returns (out, r_new, packed, scale_bytes, S_t)."""
    x = np.asarray(x, dtype=np.float32)
    v = x if r is None else (x + np.asarray(r, dtype=np.float32)).astype(np.float32)
    if st is None:
        st = tensor_scale(v)
    codes, sc = quantize(v, st, rounding, seed, step, row_ids)
    y = dequantize_f32(codes, sc, st)
    if out == "bf16":
        ob = F.f32_to_bf16_bits(y)
        of = F.bf16_bits_to_f32(ob)
    else:
        ob = y
        of = y
    r_new = None if r is None else (v - of).astype(np.float32)
    return ob, r_new, F.pack_codes(codes), sc, np.float32(st)
