"""Pins of the oracle's MXFP4 scale rule and rounding -- CPU only."""
import math

import numpy as np

from oracle import formats as F
from oracle import mxfp4


def test_scale_is_power_of_two_and_fits():
    rng = np.random.default_rng(0)
    x = (rng.standard_t(4, size=(64, 256)) * np.exp2(rng.integers(-30, 30, size=(64, 1)))).astype(np.float32)
    codes, sb = mxfp4.quantize(x)
    amax = np.abs(x).reshape(64, 8, 32).max(axis=2)
    scale = F.e8m0_decode(sb)
    q = amax / scale
    assert np.all((q >= 4) & (q < 8))                     # floor(log2 amax) - 2
    # the block maximum lands on the top two grid values
    top = np.abs(F.e2m1_decode(codes)).reshape(64, 8, 32).max(axis=2)
    assert set(np.unique(top)) <= {4.0, 6.0}


def test_exhaustive_bf16_at_several_scales():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = F.bf16_bits_to_f32(bits)
    x = x[np.isfinite(x)]
    for e in (-127, -100, -3, 0, 1, 5, 60, 125):
        # cap |x| below the block maximum, put the maximum first in each block
        xs = x[np.abs(x.astype(np.float64)) < math.ldexp(1, e + 3)]
        pad = (-xs.size) % 31
        xs = np.concatenate([xs, np.zeros(pad, np.float32)]).reshape(-1, 31)
        lead = np.full((xs.shape[0], 1), np.float32(math.ldexp(1.0, e + 2)), np.float32)
        blk = np.concatenate([lead, xs], axis=1).reshape(1, -1)
        codes, sb = mxfp4.quantize(blk)
        assert np.all(sb == max(e + 127, 0))
        flat = blk.reshape(-1)
        q = np.array([math.ldexp(float(v), -e) for v in flat])
        ref_mag = np.select([q == 0], [0], default=0)
        # independent: exact scaled value, nearest with ties to even code
        grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
        aq = np.minimum(np.abs(q), 6)
        d = np.abs(aq[:, None] - grid)
        m = d.min(axis=1, keepdims=True)
        ref_mag = np.where((d == m).sum(axis=1) == 2,
                           np.array([np.flatnonzero(row)[np.flatnonzero(row) % 2 == 0][0]
                                     if row.sum() == 2 else 0 for row in (d == m)]),
                           np.argmin(d, axis=1))
        ref = ref_mag | np.where(np.signbit(flat), 8, 0)
        np.testing.assert_array_equal(codes.reshape(-1), ref)


def test_zero_block_and_subnormal_scale():
    x = np.zeros((1, 64), np.float32)
    x[0, 32] = np.float32(2.0 ** -127)                     # subnormal block maximum
    codes, sb = mxfp4.quantize(x)
    assert sb.tolist() == [[0, 0]]
    assert F.e2m1_decode(codes[0, 32]) == 1.0               # 2**-127 / 2**-127
    assert mxfp4.dequantize_f32(codes, sb)[0, 32] == np.float32(2.0 ** -127)


def test_dequantize_is_exact_on_the_grid():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, size=(16, 64)).astype(np.uint8)
    sb = rng.integers(1, 250, size=(16, 2)).astype(np.uint8)
    y = mxfp4.dequantize_f32(codes, sb)
    ref = F.e2m1_decode(codes) * np.repeat(np.exp2(sb.astype(np.float64) - 127), 32, axis=1)
    np.testing.assert_array_equal(y.astype(np.float64), ref)
    c2, s2 = mxfp4.quantize(y)
    np.testing.assert_array_equal(mxfp4.dequantize_f32(c2, s2), y)


def test_moe_wire_bytes():
    from conftest import read_golden
    sizes = read_golden("format_sizes.txt")
    M, K = 4096, 7168
    p, sb = mxfp4.quantize_packed(np.ones((M // 64, K), np.float32))
    mx_bytes = (p.nbytes + sb.nbytes) * 64
    assert f"{mx_bytes / (M * K):.2f}" == sizes["mxfp4_bytes_per_mk"][0]
    # the fp8 layout the converter emits: 1 byte per value + one fp32 per 128
    fp8_bytes = M * K + 4 * M * K // 128
    assert f"{fp8_bytes / (M * K):.2f}" == sizes["fp8_bytes_per_mk"][0]
    # a one-byte fp8 scale would print 1.01, a 2-byte MX scale 0.56
    assert f"{(M * K + M * K // 128) / (M * K):.2f}" != sizes["fp8_bytes_per_mk"][0]


def test_sr_is_unbiased_at_power_of_two_scale():
    x = np.full((20000, 32), np.float32(2.3 * 4))      # scale 4: q = 2.3
    x[:, 0] = np.float32(6.0 * 4)
    codes, sb = mxfp4.quantize(x, "sr", seed=1, step=2)
    assert np.all(sb == 129)
    v = F.e2m1_decode(codes[:, 1:])
    assert set(np.unique(v)) == {2.0, 3.0}
    assert abs(v.mean() - 2.3) < 4 * np.sqrt(0.21 / v.size)


def test_sr_stream_depends_only_on_the_flat_index():
    """As for NVFP4: the SR draws follow the row-major position of the
    element, so reshaping the tensor's rows does not change a code."""
    rng = np.random.default_rng(22)
    R, C = 6, 128
    x = (rng.standard_normal((R, C)) * 3).astype(np.float32)
    c, s = mxfp4.quantize(x, "sr", seed=5, step=9)
    for shape in ((1, R * C), (R // 2, 2 * C)):
        c2, s2 = mxfp4.quantize(x.reshape(shape), "sr", seed=5, step=9)
        np.testing.assert_array_equal(c2.reshape(R, C), c)
        np.testing.assert_array_equal(s2.reshape(-1), s.reshape(-1))
    assert not np.array_equal(mxfp4.quantize(x, "sr", seed=5, step=10)[0], c)
