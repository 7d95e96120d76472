"""GPU parity of fp4_quantize / fp4_dequantize against the oracle
(bit-exact codes, scales, tensor scale and dequantized values)."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import Guarded, dev_bf16, dev_f32, host, host_bf16, need_gpu
from oracle import formats as F
from oracle import mxfp4, nvfp4

pytestmark = pytest.mark.gpu


def run_quant(m, x_dev, fmt, rounding="rtn", seed=0, step=0, tscale="compute", ts=None):
    rows, cols = x_dev.shape
    blk = 32 if fmt == "mxfp4" else 16
    gp = Guarded(rows * cols // 2)
    gs = Guarded(rows * cols // blk)
    if fmt == "nvfp4" and ts is None:
        ts = torch.empty(1, dtype=torch.float32, device="cuda")
    p, s, ts = m.fp4_quantize(x_dev, fmt, rounding, seed, step, tscale, ts,
                              gp.view(torch.uint8, (rows, cols // 2)),
                              gs.view(torch.uint8, (rows, cols // blk)))
    torch.cuda.synchronize()
    gp.check()
    gs.check()
    return host(p), host(s), (None if ts is None else host(ts)[0])


def run_dequant(m, p, s, rows, cols, fmt, ts=None, out=torch.bfloat16):
    es = 2 if out == torch.bfloat16 else 4
    gy = Guarded(rows * cols * es)
    y = m.fp4_dequantize(torch.from_numpy(p).cuda(), torch.from_numpy(s).cuda(), rows, cols, fmt,
                         None if ts is None else dev_f32(np.array([ts])), out,
                         gy.view(out, (rows, cols)))
    torch.cuda.synchronize()
    gy.check()
    return host_bf16(y) if out == torch.bfloat16 else host(y)


def assert_same_f32(a, b):
    a = np.asarray(a, np.float32).view(np.uint32)
    b = np.asarray(b, np.float32).view(np.uint32)
    nan_a = (a & 0x7FFFFFFF) > 0x7F800000
    nan_b = (b & 0x7FFFFFFF) > 0x7F800000
    np.testing.assert_array_equal(nan_a, nan_b)
    np.testing.assert_array_equal(a[~nan_a], b[~nan_b])


# ------------------------------------------------------------- NVFP4
def test_nvfp4_rtn_roundtrip_weight_block():
    """256 x 2048 bf16 weight block with outliers, NVFP4 RTN, computed S_t."""
    m = need_gpu()
    xb = synth.weight_block()
    x = F.bf16_bits_to_f32(xb)
    p, s, ts = run_quant(m, dev_bf16(xb), "nvfp4")
    st = nvfp4.tensor_scale(x)
    rp, rs = nvfp4.quantize_packed(x, st)
    assert np.float32(ts) == st
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(p, rp)
    y = run_dequant(m, p, s, *x.shape, "nvfp4", ts)
    np.testing.assert_array_equal(y, nvfp4.dequantize(rp, rs, st, "bf16"))
    y32 = run_dequant(m, p, s, *x.shape, "nvfp4", ts, torch.float32)
    assert_same_f32(y32, nvfp4.dequantize(rp, rs, st, "f32"))


@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (37, 176), (129, 1040)])
@pytest.mark.parametrize("rounding", ["rtn", "sr"])
def test_nvfp4_fp32_ragged_shapes(rows, cols, rounding):
    m = need_gpu()
    rng = np.random.default_rng(rows * 1000 + cols)
    x = (rng.standard_t(3, size=(rows, cols)) * np.exp2(rng.integers(-20, 20, size=(rows, 1)))).astype(np.float32)
    x[rng.random(x.shape) < 0.05] = 0.0
    x[rng.random(x.shape) < 0.02] *= -0.0
    p, s, ts = run_quant(m, dev_f32(x), "nvfp4", rounding, seed=123456789012345, step=77)
    st = nvfp4.tensor_scale(x)
    assert np.float32(ts) == st
    rp, rs = nvfp4.quantize_packed(x, st, rounding, seed=123456789012345, step=77)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(p, rp)


def test_nvfp4_given_scale_exhaustive_bf16():
    """Every finite bf16 pattern, in blocks anchored so the block scale is one
    of several E4M3 values, with a given S_t: exercises division + rounding."""
    m = need_gpu()
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = F.bf16_bits_to_f32(bits)
    x = x[np.isfinite(x)]
    for st, amax in [(1.0, 6.0), (1.0, 5.5), (0.37, 1.9), (2.0 ** -20, 3e-5), (1e4, 7.7e5)]:
        sel = x[np.abs(x.astype(np.float64)) <= amax]
        pad = (-sel.size) % 15
        sel = np.concatenate([sel, np.zeros(pad, np.float32)]).reshape(-1, 15)
        blk = np.concatenate([np.full((sel.shape[0], 1), amax, np.float32), sel], axis=1)
        blk = blk.reshape(-1, 1024) if blk.size % 1024 == 0 else blk.reshape(1, -1)
        ts = dev_f32(np.array([st], np.float32))
        p, s, _ = run_quant(m, dev_f32(blk), "nvfp4", tscale="given", ts=ts)
        rp, rs = nvfp4.quantize_packed(blk, np.float32(st))
        np.testing.assert_array_equal(s, rs)
        np.testing.assert_array_equal(p, rp)


def test_nvfp4_unit_scale_fp32_threshold_neighbourhood():
    """With block absmax 6 and S_t = 1, q = x: fp32 values a few ulp around
    every rounding threshold, both signs, RTN and SR."""
    m = need_gpu()
    vals = []
    for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0, 2.0, 4.0):
        v = np.float32(t)
        for k in range(-6, 7):
            w = v
            for _ in range(abs(k)):
                w = np.nextafter(w, np.float32(np.inf if k > 0 else -np.inf))
            vals += [w, -w]
    vals += [np.float32(1e-45), np.float32(-1e-38), np.float32(5.999999)]
    v = np.array(vals, np.float32)
    v = np.concatenate([v, np.zeros((-v.size) % 15, np.float32)]).reshape(-1, 15)
    x = np.concatenate([np.full((v.shape[0], 1), 6.0, np.float32), v], axis=1).reshape(1, -1)
    ts = dev_f32(np.array([1.0], np.float32))
    for rounding in ("rtn", "sr"):
        for step in range(4):
            p, s, _ = run_quant(m, dev_f32(x), "nvfp4", rounding, seed=3, step=step, tscale="given", ts=ts)
            rp, rs = nvfp4.quantize_packed(x, np.float32(1.0), rounding, seed=3, step=step)
            np.testing.assert_array_equal(p, rp)
            np.testing.assert_array_equal(s, rs)


def test_nvfp4_bf16_input_exact_and_ambiguous_quotients():
    """bf16 input (the octets the exact redo reloads as bf16): values at and
    next to every threshold and grid point, both signs, in blocks of absmax 6,
    under given tensor scales that make x / s_dec an exact tie (S_t = 1), a
    quotient 2^-20 off a threshold (S_t = 1 + 2^-20: ambiguous for the
    reciprocal bracket, not exact), and a subnormal S_t (no fast scale)."""
    m = need_gpu()
    vals = []
    for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0):
        b = int(F.f32_to_bf16_bits(np.array([t], np.float32))[0])
        for k in range(-2, 3):
            vals += [b + k, (b + k) | 0x8000]
    v = F.bf16_bits_to_f32(np.array(vals, np.uint16))
    v = np.concatenate([v, np.zeros((-v.size) % 15, np.float32)]).reshape(-1, 15)
    blk = np.concatenate([np.full((v.shape[0], 1), 6.0, np.float32), v], axis=1)
    blk = np.concatenate([blk] * 4, axis=0).reshape(4, -1)
    bits = F.f32_to_bf16_bits(blk)
    assert np.array_equal(F.bf16_bits_to_f32(bits), blk)          # exactly representable
    for st in (np.float32(1.0), np.float32(1.0 + 2.0 ** -20), np.float32(2.0 ** -140),
               np.float32(0.37)):
        ts = dev_f32(np.array([st], np.float32))
        p, s, _ = run_quant(m, dev_bf16(bits), "nvfp4", tscale="given", ts=ts)
        rp, rs = nvfp4.quantize_packed(blk, st)
        np.testing.assert_array_equal(s, rs)
        np.testing.assert_array_equal(p, rp)


def test_nvfp4_exact_ties_with_computed_scale():
    """Elements that share the significand of the tensor's absmax A have
    x / s_dec = 2688 * 2^k / e4m3 in exact arithmetic, a rounding threshold
    for several scale bytes: fp32 rounding of S_t and s_dec decides their
    codes.  A third of the elements are such values (both signs, many k)."""
    m = need_gpu()
    rng = np.random.default_rng(21)
    R, C = 96, 4096
    x = (rng.standard_normal((R, C)) * 0.02).astype(np.float32)
    for A in (3.984375, 1.0, 0.0234375, 96.0):
        xx = x.copy()
        xx[0, 0] = A
        sel = rng.random((R, C)) < 0.33
        k = rng.integers(0, 13, size=(R, C))
        xx[sel] = (np.float32(A) * np.exp2(-k[sel]) * rng.choice([-1, 1], size=sel.sum())).astype(np.float32)
        xb = synth.to_bf16_bits(xx)
        xv = F.bf16_bits_to_f32(xb)
        p, s, ts = run_quant(m, dev_bf16(xb), "nvfp4")
        st = nvfp4.tensor_scale(xv)
        assert np.float32(ts) == st
        rp, rs = nvfp4.quantize_packed(xv, st)
        np.testing.assert_array_equal(s, rs)
        np.testing.assert_array_equal(p, rp)


def test_nvfp4_tiny_absmax_and_extreme_scales():
    """Blocks whose absmax / 6 is subnormal at a normal S_t (the E4M3 byte
    then depends on fp32 underflow rounding), S_t outside [2^-100, 2^100],
    and blocks whose scale saturates so far that element quotients reach
    2^105: the IEEE-division paths and the saturating codes."""
    m = need_gpu()
    rng = np.random.default_rng(22)
    # absmax = (49152 + j) * 2^-149 with S_t = 2^-126: r sits at the 0 / 2^-9 boundary
    blk = np.zeros((64, 16), np.float32)
    blk[:, 0] = (np.arange(49140, 49204, dtype=np.uint32)).view(np.float32)
    blk[:, 1:] = (rng.integers(0, 1 << 16, size=(64, 15)).astype(np.uint32)).view(np.float32)
    cases = [(blk.reshape(4, -1), 2.0 ** -126)]
    x = (rng.standard_t(3, size=(8, 512)) * np.exp2(rng.integers(-30, 30, size=(8, 1)))).astype(np.float32)
    cases += [(x, 2.0 ** -110), (x, 2.0 ** 105), (x, 2.0 ** -100), (x * np.float32(2.0 ** 14), 2.0 ** -100),
              (x * np.float32(2.0 ** 40), 2.0 ** -100)]
    for xx, st in cases:
        st = np.float32(st)
        ts = dev_f32(np.array([st], np.float32))
        p, s, _ = run_quant(m, dev_f32(xx), "nvfp4", tscale="given", ts=ts)
        rp, rs = nvfp4.quantize_packed(xx, st)
        np.testing.assert_array_equal(s, rs)
        np.testing.assert_array_equal(p, rp)


def test_nvfp4_dequantize_foreign_scale_bytes():
    """Dequantize accepts any E4M3 byte (signed, subnormal, NaN) and code."""
    m = need_gpu()
    rng = np.random.default_rng(5)
    rows, cols = 64, 256
    p = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    s = rng.integers(0, 256, size=(rows, cols // 16), dtype=np.uint8)
    for st in (1.0, 3.3e-3, 7.5e30):
        for out in (torch.bfloat16, torch.float32):
            y = run_dequant(m, p, s, rows, cols, "nvfp4", st, out)
            ref = nvfp4.dequantize(p, s, np.float32(st), "bf16" if out == torch.bfloat16 else "f32")
            if out == torch.bfloat16:
                nan = np.isnan(F.bf16_bits_to_f32(ref))
                np.testing.assert_array_equal(np.isnan(F.bf16_bits_to_f32(y)), nan)
                np.testing.assert_array_equal(y[~nan], ref[~nan])
            else:
                assert_same_f32(y, ref)


@pytest.mark.parametrize("rows,cols,dtype",
                         [(1, 32, "f32"), (5, 96, "bf16"), (33, 2080, "f32"), (200, 7168, "bf16")])
@pytest.mark.parametrize("rounding", ["rtn", "sr"])
def test_mxfp4_full_compare(rows, cols, dtype, rounding):
    m = need_gpu()
    rng = np.random.default_rng(rows + cols)
    x = (rng.standard_t(4, size=(rows, cols)) * 0.5 * np.exp2(rng.integers(-60, 60, size=(rows, 1)))).astype(np.float32)
    x[rng.random(x.shape) < 0.03] = 0.0
    if dtype == "bf16":
        xb = synth.to_bf16_bits(x)
        x = F.bf16_bits_to_f32(xb)
        xd = dev_bf16(xb)
    else:
        xd = dev_f32(x)
    p, s, _ = run_quant(m, xd, "mxfp4", rounding, seed=2 ** 63 + 5, step=2 ** 40 + 1)
    rp, rs = mxfp4.quantize_packed(x, rounding, seed=2 ** 63 + 5, step=2 ** 40 + 1)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(p, rp)
    for out in (torch.bfloat16, torch.float32):
        y = run_dequant(m, p, s, rows, cols, "mxfp4", None, out)
        ref = mxfp4.dequantize(rp, rs, "bf16" if out == torch.bfloat16 else "f32")
        np.testing.assert_array_equal(y, ref)


def test_mxfp4_exhaustive_bf16_all_scales():
    """Every finite bf16 value, in blocks whose maximum fixes the scale
    exponent e, for e across the whole UE8M0 range."""
    m = need_gpu()
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    xall = F.bf16_bits_to_f32(bits)
    xall = xall[np.isfinite(xall)]
    for e in list(range(-127, 126, 9)) + [125, -126, -125, 0, 1, 2]:
        xs = xall[np.abs(xall.astype(np.float64)) < math.ldexp(1, e + 3)]
        pad = (-xs.size) % 31
        xs = np.concatenate([xs, np.zeros(pad, np.float32)]).reshape(-1, 31)
        lead = np.full((xs.shape[0], 1), np.float32(math.ldexp(1.0, e + 2)), np.float32)
        blk = np.concatenate([lead, xs], axis=1).reshape(1, -1)
        xb = synth.to_bf16_bits(blk)
        for rounding in ("rtn", "sr"):
            p, s, _ = run_quant(m, dev_bf16(xb), "mxfp4", rounding, seed=11, step=e + 200)
            rp, rs = mxfp4.quantize_packed(F.bf16_bits_to_f32(xb), rounding, seed=11, step=e + 200)
            np.testing.assert_array_equal(s, rs)
            np.testing.assert_array_equal(p, rp)


def test_mxfp4_dequantize_every_scale_byte():
    m = need_gpu()
    rows, cols = 256, 512
    codes = np.tile(np.arange(16, dtype=np.uint8), (rows, cols // 16))
    p = F.pack_codes(codes)
    s = np.tile(np.arange(256, dtype=np.uint8), (rows * cols // 32) // 256).reshape(rows, cols // 32)
    for out, tag in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        y = run_dequant(m, p, s, rows, cols, "mxfp4", None, out)
        ref = mxfp4.dequantize(p, s, tag)
        if tag == "f32":
            assert_same_f32(y, ref)
        else:
            nan = np.isnan(F.bf16_bits_to_f32(ref))
            np.testing.assert_array_equal(np.isnan(F.bf16_bits_to_f32(y)), nan)
            np.testing.assert_array_equal(y[~nan], ref[~nan])


def test_empty_tensors_are_noops():
    m = need_gpu()
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    p, s, ts = m.fp4_quantize(x, "mxfp4")
    assert p.numel() == 0 and s.numel() == 0
    y = m.fp4_dequantize(p, s, 0, 64, "mxfp4")
    assert y.numel() == 0


@pytest.mark.parametrize("step", [0, 5])
def test_nvfp4_sr_bf16_every_pattern_given_scales(step):
    """Stochastic rounding of bf16 input (division-free element quotients,
    with the IEEE division for elements or quotients below 2^-100): every
    finite bf16 pattern in blocks anchored to several block scales,
    including quotients far below 2^-100 and S_t outside [2^-100, 2^100]."""
    m = need_gpu()
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = F.bf16_bits_to_f32(bits)
    keep = np.isfinite(x)
    bits, x = bits[keep], x[keep]
    for st, amax in [(1.0, 6.0), (0.37, 1.875), (2.0 ** -20, 2.0 ** -15), (1e4, 786432.0),
                     (2.0 ** -110, 2.0 ** -100), (2.0 ** 105, 2.0 ** 110), (3.0e-20, 2.0 ** -40)]:
        sel = bits[np.abs(x.astype(np.float64)) <= amax]
        sel = np.concatenate([sel, np.zeros((-sel.size) % 15, np.uint16)]).reshape(-1, 15)
        a16 = np.uint16(np.float32(amax).view(np.uint32) >> 16)
        assert F.bf16_bits_to_f32(np.array([a16]))[0] == np.float32(amax)
        blk = np.concatenate([np.full((sel.shape[0], 1), a16, np.uint16), sel], axis=1).reshape(1, -1)
        st = np.float32(st)
        ts = dev_f32(np.array([st], np.float32))
        p, s, _ = run_quant(m, dev_bf16(blk), "nvfp4", "sr", seed=0x5EED5EED12345, step=step,
                            tscale="given", ts=ts)
        rp, rs = nvfp4.quantize_packed(F.bf16_bits_to_f32(blk), st, "sr", seed=0x5EED5EED12345,
                                       step=step)
        np.testing.assert_array_equal(s, rs)
        np.testing.assert_array_equal(p, rp)


def test_nvfp4_sr_fp32_quotients_over_the_exponent_range():
    """NVFP4 SR from fp32 with given tensor scales: the quotient x / s_dec is
    formed without a division (reciprocal plus one fma correction) where
    that is the IEEE quotient, and by an IEEE division for elements or
    quotients below 2^-100 and for blocks whose scale left the division-free
    chain.  SR reads every bit of the quotient: random fp32 significands over
    a wide exponent range, including subnormals, against the oracle."""
    m = need_gpu()
    rng = np.random.default_rng(77)
    rows, cols = 256, 1024
    for st in (1.0, 3.7e-5, 2.0 ** -99, 2.0 ** 99, 2.0 ** -110, 1.5e30):
        sig = rng.uniform(1.0, 2.0, size=(rows, cols))
        # per 16-element block a base exponent, per element a spread of 0..40 below it
        e_blk = rng.integers(-140, 60, size=(rows, cols // 16))
        e = np.repeat(e_blk, 16, axis=1) - rng.integers(0, 41, size=(rows, cols))
        x = (np.where(rng.random((rows, cols)) < 0.5, -1.0, 1.0) * sig * np.exp2(e.astype(np.float64))).astype(np.float32)
        x[rng.random(x.shape) < 0.02] = 0.0
        assert np.all(np.isfinite(x))
        ts = dev_f32(np.array([st], np.float32))
        for step in (0, 5):
            p, s, _ = run_quant(m, dev_f32(x), "nvfp4", "sr", seed=0xABCDEF, step=step, tscale="given", ts=ts)
            rp, rs = nvfp4.quantize_packed(x, np.float32(st), "sr", seed=0xABCDEF, step=step)
            np.testing.assert_array_equal(s, rs, err_msg=f"S_t {st}")
            np.testing.assert_array_equal(p, rp, err_msg=f"S_t {st}")
