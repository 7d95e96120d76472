"""GPU checks of the conversion steps that the kernels take with hardware
converters or without a division, each against the oracle, bit for bit.

- MXFP4 from bf16 divides by 2^e, rounds and packs with the gfx950 scaled
  converter: every finite bf16 value at every UE8M0 scale byte that bf16 or
  fp32 data can produce (0 .. 252), with RTN and with stochastic rounding.
- MXFP4 from fp32 rescales exactly by 2^-e and rounds at unit scale with the
  same converter: fp32 values within 48 ulps of every E2M1 decision point
  (the midpoints 0.25 .. 5) and every grid value, times every scale 2^e.
- NVFP4 from fp32 with a given S_t forms each quotient x / s_dec as the
  product with the correctly rounded reciprocal plus one fma correction
  (no division): numerators within 48 ulps of t * s_dec for every E2M1
  decision point and grid value t, for 40 S_t significands spread over the
  range and every positive E4M3 scale code.
The stochastic-rounding quotient of bf16 input is covered in
test_gpu_quant.py (every bf16 pattern, seven given scales)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import Guarded, dev_bf16, dev_f32, host, need_gpu
from oracle import formats as F
from oracle import mxfp4, nvfp4

pytestmark = pytest.mark.gpu

THRESHOLDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
GRID = (0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _quantize(m, x_dev, fmt, rounding="rtn", seed=0, step=0, tscale="compute", ts=None):
    rows, cols = x_dev.shape
    blk = 32 if fmt == "mxfp4" else 16
    gp, gs = Guarded(rows * cols // 2), Guarded(rows * cols // blk)
    p, s, _ = m.fp4_quantize(x_dev, fmt, rounding, seed, step, tscale, ts,
                             gp.view(torch.uint8, (rows, cols // 2)),
                             gs.view(torch.uint8, (rows, cols // blk)))
    torch.cuda.synchronize()
    gp.check()
    gs.check()
    return host(p), host(s)


def _ulp_neighbourhood(v, k=48):
    """fp32 values within k ulps of each of v (float32 array), both directions."""
    v = np.asarray(v, np.float32).view(np.int32).astype(np.int64)
    offs = np.arange(-k, k + 1, dtype=np.int64)
    return (v[:, None] + offs[None, :]).astype(np.int32).view(np.float32).reshape(-1)


def _blocks(values, lead, width):
    """Rows of `width` elements: the first is `lead` (which fixes the block
    scale), the rest are the values, zero-padded."""
    vals = np.asarray(values, np.float32)
    n = width - 1
    vals = np.concatenate([vals, np.zeros((-vals.size) % n, np.float32)]).reshape(-1, n)
    return np.concatenate([np.full((vals.shape[0], 1), lead, np.float32), vals], axis=1)


@pytest.mark.parametrize("rounding", ["rtn", "sr"])
def test_mxfp4_bf16_every_pattern_every_scale_byte(rounding):
    m = need_gpu()
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    xall = F.bf16_bits_to_f32(bits)
    xall = xall[np.isfinite(xall)]
    mags = np.abs(xall.astype(np.float64))
    rows = []
    for b in range(0, 253):
        lead = np.float32(2.0 ** (b - 125))              # floor(log2) = b - 125 gives byte b
        rows.append(_blocks(xall[mags < 2.0 ** (b - 124)], lead, 32))
    x = np.concatenate(rows, axis=0)
    x = x.reshape(-1, 32 * 64) if x.shape[0] % 64 == 0 else np.concatenate(
        [x, np.zeros((-x.shape[0] % 64, 32), np.float32)]).reshape(-1, 32 * 64)
    xb = synth.to_bf16_bits(x)
    assert np.array_equal(F.bf16_bits_to_f32(xb), x)       # every value is a bf16 value
    p, s = _quantize(m, dev_bf16(xb), "mxfp4", rounding, seed=0xC0FFEE, step=3)
    rp, rs = mxfp4.quantize_packed(x, rounding, seed=0xC0FFEE, step=3)
    assert set(np.unique(rs).tolist()) >= set(range(0, 253))
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(p, rp)


def test_mxfp4_fp32_decision_points_every_scale():
    m = need_gpu()
    base = _ulp_neighbourhood(np.array(THRESHOLDS + GRID, np.float32))
    base = np.concatenate([base, -base])
    rows = []
    for b in range(1, 253):
        e = b - 127
        vals = (base.astype(np.float64) * 2.0 ** e).astype(np.float32)
        lead = np.float32(2.0 ** (b - 125))
        vals = vals[np.abs(vals.astype(np.float64)) < 2.0 ** (b - 124)]
        rows.append(_blocks(vals, lead, 32))
    x = np.concatenate(rows, axis=0)
    x = np.concatenate([x, np.zeros((-x.shape[0] % 64, 32), np.float32)]).reshape(-1, 32 * 64)
    assert np.all(np.isfinite(x))
    p, s = _quantize(m, dev_f32(x), "mxfp4")
    rp, rs = mxfp4.quantize_packed(x)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(p, rp)


def test_nvfp4_fp32_quotients_near_decision_points():
    m = need_gpu()
    rng = np.random.default_rng(31)
    # S_t significands in [1, 2) (the two ends and random ones) at exponents over the range
    sig = np.concatenate([[1.0, np.nextafter(np.float32(2.0), np.float32(0))],
                          rng.uniform(1.0, 2.0, 38)]).astype(np.float32)
    exps = rng.integers(-60, 40, size=sig.size)
    tscales = (sig.astype(np.float64) * 2.0 ** exps).astype(np.float32)
    codes = np.arange(1, 127)                              # every positive finite E4M3 code
    e4 = F.e4m3_decode(codes)
    t_all = _ulp_neighbourhood(np.array(THRESHOLDS + GRID, np.float32), 48).astype(np.float64)
    for st in tscales:
        blocks = []
        for c, v in zip(codes, e4):
            s_dec = np.float32(np.float32(v) * st)
            if s_dec == 0 or not np.isfinite(s_dec):
                continue
            amax = np.float32(6.0 * float(s_dec))
            x = (t_all * float(s_dec)).astype(np.float32)
            x = np.concatenate([x, -x])
            x = x[np.abs(x) <= amax]
            blocks.append(_blocks(x, amax, 16))
        xs = np.concatenate(blocks, axis=0)
        xs = np.concatenate([xs, np.zeros((-xs.shape[0] % 64, 16), np.float32)]).reshape(-1, 16 * 64)
        ts = dev_f32(np.array([st], np.float32))
        p, s = _quantize(m, dev_f32(xs), "nvfp4", tscale="given", ts=ts)
        rp, rs = nvfp4.quantize_packed(xs, st)
        np.testing.assert_array_equal(s, rs, err_msg=f"S_t {st!r}")
        np.testing.assert_array_equal(p, rp, err_msg=f"S_t {st!r}")
