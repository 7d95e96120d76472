"""Seeded random sweep of fp4_quantize / fp4_dequantize against the oracle:
random shapes (ragged rows, several block rows), random value mixes (heavy
tails, exact zeros and negative zeros, tiny and large magnitudes, per-row
exponent spread) over every format x rounding x input dtype x tensor-scale
mode, and inputs over the whole fp32 exponent range for quantize,
dequantize and error feedback.  Bit-exact codes, scales, tensor scale,
dequantized values and residuals."""
import numpy as np
import pytest
import torch

from gpu_util import Guarded, dev_bf16, dev_f32, host, host_bf16, need_gpu
from oracle import formats as F
from oracle import mxfp4, nvfp4

pytestmark = pytest.mark.gpu


def _values(rng, rows, cols):
    x = rng.standard_t(2.5, size=(rows, cols)) * np.exp2(rng.integers(-40, 40, size=(rows, 1)))
    r = rng.random((rows, cols))
    x[r < 0.03] = 0.0
    x[(r >= 0.03) & (r < 0.05)] = -0.0
    x[(r >= 0.05) & (r < 0.06)] *= 2.0 ** -90
    x[(r >= 0.06) & (r < 0.07)] *= 2.0 ** 60
    return x.astype(np.float32)


def _cases():
    out = []
    rng = np.random.default_rng(2024)
    for fmt in ("nvfp4", "mxfp4"):
        for rounding in ("rtn", "sr"):
            for dtype in ("bf16", "f32"):
                for tscale in (("compute", "given") if fmt == "nvfp4" else ("compute",)):
                    for _ in range(2):
                        rows = int(rng.integers(1, 300))
                        cols = 32 * int(rng.integers(1, 64))
                        out.append((fmt, rounding, dtype, tscale, rows, cols, int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("fmt,rounding,dtype,tscale,rows,cols,seed", _cases())
def test_random_quantize_dequantize(fmt, rounding, dtype, tscale, rows, cols, seed):
    m = need_gpu()
    rng = np.random.default_rng(seed)
    x = _values(rng, rows, cols)
    sr_seed, step = int(rng.integers(1 << 62)), int(rng.integers(1 << 40))
    st = np.float32(rng.uniform(1e-3, 10.0)) if tscale == "given" else None
    _check_quantize_dequantize(m, x, fmt, rounding, dtype, tscale, st, sr_seed, step)


def _check_quantize_dequantize(m, x, fmt, rounding, dtype, tscale, st, sr_seed, step):
    rows, cols = x.shape
    if dtype == "bf16":
        xb = F.f32_to_bf16_bits(x)
        x = F.bf16_bits_to_f32(xb)
        x_dev = dev_bf16(xb)
    else:
        x_dev = dev_f32(x)
    blk = 16 if fmt == "nvfp4" else 32
    if fmt == "nvfp4" and tscale == "compute":
        st = nvfp4.tensor_scale(x)
    gp, gs = Guarded(rows * cols // 2), Guarded(rows * cols // blk)
    ts = dev_f32(np.array([0.0 if fmt == "mxfp4" or tscale == "compute" else st], np.float32))
    p, s, ts_out = m.fp4_quantize(x_dev, fmt, rounding, sr_seed, step, tscale,
                                  ts if fmt == "nvfp4" else None,
                                  gp.view(torch.uint8, (rows, cols // 2)),
                                  gs.view(torch.uint8, (rows, cols // blk)))
    torch.cuda.synchronize()
    gp.check()
    gs.check()
    p, s = host(p), host(s)
    if fmt == "nvfp4":
        assert np.float32(host(ts_out)[0]) == np.float32(st)
        rp, rs = nvfp4.quantize_packed(x, np.float32(st), rounding, seed=sr_seed, step=step)
    else:
        rp, rs = mxfp4.quantize_packed(x, rounding, seed=sr_seed, step=step)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(p, rp)
    for out in (torch.bfloat16, torch.float32):
        es = 2 if out == torch.bfloat16 else 4
        gy = Guarded(rows * cols * es)
        y = m.fp4_dequantize(torch.from_numpy(p).cuda(), torch.from_numpy(s).cuda(), rows, cols, fmt,
                             dev_f32(np.array([st], np.float32)) if fmt == "nvfp4" else None, out,
                             gy.view(out, (rows, cols)))
        torch.cuda.synchronize()
        gy.check()
        kind = "bf16" if out == torch.bfloat16 else "f32"
        if fmt == "nvfp4":
            ref = nvfp4.dequantize(rp, rs, np.float32(st), kind)
        else:
            ref = mxfp4.dequantize(rp, rs, kind)
        got = host_bf16(y) if out == torch.bfloat16 else host(y)
        if out == torch.bfloat16:
            np.testing.assert_array_equal(got, ref)
        else:
            np.testing.assert_array_equal(got.view(np.uint32), np.asarray(ref, np.float32).view(np.uint32))


def _extreme_values(rng, rows, cols, blk, cap=3.0e38):
    """Every row at its own binary exponent in [-150, 127], 30% of the blocks
    shifted by another 2^-30 .. 2^30 (blocks far above and below their row,
    fp32 subnormals, values near the fp32 maximum), exact and negative zeros."""
    e = rng.integers(-150, 128, size=(rows, 1))
    t = np.clip(rng.standard_t(3, size=(rows, cols)), -1.99, 1.99)
    nb = cols // blk
    kb = rng.integers(-30, 31, size=(rows, nb)) * (rng.random((rows, nb)) < 0.3)
    x = t * np.exp2(np.clip(e + np.repeat(kb, blk, axis=1), -160, 127).astype(np.float64))
    r = rng.random((rows, cols))
    x[r < 0.03] = 0.0
    x[(r >= 0.03) & (r < 0.04)] = -0.0
    return np.clip(x, -cap, cap).astype(np.float32)


def _extreme_cases():
    rng = np.random.default_rng(4242)
    out = []
    for fmt in ("nvfp4", "mxfp4"):
        for rounding in ("rtn", "sr"):
            for dtype in ("bf16", "f32"):
                for tscale in (("compute", "given") if fmt == "nvfp4" else ("compute", "compute")):
                    out.append((fmt, rounding, dtype, tscale, int(rng.integers(1, 200)),
                                32 * int(rng.integers(1, 48)), int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("fmt,rounding,dtype,tscale,rows,cols,seed", _extreme_cases())
def test_extreme_magnitudes_quantize_dequantize(fmt, rounding, dtype, tscale, rows, cols, seed):
    """Inputs over the whole fp32 exponent range and, for a given S_t, tensor
    scales from 2^-149 to 2^127.9 (outside the range where the kernels use
    division-free quotients): still bit-exact."""
    m = need_gpu()
    rng = np.random.default_rng(seed)
    x = _extreme_values(rng, rows, cols, 16 if fmt == "nvfp4" else 32)
    sr_seed, step = int(rng.integers(1 << 62)), int(rng.integers(1 << 40))
    st = np.float32(np.exp2(rng.uniform(-149, 127.9))) if tscale == "given" else None
    _check_quantize_dequantize(m, x, fmt, rounding, dtype, tscale, st, sr_seed, step)


def _extreme_ef_cases():
    rng = np.random.default_rng(4343)
    out = []
    for rounding in ("rtn", "sr"):
        for xdt, odt in (("bf16", "bf16"), ("f32", "f32"), ("f32", "bf16"), ("bf16", "f32")):
            for tscale in ("compute", "given"):
                out.append((rounding, xdt, odt, tscale, int(rng.integers(1, 150)),
                            16 * int(rng.integers(1, 64)), int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("rounding,xdt,odt,tscale,rows,cols,seed", _extreme_ef_cases())
def test_extreme_magnitudes_error_feedback(rounding, xdt, odt, tscale, rows, cols, seed):
    """Error feedback on the same extreme inputs (|x| <= 1e38 so that x + r
    stays finite), residuals up to 0.3 |x|, with and without codes: output,
    residual, codes, scales and S_t bit-exact."""
    m = need_gpu()
    rng = np.random.default_rng(seed)
    x = _extreme_values(rng, rows, cols, 16, cap=1e38)
    if xdt == "bf16":
        xb = F.f32_to_bf16_bits(x)
        x = F.bf16_bits_to_f32(xb)
        x_dev = dev_bf16(xb)
    else:
        x_dev = dev_f32(x)
    r = (x * rng.uniform(-0.3, 0.3, size=x.shape)).astype(np.float32)
    v = (x + r).astype(np.float32)
    assert np.all(np.isfinite(v))
    st = np.float32(np.exp2(rng.uniform(-149, 127.9))) if tscale == "given" else None
    sr_seed, step = int(rng.integers(1 << 62)), int(rng.integers(1 << 40))
    codes = bool(seed & 1)
    od = torch.bfloat16 if odt == "bf16" else torch.float32
    gy = Guarded(rows * cols * (2 if odt == "bf16" else 4))
    y = gy.view(od, (rows, cols))
    ts = dev_f32(np.array([st if tscale == "given" else 0.0], np.float32))
    gp = Guarded(rows * cols // 2) if codes else None
    gs = Guarded(rows * cols // 16) if codes else None
    r_dev = dev_f32(r)
    m.fp4_errfeedback_qdq(x_dev, r_dev, y, None, rounding, sr_seed, step, tscale, ts,
                          gp.view(torch.uint8, (rows, cols // 2)) if codes else None,
                          gs.view(torch.uint8, (rows, cols // 16)) if codes else None)
    torch.cuda.synchronize()
    for g in (gy, gp, gs):
        if g is not None:
            g.check()
    oy, orr, op, osc, ost = nvfp4.errfeedback_qdq(x, r, st, rounding, seed=sr_seed, step=step, out=odt)
    assert np.float32(host(ts)[0]) == np.float32(ost)
    if odt == "bf16":
        np.testing.assert_array_equal(host_bf16(y), oy)
    else:
        np.testing.assert_array_equal(host(y).view(np.uint32), np.asarray(oy, np.float32).view(np.uint32))
    np.testing.assert_array_equal(host(r_dev).view(np.uint32), orr.view(np.uint32))
    if codes:
        np.testing.assert_array_equal(host(gs.view(torch.uint8, (rows, cols // 16))), osc)
        np.testing.assert_array_equal(host(gp.view(torch.uint8, (rows, cols // 2))), op)


def _fp8_cases():
    rng = np.random.default_rng(77)
    shapes = [(1, 896), (3, 384), (40, 896), (300, 256), (2100, 128), (3, 1024), (40, 512), (300, 640)]
    return [(E, H, int(rng.integers(1 << 30))) for E, H in shapes]


@pytest.mark.parametrize("E,H,seed", _fp8_cases())
def test_random_fp8_row_and_column(E, H, seed):
    """Random expert counts (geometric, with empty experts and a few large
    ones) and hidden sizes: FP8 rows and per-expert FP8 columns, bit-exact."""
    from oracle import fp8col
    import synth
    m = need_gpu()
    rng = np.random.default_rng(seed)
    counts = rng.geometric(0.25, size=E) - 1
    counts[rng.random(E) < 0.2] = 0
    big = rng.random(E) < (0.5 if E < 10 else 0.01)
    counts[big] = rng.integers(200, 700, size=int(big.sum()))
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    if T == 0:
        pytest.skip("no tokens drawn")
    packed, sb = synth.random_mxfp4(T, H, seed=seed, scale_lo=100, scale_hi=150)
    go, gs = Guarded(T * H), Guarded(T * H // 128 * 4)
    o, s = m.mxfp4_row_to_fp8_col(torch.from_numpy(packed).cuda(), torch.from_numpy(sb).cuda(),
                                  torch.from_numpy(off).cuda(), H, go.view(torch.uint8, (T * H,)),
                                  gs.view(torch.float32, (T * H // 128,)))
    torch.cuda.synchronize()
    go.check()
    gs.check()
    ro, rs = fp8col.convert(packed, sb, off, H)
    np.testing.assert_array_equal(host(o), ro)
    np.testing.assert_array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    gr, grs = Guarded(T * H), Guarded(T * H // 128 * 4)
    r, rsc = m.mxfp4_row_to_fp8_row(torch.from_numpy(packed).cuda(), torch.from_numpy(sb).cuda(), H,
                                    gr.view(torch.uint8, (T, H)), grs.view(torch.float32, (T, H // 128)))
    torch.cuda.synchronize()
    gr.check()
    grs.check()
    qo, qs = fp8col.convert_rows(packed, sb, H)
    np.testing.assert_array_equal(host(r), qo)
    np.testing.assert_array_equal(host(rsc).view(np.uint32), qs.view(np.uint32))


def test_binding_checks_tensor_arguments():
    """The C ABI sees plain pointers, so the binding checks every tensor it
    passes: an output that is too small, of the wrong dtype, strided or on
    the host is refused before anything is launched."""
    m = need_gpu()
    x = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        m.fp4_quantize(x, "mxfp4", packed=torch.empty((64, 100), dtype=torch.uint8, device="cuda"))
    with pytest.raises(TypeError):
        m.fp4_quantize(x, "mxfp4", scales=torch.empty((64, 8), dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        m.fp4_quantize(x, "mxfp4", packed=torch.empty((128, 128), dtype=torch.uint8, device="cuda")[::2])
    with pytest.raises(ValueError):
        m.fp4_quantize(x, "nvfp4", tensor_scale=torch.empty(1, dtype=torch.float32))
    p, s, _ = m.fp4_quantize(x, "mxfp4")
    with pytest.raises(ValueError):
        m.fp4_dequantize(p, s, 64, 256, "mxfp4", y=torch.empty((64, 255), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        m.mxfp4_row_to_fp8_row(p, s, 256, fp8_out=torch.empty((64, 128), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
