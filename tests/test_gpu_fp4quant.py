"""GPU parity of fp4quant_encode / fp4quant_decode against the oracle.

Tolerances follow from fp32 arithmetic (u = 2^-24).  Each output of the
transform is a depth-log2(G) tree sum of +-x, so its error is at most
gamma_n sum|x| <= gamma_n sqrt(G) max|Hx| = eta max|Hx|.  A code may then
differ from the oracle's by one step of the signed grid (+-0 merged), and
only where the oracle's z / s2 lies within 6 (2 eta + 4u) of an E2M1
rounding boundary; s2 agrees within eta + (log2 G + 8) u, s1 within 1e-6
(a fp32 sum of squares) or one subnormal step.  The decoder, run on the
oracle's own codes and scales, agrees with the oracle's decode within 1e-6
of each output plus two subnormal steps (within 1e-6 of the group's
largest output for groups at the ends of fp32's range).  The full-size
workload and its tighter scale bar are in test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import Guarded, dev_bf16, dev_f32, host, host_bf16, need_gpu
from oracle import formats as F
from oracle import fp4quant as Q
from oracle.philox import sr_uniform

pytestmark = pytest.mark.gpu

SCALE_RTOL = 1e-6
RECON_RTOL = 1e-6
U32 = 2.0 ** -24
SUBNORMAL = 2.0 ** -149


def wht_eta(G):
    n = int(np.log2(G))
    return n * U32 / (1 - n * U32) * np.sqrt(G)


def code_tol(G):
    eta = wht_eta(G)
    return 6.0 * (2 * eta / (1 - eta) + 4 * U32) + 1e-12


def s2_rtol(G):
    return wht_eta(G) + (np.log2(G) + 8) * U32


def grid_pos(codes):
    mag = np.asarray(codes).astype(np.int64) & 7
    sign = np.where((np.asarray(codes) & 8) != 0, -1, 1)
    return np.where(mag == 0, 0, sign * mag)


def encode_gpu(m, x_dev, G):
    rows, cols = x_dev.shape
    gp, g1, g2 = Guarded(rows * cols // 2), Guarded(rows * cols // G * 4), Guarded(rows * cols // G * 4)
    p, s1, s2 = m.fp4quant_encode(x_dev, G, gp.view(torch.uint8, (rows, cols // 2)),
                                  g1.view(torch.float32, (rows, cols // G)),
                                  g2.view(torch.float32, (rows, cols // G)))
    torch.cuda.synchronize()
    for g in (gp, g1, g2):
        g.check()
    return host(p), host(s1), host(s2)


def decode_gpu(m, p, s1, s2, G, out):
    rows, cols = p.shape[0], p.shape[1] * 2
    gy = Guarded(rows * cols * (2 if out == torch.bfloat16 else 4))
    y = m.fp4quant_decode(torch.from_numpy(p).cuda(), dev_f32(s1), dev_f32(s2), rows, cols, G, out,
                          gy.view(out, (rows, cols)))
    torch.cuda.synchronize()
    gy.check()
    return host_bf16(y) if out == torch.bfloat16 else host(y)


def check_encode(p, s1, s2, x32, G, code_frac=None):
    rc, r1, r2 = Q.encode(x32, G)
    codes = F.unpack_codes(p)
    d = np.abs(grid_pos(codes) - grid_pos(rc))
    assert d.max() <= 1
    margin = F.e2m1_rtn_margin(Q.ratios(x32, G))[d > 0]
    assert np.all(margin <= code_tol(G)), (margin.max(), code_tol(G))
    if code_frac is not None:
        assert np.mean(d > 0) < code_frac, np.mean(d > 0)
    np.testing.assert_allclose(s1, r1, rtol=SCALE_RTOL, atol=SUBNORMAL)
    np.testing.assert_allclose(s2, r2, rtol=s2_rtol(G), atol=0)
    return codes


def encode_gpu_sr(m, x_dev, G, seed, step):
    rows, cols = x_dev.shape
    gp, g1, g2 = Guarded(rows * cols // 2), Guarded(rows * cols // G * 4), Guarded(rows * cols // G * 4)
    p, s1, s2 = m.fp4quant_encode_ex(x_dev, G, "sr", seed, step, gp.view(torch.uint8, (rows, cols // 2)),
                                     g1.view(torch.float32, (rows, cols // G)),
                                     g2.view(torch.float32, (rows, cols // G)))
    torch.cuda.synchronize()
    for g in (gp, g1, g2):
        g.check()
    return host(p), host(s1), host(s2)


def check_encode_sr(p, s1, s2, x32, G, seed, step, row_ids=None, code_frac=None):
    """SR variant: a code may differ from the oracle's only where the oracle's
    z / s2 lies within the transform's error bound of that element's SR
    threshold (formats.e2m1_sr_margin with its draw u), by one grid step, or
    by two where z / s2 itself is that close to 0 (a sign flip at u near 0).
    Scales as for RTN."""
    rc, r1, r2 = Q.encode(x32, G, "sr", seed=seed, step=step, row_ids=row_ids)
    codes = F.unpack_codes(p)
    d = np.abs(grid_pos(codes) - grid_pos(rc))
    R, C = x32.shape
    rows = np.arange(R, dtype=np.int64) if row_ids is None else np.asarray(row_ids, np.int64)
    u = sr_uniform(rows[:, None] * C + np.arange(C, dtype=np.int64)[None, :], seed, step)
    q = Q.ratios(x32, G)
    tol = code_tol(G)
    assert d.max() <= 2
    margin = F.e2m1_sr_margin(q, u)[d > 0]
    assert np.all(margin <= tol), (margin.max(), tol)
    assert np.all(np.abs(q)[d == 2] <= tol)
    if code_frac is not None:
        assert np.mean(d > 0) < code_frac, np.mean(d > 0)
    np.testing.assert_allclose(s1, r1, rtol=SCALE_RTOL, atol=SUBNORMAL)
    np.testing.assert_allclose(s2, r2, rtol=s2_rtol(G), atol=0)
    return codes


def check_decode(m, x32, G, per_element=True, rows=None):
    """The decoder run on the oracle's own codes and scales (its encode of
    x32, rows `rows` of it) against the oracle's float64 decode of them.
    per_element: each output within RECON_RTOL of its own value plus two
    subnormal steps (the decoder's butterflies are exact sums of
    half-integers, followed by one product with a factor rounded twice);
    otherwise within RECON_RTOL of its group's largest value (groups whose
    magnitudes leave fp32's range)."""
    rc, r1, r2 = Q.encode(x32, G)
    if rows is not None:
        rc, r1, r2 = rc[rows], r1[rows], r2[rows]
    p = F.pack_codes(rc)
    ref = Q.decode64(rc, r1, r2, G)
    n_rows, cols = ref.shape
    if per_element:
        tol = RECON_RTOL * np.abs(ref)
    else:
        tol = RECON_RTOL * np.repeat(np.abs(ref).reshape(-1, G).max(axis=1), G).reshape(n_rows, cols)
    tol = tol + 2 * SUBNORMAL
    y = decode_gpu(m, p, r1, r2, G, torch.float32)
    assert np.all(np.abs(y.astype(np.float64) - ref) <= tol)
    yb = F.bf16_bits_to_f32(decode_gpu(m, p, r1, r2, G, torch.bfloat16)).astype(np.float64)
    lo = F.bf16_bits_to_f32(F.f32_to_bf16_bits((ref - tol).astype(np.float32))).astype(np.float64)
    hi = F.bf16_bits_to_f32(F.f32_to_bf16_bits((ref + tol).astype(np.float32))).astype(np.float64)
    assert np.all((yb >= np.minimum(lo, hi)) & (yb <= np.maximum(lo, hi)))


@pytest.mark.parametrize("G", [16, 32, 64, 128, 256, 512, 1024])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_all_group_sizes_small(G, dtype):
    m = need_gpu()
    rng = np.random.default_rng(G)
    rows, cols = 37, 2 * 1024
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[:, rng.choice(cols, 20, replace=False)] *= 20
    x[3] = 0.0                                       # zero groups
    x[4, :G] = 0.0
    x[4, 7] = -2.5                                   # one-hot group
    x[5, :G] = 0.375                                 # constant group
    x[6] *= 2.0 ** -60                               # tiny and huge rows
    x[7] *= 2.0 ** 40
    if dtype == "bf16":
        xb = synth.to_bf16_bits(x)
        x = F.bf16_bits_to_f32(xb)
        xd = dev_bf16(xb)
    else:
        xd = dev_f32(x)
    p, s1, s2 = encode_gpu(m, xd, G)
    codes = check_encode(p, s1, s2, x, G)
    assert np.all(codes[3] == 0) and np.all(s1[3] == 0) and np.all(s2[3] == 0)
    assert np.all(np.abs(F.e2m1_decode(codes[4, :G])) == 6.0)
    check_decode(m, x, G)
    # closed forms reconstruct exactly (to fp32 rounding of the scales)
    y = decode_gpu(m, p, s1, s2, G, torch.float32)
    np.testing.assert_allclose(y[4, :G], x[4, :G], atol=1e-6 * 2.5)
    np.testing.assert_allclose(y[5, :G], x[5, :G], rtol=1e-6)


def test_power_of_two_invariance_on_gpu():
    m = need_gpu()
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 1024)).astype(np.float32)
    p, s1, s2 = encode_gpu(m, dev_f32(x), 256)
    p2, t1, t2 = encode_gpu(m, dev_f32(np.ldexp(x, 13).astype(np.float32)), 256)
    np.testing.assert_array_equal(p2, p)
    np.testing.assert_array_equal(t2, s2)
    np.testing.assert_array_equal(t1, np.ldexp(s1, 13).astype(np.float32))


@pytest.mark.parametrize("G", [16, 32, 64, 128, 256, 512, 1024])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_extreme_magnitudes(G, dtype):
    """Groups whose squares overflow or underflow fp32 (rows scaled by 2^124
    down to 2^-140, outliers 2^60 above a row scaled by 2^40, mixtures of
    2^-90 and normal elements, the largest and the smallest subnormal
    magnitudes): scales, codes and the decode stay within the fp32 bounds."""
    m = need_gpu()
    rng = np.random.default_rng(1000 + G)
    cols = 2048
    exps = [0, 60, 100, 124, -60, -100, -120, -126, -133, -140]
    x = np.clip(rng.standard_normal((len(exps) + 5, cols)), -1.9, 1.9)
    for i, e in enumerate(exps):
        x[i] *= 2.0 ** e
    k = len(exps)
    hot = rng.random(cols) < 0.01
    x[k] *= 2.0 ** 40
    x[k, hot] *= 2.0 ** 60                              # a few 2^100 outliers per group
    tiny = rng.random(cols) < 0.5
    x[k + 1, tiny] *= 2.0 ** -90                        # normal and 2^-90 elements mixed
    x[k + 2] = np.where(rng.random(cols) < 0.5, 1.0, -1.0) * 1.9 * 2.0 ** 126
    x[k + 3] = np.where(rng.random(cols) < 0.5, 1.0, -1.0) * 2.0 ** (-133 if dtype == "bf16" else -149)
    x[k + 4, :] = 0.0
    x[k + 4, ::G] = 2.0 ** -130                         # one-hot groups below the normal range
    x = x.astype(np.float32)
    if dtype == "bf16":
        xb = synth.to_bf16_bits(x)
        x = F.bf16_bits_to_f32(xb)
        xd = dev_bf16(xb)
    else:
        xd = dev_f32(x)
    assert np.all(np.isfinite(x))
    p, s1, s2 = encode_gpu(m, xd, G)
    check_encode(p, s1, s2, x, G)
    nonzero = np.abs(x).reshape(len(x), -1, G).max(axis=2) > 0
    assert np.all((s1 > 0) == nonzero) and np.all((s2 > 0) == nonzero)
    # the decode of the rows whose reconstruction stays inside fp32's range
    keep = np.array([i for i in range(len(x)) if i != k + 2])
    check_decode(m, x, G, per_element=False, rows=keep)


@pytest.mark.parametrize("G", [16, 32, 64, 128, 256, 512, 1024])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sr_variant_all_group_sizes(G, dtype):
    """fp4quant_encode_ex with stochastic rounding on the edge-case data of
    test_all_group_sizes_small, two (seed, step) pairs; the RTN entry point
    and the _ex entry point with RTN give the same bytes."""
    m = need_gpu()
    rng = np.random.default_rng(100 + G)
    rows, cols = 37, 2 * 1024
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[:, rng.choice(cols, 20, replace=False)] *= 20
    x[3] = 0.0
    x[4, :G] = 0.0
    x[4, 7] = -2.5
    x[5, :G] = 0.375
    x[6] *= 2.0 ** -60
    x[7] *= 2.0 ** 40
    if dtype == "bf16":
        xb = synth.to_bf16_bits(x)
        x = F.bf16_bits_to_f32(xb)
        xd = dev_bf16(xb)
    else:
        xd = dev_f32(x)
    for seed, step in ((7, 0), (0x0123456789ABCDEF, (1 << 40) + 3)):
        p, s1, s2 = encode_gpu_sr(m, xd, G, seed, step)
        codes = check_encode_sr(p, s1, s2, x, G, seed, step)
        assert np.all(codes[3] == 0) and np.all(s1[3] == 0)
    pr, _, _ = encode_gpu(m, xd, G)
    pe, _, _ = m.fp4quant_encode_ex(xd, G, "rtn")
    np.testing.assert_array_equal(host(pe), pr)


@pytest.mark.parametrize("G", [64, 256, 1024])
def test_sr_variant_is_unbiased_on_the_gpu(G):
    """Over 256 steps the GPU's SR codes average to the oracle's z / s2
    (each draw spreads at most half the widest grid gap, 1: six sigma of a
    mean of 256 is 6 / 16), while RTN's codes keep their rounding error."""
    m = need_gpu()
    rng = np.random.default_rng(200 + G)
    x = rng.standard_normal((8, 1024)).astype(np.float32)
    xd = dev_f32(x)
    q = Q.ratios(x, G)
    acc = np.zeros_like(q)
    steps = 256
    for t in range(steps):
        p, _, _ = m.fp4quant_encode_ex(xd, G, "sr", 11, t)
        acc += F.e2m1_decode(F.unpack_codes(host(p)))
    err = np.abs(acc / steps - q)
    assert err.max() < 6 / 16
    rtn = F.e2m1_decode(F.unpack_codes(encode_gpu(m, xd, G)[0]))
    assert np.mean(err) < 0.5 * np.mean(np.abs(rtn - q))
