"""Pins for the element formats of the oracle (CPU only)."""
import math

import numpy as np
import pytest
import torch

from conftest import read_golden_rows
from oracle import formats as F


def test_e2m1_table_matches_page():
    rows = read_golden_rows("e2m1_table.txt")
    assert len(rows) == 8
    for eb, mb, val in rows:
        m3 = (int(eb, 2) << 1) | int(mb)
        assert F.e2m1_decode(m3) == float(val)
        assert F.e2m1_decode(m3 | 8) == -float(val)     # sign bit gives the copies
    assert math.copysign(1.0, F.e2m1_decode(8)) == -1.0


def test_e2m1_closed_form_bias_one():
    # independent derivation: 1 sign, 2 exponent, 1 mantissa bit, bias 1,
    # subnormal when the exponent field is 0
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        v = (2.0 ** (e - 1)) * (1 + m / 2) if e else 0.5 * m
        assert F.e2m1_decode(code) == (-v if s else v)


def _rtn_by_thresholds(a):
    """Second formulation of E2M1 RTN on a magnitude: the interval table with
    its tie rule (ties go to the value whose code is even)."""
    if a <= 0.25:
        return 0
    if a < 0.75:
        return 1
    if a <= 1.25:
        return 2
    if a < 1.75:
        return 3
    if a <= 2.5:
        return 4
    if a < 3.5:
        return 5
    if a <= 5.0:
        return 6
    return 7


def test_e2m1_rtn_exhaustive_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = F.bf16_bits_to_f32(bits)
    finite = np.isfinite(x)
    x = x[finite]
    got = F.e2m1_rtn(x)
    want = np.array([_rtn_by_thresholds(abs(float(v))) | (8 if math.copysign(1, v) < 0 else 0)
                     for v in x], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def test_e2m1_rtn_fp32_around_thresholds():
    vals = []
    for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0):
        v = np.float32(t)
        for k in range(-4, 5):
            w = v
            step = np.float32(np.inf) if k > 0 else np.float32(-np.inf)
            for _ in range(abs(k)):
                w = np.nextafter(w, step)
            vals += [w, -w]
    vals = np.array(vals + [np.float32(1e30), np.float32(np.inf), np.float32(-np.inf),
                            np.float32(1e-45), np.float32(0.0), np.float32(-0.0)], dtype=np.float32)
    got = F.e2m1_rtn(vals)
    want = [_rtn_by_thresholds(min(abs(float(v)), 6.0)) | (8 if math.copysign(1, v) < 0 else 0)
            for v in vals]
    np.testing.assert_array_equal(got, np.array(want, dtype=np.uint8))


def test_e2m1_rtn_grid_points_map_to_themselves_and_monotone():
    for code in range(16):
        assert F.e2m1_rtn(np.float32(F.e2m1_decode(code))) == code
    xs = np.linspace(0, 8, 100001, dtype=np.float32)
    c = F.e2m1_rtn(xs).astype(int)
    assert np.all(np.diff(c) >= 0)


def test_e2m1_rtn_margin_is_distance_to_first_decision_change():
    """Brute force: from each q, bisect in both directions for the first
    point where e2m1_rtn picks another signed grid magnitude (+-0 merged);
    the nearer of the two is the margin."""
    rng = np.random.default_rng(11)
    mids = F.E2M1_MIDPOINTS
    q = np.concatenate([rng.uniform(-6.5, 6.5, 600), F.E2M1_MAG, -F.E2M1_MAG, mids, -mids,
                        mids + 1e-9, mids - 1e-9, [0.0, -0.0, 6.0, 6.5, -6.5]])

    def decision(v):
        c = F.e2m1_rtn(v).astype(np.int64)
        return np.where((c & 8) != 0, -1, 1) * (c & 7)

    d0 = decision(q)

    def first_change(sgn):
        reach = 8.0
        far = decision(q + sgn * reach) != d0
        lo, hi = np.zeros_like(q), np.full_like(q, reach)
        for _ in range(80):
            mid = (lo + hi) / 2
            ch = decision(q + sgn * mid) != d0
            hi, lo = np.where(ch, mid, hi), np.where(ch, lo, mid)
        return np.where(far, hi, np.inf)

    brute = np.minimum(first_change(1.0), first_change(-1.0))
    np.testing.assert_allclose(F.e2m1_rtn_margin(q), brute, rtol=0, atol=1e-12)
    assert np.all(F.e2m1_rtn_margin(mids) == 0) and np.all(F.e2m1_rtn_margin(F.E2M1_MAG[1:-1]) > 0.2)


def test_e2m1_rtn_nan_raises():
    with pytest.raises(ValueError):
        F.e2m1_rtn(np.array([np.nan], dtype=np.float32))


def test_e2m1_sr_limits():
    # u = 0 always rounds up off-grid, u -> 1 always down; grid points stay
    q = np.array([2.3, -2.3, 0.1, 5.5, 7.0, 3.0], dtype=np.float32)
    up = F.e2m1_sr(q, np.zeros(6))
    dn = F.e2m1_sr(q, np.full(6, 1 - 2.0 ** -24))
    assert list(F.e2m1_decode(up)) == [3.0, -3.0, 0.5, 6.0, 6.0, 3.0]
    assert list(F.e2m1_decode(dn)) == [2.0, -2.0, 0.0, 4.0, 6.0, 3.0]


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = F.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_e4m3_encode_matches_torch_rne():
    # torch's CPU cast is RNE; it agrees with saturation for |x| <= 464
    pos = F.e4m3_decode(np.arange(0x7F))
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(0)
    vals = np.concatenate([pos, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                           rng.uniform(0, 464, 20000), np.exp2(rng.uniform(-14, 8.85, 20000)),
                           [464.0, 2.0 ** -10, 1.5 * 2.0 ** -10, 0.00785]])
    vals = vals[vals <= 464].astype(np.float32)
    vals = np.concatenate([vals, -vals])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(F.e4m3_encode(vals.astype(np.float64)), ref)


def test_e4m3_encode_saturates():
    assert F.e4m3_encode(np.float64(465.0)) == 0x7E
    assert F.e4m3_encode(np.float64(1e30)) == 0x7E
    assert F.e4m3_encode(np.float64(-1e30)) == 0xFE
    assert F.e4m3_encode(np.float64(-0.0)) == 0x80


def test_e8m0_decode():
    b = np.arange(255)
    np.testing.assert_array_equal(F.e8m0_decode(b), [math.ldexp(1.0, int(k) - 127) for k in b])
    assert np.isnan(F.e8m0_decode(255))


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    # plant exact ties and near-ties in the dropped half
    u[:5000] = (u[:5000] & 0xFFFF0000) | 0x8000
    u[5000:10000] = (u[5000:10000] & 0xFFFF0000) | 0x7FFF
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(F.f32_to_bf16_bits(x), ref)


def test_pack_roundtrip_and_nibble_order():
    c = np.arange(16, dtype=np.uint8)
    p = F.pack_codes(c)
    assert p[0] == 0x10 and p[7] == 0xFE
    np.testing.assert_array_equal(F.unpack_codes(p), c)


def test_e2m1_sr_margin_is_distance_to_first_decision_change():
    """Brute force, as for the RTN margin: with u fixed, bisect in both
    directions for the first point where e2m1_sr picks another signed grid
    magnitude (+-0 merged)."""
    rng = np.random.default_rng(12)
    q = np.concatenate([rng.uniform(-6.5, 6.5, 500), F.E2M1_MAG, -F.E2M1_MAG, [0.0, 0.3, -0.3]])
    u = np.concatenate([rng.random(500), np.zeros(8), np.full(8, 0.5), [0.0, 0.0, 1 - 2.0 ** -24]])
    u = np.floor(u * 2 ** 24) * 2.0 ** -24                   # the stream's 24-bit values

    def decision(v):
        c = F.e2m1_sr(v, u).astype(np.int64)
        return np.where((c & 8) != 0, -1, 1) * (c & 7)

    d0 = decision(q)

    def first_change(sgn):
        reach = 8.0
        far = decision(q + sgn * reach) != d0
        lo, hi = np.zeros_like(q), np.full_like(q, reach)
        for _ in range(80):
            mid = (lo + hi) / 2
            ch = decision(q + sgn * mid) != d0
            hi, lo = np.where(ch, mid, hi), np.where(ch, lo, mid)
        return np.where(far, hi, np.inf)

    brute = np.minimum(first_change(1.0), first_change(-1.0))
    np.testing.assert_allclose(F.e2m1_sr_margin(q, u), brute, rtol=0, atol=1e-12)


def _rocm_fp4x2(pairs):
    """Bytes from ROCm's host-side fp4x2 packing of float pairs (first element
    of the pair is the .x component)."""
    import os
    import shutil
    import subprocess
    import tempfile
    hipcc = next((c for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")) if c and os.path.exists(c)),
                 None)
    if hipcc is None or not os.path.exists("/opt/rocm/include/hip/hip_fp4.h"):
        pytest.skip("hipcc or hip_fp4.h missing")
    src = os.path.join(os.path.dirname(__file__), "hip_fp4x2_ref.cpp")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "ref")
        subprocess.run([hipcc, "-O1", "-std=c++17", src, "-o", exe], check=True, capture_output=True)
        inp = "".join(f"{a!r} {b!r}\n" for a, b in pairs)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    return np.array([int(t) for t in out.split()], dtype=np.uint8)


def test_pack_order_matches_rocm_fp4x2_storage():
    """The packed layout (two codes per byte, "fp4-train" "How it works";
    the FP4Quant article's "Making compression cheap enough to help") against
    an implementation outside the oracle: ROCm's fp4x2 storage type puts the
    first element of a pair in the low nibble.  Every pair of grid values
    (16 x 16 codes, so no rounding is involved) pins the nibble order and the
    sign bit; random pairs inside [-6, 6] also pin e2m1_rtn away from ties."""
    grid = F.e2m1_decode(np.arange(16))
    a, b = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    pairs = [(float(grid[i]), float(grid[j])) for i, j in zip(a.ravel(), b.ravel())]
    rng = np.random.default_rng(11)
    r = rng.uniform(-6.0, 6.0, size=(4000, 2)).astype(np.float32)
    pairs += [(float(x), float(y)) for x, y in r]
    got = _rocm_fp4x2(pairs)
    codes = np.stack([np.arange(16)[a.ravel()], np.arange(16)[b.ravel()]], axis=-1).astype(np.uint8)
    np.testing.assert_array_equal(got[:256], F.pack_codes(codes).ravel())
    np.testing.assert_array_equal(got[256:], F.pack_codes(F.e2m1_rtn(r)).ravel())
