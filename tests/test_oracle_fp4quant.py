"""Pins of the FP4Quant group codec ("FP4Quant speeds up GPU communication",
"Why four bits need more than rounding") -- CPU only."""
import numpy as np
import pytest

from oracle import formats as F
from oracle import fp4quant as Q


@pytest.mark.parametrize("G", [16, 64, 256])
def test_hadamard_natural_order_and_self_inverse(G):
    H = Q.hadamard(G)
    i = np.arange(G)
    pop = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    np.testing.assert_array_equal(H, (-1.0) ** pop)
    np.testing.assert_array_equal(H @ H, G * np.eye(G))


def _butterfly_f32(x):
    """Independent in-place add/sub butterflies (natural order), float32."""
    v = x.astype(np.float32).copy()
    G = v.shape[-1]
    h = 1
    while h < G:
        v = v.reshape(v.shape[0], -1, 2, h)
        a, b = v[:, :, 0, :].copy(), v[:, :, 1, :].copy()
        v[:, :, 0, :], v[:, :, 1, :] = a + b, a - b
        v = v.reshape(-1, G)
        h *= 2
    return v


@pytest.mark.parametrize("G", [64, 256])
def test_one_hot_group_reconstructs_exactly(G):
    x = np.zeros((1, G), np.float32)
    x[0, 5] = -3.0
    codes, s1, s2 = Q.encode(x, G)
    assert s1[0, 0] == np.float32(3.0 / np.sqrt(G))
    assert s2[0, 0] == np.float32(1.0 / 6.0)
    assert np.all(np.abs(F.e2m1_decode(codes)) == 6.0)
    np.testing.assert_allclose(Q.decode64(codes, s1, s2, G), x, rtol=0, atol=1e-6)


@pytest.mark.parametrize("G", [64, 256])
def test_constant_group_reconstructs(G):
    x = np.full((1, G), 0.75, np.float32)
    codes, s1, s2 = Q.encode(x, G)
    assert F.e2m1_decode(codes[0, 0]) == 6.0 and np.all(codes[0, 1:] == 0)
    np.testing.assert_allclose(Q.decode64(codes, s1, s2, G), x, rtol=1e-6)


@pytest.mark.parametrize("G", [64, 256])
def test_power_of_two_scaling_invariance(G):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 4 * G)).astype(np.float32)
    c, s1, s2 = Q.encode(x, G)
    for k in (-20, 3, 40):
        c2, t1, t2 = Q.encode(np.ldexp(x, k).astype(np.float32), G)
        np.testing.assert_array_equal(c2, c)
        np.testing.assert_array_equal(t2, s2)
        np.testing.assert_array_equal(t1, np.ldexp(s1, k).astype(np.float32))


@pytest.mark.parametrize("G", [64, 256])
def test_against_fp32_butterflies(G):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((256, 1024)).astype(np.float32)
    x[:, rng.choice(1024, 10, replace=False)] *= 20
    codes, s1, s2 = Q.encode(x, G)
    xg = x.reshape(-1, G)
    w = _butterfly_f32(xg)
    mx = np.max(np.abs(w), axis=1, keepdims=True)
    c32 = F.e2m1_rtn((w * (np.float32(6) / mx)).astype(np.float32)).reshape(codes.shape)
    grid_pos = lambda c: np.sign(F.e2m1_decode(c)) * np.searchsorted(F.E2M1_MAG, np.abs(F.e2m1_decode(c)))
    diff = np.abs(grid_pos(c32) - grid_pos(codes))
    assert diff.max() <= 1 and np.mean(diff > 0) < 1e-4
    ref_s1 = np.sqrt(np.mean(xg.astype(np.float64) ** 2, axis=1))
    np.testing.assert_allclose(s1.reshape(-1), ref_s1, rtol=1e-6)
    np.testing.assert_allclose(s2.reshape(-1), mx[:, 0] / (6 * np.sqrt(G) * ref_s1), rtol=1e-6)


def test_transform_without_rounding_is_identity():
    G = 64
    rng = np.random.default_rng(6)
    y = rng.standard_normal((10, G))
    H = Q.hadamard(G) / np.sqrt(G)
    np.testing.assert_allclose(y @ H.T @ H.T, y, atol=1e-12)


@pytest.mark.parametrize("G", [16, 64, 1024])
def test_two_hot_group_ratios_closed_form(G):
    """x = a e_i + b e_j (i != j): z is proportional to a H[:, i] + b H[:, j],
    whose largest magnitude |a| + |b| is reached on the rows where the two
    columns agree in sign (half of them), so z / s2 is
    6 (a H[k, i] + b H[k, j]) / (|a| + |b|) for every k."""
    rng = np.random.default_rng(G)
    H = Q.hadamard(G)
    for _ in range(5):
        i, j = rng.choice(G, 2, replace=False)
        a, b = np.float32(rng.standard_normal() * 3), np.float32(rng.standard_normal())
        x = np.zeros((1, G), np.float32)
        x[0, i], x[0, j] = a, b
        want = 6.0 * (float(a) * H[:, i] + float(b) * H[:, j]) / (abs(float(a)) + abs(float(b)))
        np.testing.assert_allclose(Q.ratios(x, G)[0], want, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(Q.encode(x, G)[0][0], F.e2m1_rtn(want))


def test_zero_group():
    x = np.zeros((2, 128), np.float32)
    x[1, 64:] = 1.0
    c, s1, s2 = Q.encode(x, 64)
    assert np.all(c[0] == 0) and s1[0, 0] == 0 and s2[0, 0] == 0
    assert np.all(Q.decode64(c, s1, s2, 64)[0] == 0)


def _signed_grid(codes):
    return F.e2m1_decode(codes)


def test_sr_variant_brackets_and_is_unbiased():
    """Stochastic rounding of z / s2: every code is one of the two grid
    values around z / s2, and over many steps the codes average to z / s2
    (the SR draws are uniform, so the rounding is unbiased)."""
    rng = np.random.default_rng(31)
    G = 64
    x = rng.standard_normal((1, 2 * G)).astype(np.float32)
    q = Q.ratios(x, G)[0]
    a = np.abs(q)
    lo_i = np.clip(np.searchsorted(F.E2M1_MAG, a, side="right") - 1, 0, 7)
    lo = np.sign(q) * F.E2M1_MAG[lo_i]
    hi = np.sign(q) * F.E2M1_MAG[np.minimum(lo_i + 1, 7)]
    steps = 1024
    acc = np.zeros_like(q)
    for t in range(steps):
        c = Q.encode(x, G, "sr", seed=3, step=t)[0][0]
        v = _signed_grid(c)
        assert np.all((v == lo) | (v == hi) | (np.abs(v) == np.abs(lo)) & (lo == 0))
        acc += v
    # the spread of one draw is at most half the widest gap (1), so 6 sigma
    # of the mean of 1024 draws is 6 / 32
    assert np.max(np.abs(acc / steps - q)) < 6 / 32
    assert not np.array_equal(Q.encode(x, G, "sr", seed=3, step=0)[0], Q.encode(x, G)[0])


def test_sr_variant_stream_follows_the_flat_index():
    """Codes of the SR variant do not change when the rows are reshaped
    (groups stay whole) and a sample of rows with row_ids matches those rows
    of the whole tensor."""
    rng = np.random.default_rng(32)
    R, C, G = 4, 256, 64
    x = rng.standard_normal((R, C)).astype(np.float32)
    c = Q.encode(x, G, "sr", seed=9, step=4)[0]
    c2 = Q.encode(x.reshape(1, R * C), G, "sr", seed=9, step=4)[0]
    np.testing.assert_array_equal(c2.reshape(R, C), c)
    rows = np.array([1, 3])
    np.testing.assert_array_equal(Q.encode(x[rows], G, "sr", seed=9, step=4, row_ids=rows)[0], c[rows])
