"""Pins of NVFP4 rounding, SR and error feedback against "fp4-train"
("How it works", "Correctness") -- CPU only."""
import numpy as np

from conftest import read_golden
from oracle import formats as F
from oracle import nvfp4

C = read_golden("fp4_train_correctness.txt")
ONE = np.float32(1.0)


def _anchored(rows, value, dtype=np.float32):
    """Blocks whose element 0 is 6.0: with S_t = 1 the block scale is 1, so
    the other fifteen elements are rounded at unit scale."""
    x = np.full((rows, 16), value, dtype=dtype)
    x[:, 0] = 6.0
    return x


def test_sr_mean_of_2_3_and_rtn():
    x = _anchored(1 << 16, np.float32(2.3))            # 983,040 draws of 2.3
    codes, sc = nvfp4.quantize(x, ONE, "sr", seed=0, step=0)
    assert np.all(sc == 0x38)                         # e4m3 1.0
    vals = F.e2m1_decode(codes[:, 1:])
    n = vals.size
    sigma = np.sqrt(0.3 * 0.7 / n)
    assert set(np.unique(vals)) == {2.0, 3.0}
    assert abs(vals.mean() - float(np.float32(2.3))) < 4 * sigma
    assert abs(vals.mean() - float(C["sr_mean_of_2.3"][0])) < 0.0015
    rcodes, _ = nvfp4.quantize(x, ONE, "rtn")
    assert np.all(F.e2m1_decode(rcodes[:, 1:]) == float(C["rtn_of_2.3"][0]))


def test_sr_unbiased_on_random_values():
    rng = np.random.default_rng(11)
    base = rng.uniform(-6, 6, size=15).astype(np.float32)
    x = np.tile(np.concatenate([[6.0], base]).astype(np.float32), (40000, 1))
    codes, _ = nvfp4.quantize(x, ONE, "sr", seed=9, step=3)
    mean = F.e2m1_decode(codes[:, 1:]).mean(axis=0)
    assert np.all(np.abs(mean - base) < 4 * 1.0 / np.sqrt(40000))


def test_rtn_with_error_feedback_time_average_is_2_297():
    # bf16 input 2.3 (= 2.296875), constant; RTN + EF; running mean of the output
    x = _anchored(1, F.bf16_bits_to_f32(np.array([0x4013], np.uint16))[0])
    assert x[0, 1] == np.float32(2.296875)
    r = np.zeros_like(x)
    outs = []
    for step in range(4000):
        ob, r, _, _, _ = nvfp4.errfeedback_qdq(x, r, ONE, "rtn", step=step)
        outs.append(F.bf16_bits_to_f32(ob)[0, 1])
    outs = np.array(outs, dtype=np.float64)
    assert outs[:6].tolist() == [2, 3, 2, 2, 2, 3]
    assert f"{outs.mean():.3f}" == C["ef_time_average_of_2.3"][0]
    # without feedback round-to-nearest stays at 2
    ob, _, _, _, _ = nvfp4.errfeedback_qdq(x, None, ONE, "rtn")
    assert F.bf16_bits_to_f32(ob)[0, 1] == 2.0


def _accumulate(mode, steps=100, inc=0.01, rows=4096):
    w = _anchored(rows, np.float32(0.5))
    r = np.zeros_like(w) if mode != "none" else None
    rounding = "rtn" if mode in ("none", "ef") else "sr"
    res = None if mode == "sr" else r
    for step in range(steps):
        x = (w + np.where(np.arange(16) == 0, 0, np.float32(inc))).astype(np.float32)
        ob, res_new, _, _, _ = nvfp4.errfeedback_qdq(x, res, ONE, rounding, seed=5, step=step,
                                                     out="f32")
        w = ob
        res = res_new if res is not None else None
    return w[:, 1:]


def test_sub_ulp_accumulation():
    target = float(C["subulp_target"][0])
    assert np.all(_accumulate("none") == float(C["subulp_rtn"][0]))        # RTN stalls
    ef = _accumulate("ef", rows=4)
    assert np.all(ef == float(C["subulp_ef"][0]))                         # EF recovers exactly
    sr = _accumulate("sr")
    assert f"{sr.mean():.2f}" == C["subulp_sr"][0]
    assert abs(sr.mean() - target) < 0.01


def test_error_feedback_telescopes():
    rng = np.random.default_rng(2)
    x0 = rng.normal(0, 0.02, size=(64, 64)).astype(np.float32)
    r = np.zeros_like(x0)
    r0 = r.copy()
    tot_in = np.zeros(x0.shape)
    tot_out = np.zeros(x0.shape)
    for step in range(20):
        x = (x0 + np.float32(1e-4) * rng.standard_normal(x0.shape).astype(np.float32)).astype(np.float32)
        ob, r, _, _, _ = nvfp4.errfeedback_qdq(x, r, None, "sr", seed=4, step=step)
        tot_in += x
        tot_out += F.bf16_bits_to_f32(ob)
    lhs = tot_out
    rhs = tot_in + r0 - r
    assert np.max(np.abs(lhs - rhs)) < 20 * 2.0 ** -24 * 0.2


def test_tensor_and_block_scale_reach_the_top():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 0.02, size=(32, 64)).astype(np.float32)
    x[5, 7] = 1.21
    st = nvfp4.tensor_scale(x)
    assert st == np.float32(np.float32(1.21) / np.float32(2688))
    codes, sc = nvfp4.quantize(x, st)
    assert sc[5, 0] == 0x7E                                 # 448: the largest e4m3
    assert F.e2m1_decode(codes[5, 7]) == 6.0
    assert nvfp4.tensor_scale(np.zeros((2, 16), np.float32)) == 1.0


def test_zero_scale_block_keeps_sign():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    x[0, 16:] = -1e-30                                      # block scale underflows to 0
    codes, sc = nvfp4.quantize(x, nvfp4.tensor_scale(x))
    assert sc[0, 1] == 0 and np.all(codes[0, 16:] == 8)


def test_sampled_rows_use_global_indices():
    rng = np.random.default_rng(12)
    x = rng.normal(size=(40, 64)).astype(np.float32)
    st = nvfp4.tensor_scale(x)
    full, _ = nvfp4.quantize(x, st, "sr", seed=7, step=3)
    rows = np.array([0, 5, 39])
    part, _ = nvfp4.quantize(x[rows], st, "sr", seed=7, step=3, row_ids=rows)
    np.testing.assert_array_equal(part, full[rows])


def test_sr_stream_depends_only_on_the_flat_index():
    """The SR draws are keyed by (seed, step, global index), the row-major
    position of the element in the tensor, so the codes of an [R, C] tensor
    are those of the same data seen as [1, R C] or [R / 2, 2 C]: the row pitch
    of the index is the row length."""
    rng = np.random.default_rng(21)
    R, C = 6, 64
    x = (rng.standard_normal((R, C)) * 3).astype(np.float32)
    st = nvfp4.tensor_scale(x)
    c, s = nvfp4.quantize(x, st, "sr", seed=5, step=9)
    for shape in ((1, R * C), (R // 2, 2 * C)):
        c2, s2 = nvfp4.quantize(x.reshape(shape), st, "sr", seed=5, step=9)
        np.testing.assert_array_equal(c2.reshape(R, C), c)
        np.testing.assert_array_equal(s2.reshape(-1), s.reshape(-1))
    assert not np.array_equal(nvfp4.quantize(x, st, "sr", seed=6, step=9)[0], c)
