"""GPU parity of fp4_errfeedback_qdq against the oracle, step by step
(bit-exact output, residual, packed codes, scales and tensor scale)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import Guarded, dev_bf16, dev_f32, host, host_bf16, need_gpu
from oracle import formats as F
from oracle import nvfp4

pytestmark = pytest.mark.gpu


def _ef_run(m, x_host, xdtype, r_dev, step, rounding, seed, out_dtype, tscale="compute", st=None,
            codes=True):
    rows, cols = x_host.shape
    x_dev = dev_bf16(x_host) if xdtype == "bf16" else dev_f32(x_host)
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    gy = Guarded(rows * cols * (2 if out_dtype == "bf16" else 4))
    y = gy.view(od, (rows, cols))
    ts = dev_f32(np.array([st if st is not None else 0.0], np.float32))
    gp = Guarded(rows * cols // 2) if codes else None
    gs = Guarded(rows * cols // 16) if codes else None
    m.fp4_errfeedback_qdq(x_dev, r_dev, y, None, rounding, seed, step, tscale, ts,
                          gp.view(torch.uint8, (rows, cols // 2)) if codes else None,
                          gs.view(torch.uint8, (rows, cols // 16)) if codes else None)
    torch.cuda.synchronize()
    for g in (gy, gp, gs):
        if g is not None:
            g.check()
    yh = host_bf16(y) if out_dtype == "bf16" else host(y)
    return (yh, host(ts)[0], host(gp.view(torch.uint8, (rows, cols // 2))) if codes else None,
            host(gs.view(torch.uint8, (rows, cols // 16))) if codes else None)


@pytest.mark.parametrize("rounding", ["sr", "rtn"])
@pytest.mark.parametrize("xdtype,out_dtype", [("bf16", "bf16"), ("f32", "f32"), ("f32", "bf16")])
def test_ef_ten_steps_small(rounding, xdtype, out_dtype):
    """The in-place NVFP4 weight loop of the workload at 192 x 1024: each step
    adds fl32(1e-4 g) to the stored weight and runs qdq with the residual.
    Even steps also return the codes (the tensor-scale pass keeps its partial
    maxima in the packed output), odd steps do not (it keeps them in y)."""
    m = need_gpu()
    rows, cols = 192, 1024
    wb = synth.ef_weight(rows, cols, seed=4)
    w = F.bf16_bits_to_f32(wb)
    r_ref = np.zeros((rows, cols), np.float32)
    r_dev = torch.zeros((rows, cols), dtype=torch.float32, device="cuda")
    for step in range(10):
        u = synth.ef_update(rows, cols, seed=4, step=step)
        x = (w + u).astype(np.float32)
        x_host = synth.to_bf16_bits(x) if xdtype == "bf16" else x
        x32 = F.bf16_bits_to_f32(x_host) if xdtype == "bf16" else x
        codes = step % 2 == 0
        y, ts, p, s = _ef_run(m, x_host, xdtype, r_dev, step, rounding, 4, out_dtype, codes=codes)
        oy, r_ref, op, osc, ost = nvfp4.errfeedback_qdq(x32, r_ref, None, rounding, seed=4, step=step,
                                                       out=out_dtype)
        assert np.float32(ts) == ost, step
        if codes:
            np.testing.assert_array_equal(s, osc)
            np.testing.assert_array_equal(p, op)
        if out_dtype == "bf16":
            np.testing.assert_array_equal(y, oy)
            w = F.bf16_bits_to_f32(y)
        else:
            np.testing.assert_array_equal(y.view(np.uint32), oy.view(np.uint32))
            w = y
        np.testing.assert_array_equal(host(r_dev).view(np.uint32), r_ref.view(np.uint32))


def test_ef_in_place_and_without_residual():
    m = need_gpu()
    rows, cols = 64, 512
    xb = synth.ef_weight(rows, cols, seed=8)
    x = dev_bf16(xb)
    r = torch.zeros((rows, cols), dtype=torch.float32, device="cuda")
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    m.fp4_errfeedback_qdq(x, r, x, None, "sr", 9, 1, "compute", ts)        # y is x
    torch.cuda.synchronize()
    oy, orr, _, _, _ = nvfp4.errfeedback_qdq(F.bf16_bits_to_f32(xb), np.zeros((rows, cols), np.float32),
                                             None, "sr", seed=9, step=1)
    np.testing.assert_array_equal(host_bf16(x), oy)
    np.testing.assert_array_equal(host(r).view(np.uint32), orr.view(np.uint32))
    # residual NULL: plain qdq, given scale
    y, ts2, p, s = _ef_run(m, xb, "bf16", None, 0, "rtn", 0, "bf16", "given", 1e-4, codes=False)
    oy2, _, _, _, _ = nvfp4.errfeedback_qdq(F.bf16_bits_to_f32(xb), None, np.float32(1e-4), "rtn")
    np.testing.assert_array_equal(y, oy2)
