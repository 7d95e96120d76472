"""Tensors past 32-bit element counts on one GPU (HBM holds them): byte
offsets above 2^32 in the quantize / dequantize kernels, and stochastic-
rounding counters whose high word is non-zero (elements at or above 2^34,
the general Philox counter path).  Inputs are generated on the device in
row chunks; sampled rows, including the last ones, are checked bit for bit
against the oracle."""
import numpy as np
import pytest
import torch

from gpu_util import host, host_bf16, need_gpu
from oracle import formats as F
from oracle import mxfp4, nvfp4

pytestmark = pytest.mark.gpu


def _need_memory(nbytes):
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < 1.2 * nbytes:
        pytest.skip(f"needs {nbytes / 2**30:.0f} GiB of free device memory")


def _fill(rows, cols, seed):
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    step = 1 << 14
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x[r0:r1] = (torch.randn((r1 - r0, cols), generator=g, device="cuda") * 1.5).to(torch.bfloat16)
    return x


def _rows(x, ids):
    return F.bf16_bits_to_f32(host_bf16(x[torch.tensor(ids, device="cuda")]))


def test_mxfp4_roundtrip_past_2_32_elements():
    m = need_gpu()
    R, C = (1 << 17) + 3, 1 << 15                      # 2^32 + 98,304 elements, 8 GiB bf16
    _need_memory(R * C * (2 + 0.5 + 2))
    x = _fill(R, C, 11)
    p, s, _ = m.fp4_quantize(x, "mxfp4", "rtn")
    y = m.fp4_dequantize(p, s, R, C, "mxfp4")
    torch.cuda.synchronize()
    ids = [0, 1, R // 2, R - 3, R - 2, R - 1]
    xs = _rows(x, ids)
    rp, rs = mxfp4.quantize_packed(xs)
    np.testing.assert_array_equal(host(p[torch.tensor(ids, device="cuda")]), rp)
    np.testing.assert_array_equal(host(s[torch.tensor(ids, device="cuda")]), rs)
    np.testing.assert_array_equal(host_bf16(y[torch.tensor(ids, device="cuda")]),
                                  mxfp4.dequantize(rp, rs, "bf16"))


def test_nvfp4_sr_counters_past_2_34_elements():
    m = need_gpu()
    R, C = (1 << 19) + 64, 1 << 15                     # 2^34 + 2^21 elements, 32 GiB bf16
    _need_memory(R * C * (2 + 0.5 + 1 / 16))
    x = _fill(R, C, 12)
    st = np.float32(4.5 / 2688)
    ts = torch.tensor([st], dtype=torch.float32, device="cuda")
    seed, step = 0x0123456789ABCDEF, (1 << 33) + 5
    p, s, _ = m.fp4_quantize(x, "nvfp4", "sr", seed=seed, step=step, tscale="given",
                             tensor_scale=ts)
    torch.cuda.synchronize()
    ids = [0, R // 3, R - 65, R - 64, R - 2, R - 1]     # the last 64 rows lie past 2^34
    xs = _rows(x, ids)
    rp, rs = nvfp4.quantize_packed(xs, st, "sr", seed=seed, step=step, row_ids=ids)
    np.testing.assert_array_equal(host(s[torch.tensor(ids, device="cuda")]), rs)
    np.testing.assert_array_equal(host(p[torch.tensor(ids, device="cuda")]), rp)
