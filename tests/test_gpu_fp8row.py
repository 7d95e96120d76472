"""GPU parity of mxfp4_row_to_fp8_row against the oracle (bit-exact FP8
bytes and fp32 scales, guard bands)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import Guarded, dev_u8, host, need_gpu
from oracle import formats as F
from oracle import fp8col, mxfp4

pytestmark = pytest.mark.gpu


def convert_gpu(m, packed, sb, H):
    T = packed.shape[0]
    go, gs = Guarded(T * H), Guarded(T * H // 128 * 4)
    o, s = m.mxfp4_row_to_fp8_row(dev_u8(packed), dev_u8(sb), H,
                                  go.view(torch.uint8, (T, H)), gs.view(torch.float32, (T, H // 128)))
    torch.cuda.synchronize()
    go.check()
    gs.check()
    return host(o), host(s)


@pytest.mark.parametrize("T,H", [(1, 128), (3, 384), (37, 7168), (515, 256), (2048, 1024)])
def test_rows_from_quantized_activations(T, H):
    m = need_gpu()
    x = synth.expert_activations(tokens=T, hidden=H, seed=T + H)
    packed, sb = mxfp4.quantize_packed(F.bf16_bits_to_f32(x))
    o, s = convert_gpu(m, packed, sb, H)
    ro, rs = fp8col.convert_rows(packed, sb, H)
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(s.view(np.uint32), rs.view(np.uint32))


def test_every_code_and_shift():
    """All 16 codes under every shift d = 0..254 of sub-block 1 (and smaller
    shifts of sub-blocks 2, 3)."""
    m = need_gpu()
    H = 128
    sb = np.zeros((255, 4), np.uint8)
    for d in range(255):
        sb[d] = (254, 254 - d, 254 - min(d, 3), 200)
    codes = np.tile(np.arange(16, dtype=np.uint8), (255, H // 16))
    packed = F.pack_codes(codes)
    o, s = convert_gpu(m, packed, sb, H)
    ro, rs = fp8col.convert_rows(packed, sb, H)
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(s.view(np.uint32), rs.view(np.uint32))


def test_empty_is_noop():
    m = need_gpu()
    p = torch.empty((0, 64), dtype=torch.uint8, device="cuda")
    s = torch.empty((0, 4), dtype=torch.uint8, device="cuda")
    o, sc = m.mxfp4_row_to_fp8_row(p, s, 128)
    assert o.numel() == 0 and sc.numel() == 0
