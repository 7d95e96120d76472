"""GPU parity of mxfp4_row_to_fp8_col against the oracle (bit-exact FP8
bytes and fp32 scales, ragged expert shards, guard bands)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import Guarded, dev_i64, dev_u8, host, need_gpu
from oracle import formats as F
from oracle import fp8col, mxfp4

pytestmark = pytest.mark.gpu


def convert_gpu(m, packed, sb, off, H):
    T = packed.shape[0]
    go, gs = Guarded(T * H), Guarded(T * H // 128 * 4)
    o, s = m.mxfp4_row_to_fp8_col(dev_u8(packed), dev_u8(sb), dev_i64(off), H,
                                  go.view(torch.uint8, (T * H,)), gs.view(torch.float32, (T * H // 128,)))
    torch.cuda.synchronize()
    go.check()
    gs.check()
    return host(o), host(s)


@pytest.mark.parametrize("counts,H", [
    ([3, 0, 5, 1, 0, 64, 130, 0, 7], 384),
    ([0, 0, 1], 128),
    ([64, 64, 64], 256),
    ([200], 7168),
    ([1009, 3, 2020, 0, 1007, 4, 1], 256),               # pieces across token chunks
    ([5001], 128),
])
def test_small_ragged_from_quantized_activations(counts, H):
    m = need_gpu()
    counts = np.array(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    x = synth.expert_activations(tokens=T, hidden=H, seed=int(T + H))
    packed, sb = mxfp4.quantize_packed(F.bf16_bits_to_f32(x))
    o, s = convert_gpu(m, packed, sb, off, H)
    ro, rs = fp8col.convert(packed, sb, off, H)
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(s.view(np.uint32), rs.view(np.uint32))


def test_every_code_and_shift():
    m = need_gpu()
    H = 128
    rows = []
    for d in range(255):
        r = np.zeros(4, np.uint8)
        r[0], r[1], r[2], r[3] = 254, 254 - d, 254 - min(d, 3), 200
        rows.append(r)
    sb = np.array(rows, np.uint8)
    T = sb.shape[0]
    codes = np.tile(np.arange(16, dtype=np.uint8), (T, H // 16))
    packed = F.pack_codes(codes)
    off = np.array([0, 100, 100, T], np.int64)
    o, s = convert_gpu(m, packed, sb, off, H)
    ro, rs = fp8col.convert(packed, sb, off, H)
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(s.view(np.uint32), rs.view(np.uint32))


def test_many_empty_experts_inside_one_tile():
    m = need_gpu()
    H = 256
    counts = np.zeros(500, np.int64)
    counts[[3, 100, 101, 250, 499]] = [10, 5, 1, 40, 90]
    counts[400:470] = 1                                   # 70 one-token experts in one tile
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    packed, sb = synth.random_mxfp4(T, H, seed=3)
    o, s = convert_gpu(m, packed, sb, off, H)
    ro, rs = fp8col.convert(packed, sb, off, H)
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(s.view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("E", [2047, 2048, 2600])
def test_expert_table_in_lds_and_in_global_memory(E):
    """Up to 2047 experts the expert lookups read a table in LDS, beyond that
    global memory; both sides of the switch, with many tiny and empty
    experts (so that tiles meet many experts) and an odd block count."""
    m = need_gpu()
    H = 384
    rng = np.random.default_rng(E)
    counts = rng.integers(0, 7, size=E)
    counts[rng.choice(E, 12, replace=False)] = rng.integers(200, 600, size=12)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    packed, sb = synth.random_mxfp4(T, H, seed=E)
    o, s = convert_gpu(m, packed, sb, off, H)
    ro, rs = fp8col.convert(packed, sb, off, H)
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(s.view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("counts,H", [
    ([255, 1, 256, 257, 17, 16, 15, 240, 512], 640),      # experts ending on and off 256-seams
    ([511, 1, 512, 513, 33, 32, 31, 496, 1024], 384),     # and on and off 512-position seams
    ([8200], 256),                                        # one expert over 17 tiles
])
def test_tile_seams(counts, H):
    m = need_gpu()
    counts = np.array(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    packed, sb = synth.random_mxfp4(T, H, seed=T)
    o, s = convert_gpu(m, packed, sb, off, H)
    ro, rs = fp8col.convert(packed, sb, off, H)
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(s.view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("off", [
    [0, 50, 20, 90, 90],
    [0, 300, 1000, 40, 600],
    [-30, 10, 10, 600, 5000],
    [400, 100, 0, 600],
])
def test_malformed_offsets_stay_in_bounds(off):
    """Offsets that are not ascending or leave [0, T] are clamped on the
    device (the header leaves the outputs unspecified): the call completes
    and nothing is written outside the two output buffers.  The index
    arithmetic for these inputs is checked on the CPU in
    test_fp8col_index_model.py."""
    m = need_gpu()
    T, H = 600, 384
    packed, sb = synth.random_mxfp4(T, H, seed=9)
    convert_gpu(m, packed, sb, np.array(off, np.int64), H)    # guard bands checked inside


# ---- FP8 blocks of 128 tokens per channel (mxfp4_row_to_fp8_col_tokblk) ----

def convert_tokblk_gpu(m, packed, sb, off, H):
    """The library's token-block conversion into canary-filled buffers; also
    returns the raw scale words so that unwritten entries can be checked."""
    T, E = packed.shape[0], off.size - 1
    nsc = m.tokblk_scale_count(T, E, H)
    go, gs = Guarded(T * H), Guarded(nsc * 4)
    o, s = m.mxfp4_row_to_fp8_col_tokblk(dev_u8(packed), dev_u8(sb), dev_i64(off), H,
                                         go.view(torch.uint8, (T * H,)), gs.view(torch.float32, (nsc,)))
    torch.cuda.synchronize()
    go.check()
    gs.check()
    return host(o), host(s)


def check_tokblk(m, packed, sb, off, H):
    o, s = convert_tokblk_gpu(m, packed, sb, off, H)
    ro, rs, written = fp8col.convert_token_blocks(packed, sb, off, H)
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(s.view(np.uint32)[written], rs.view(np.uint32)[written])
    # entries between the experts' scale matrices are left as they were
    assert np.all(s.view(np.uint32)[~written] == 0xA5A5A5A5)


@pytest.mark.parametrize("counts,H", [
    ([3, 0, 5, 1, 0, 64, 130, 0, 7], 384),
    ([0, 0, 1], 128),
    ([128, 127, 129, 256, 255, 257], 256),                # blocks ending on and off 128
    ([200], 7168),
    ([1009, 3, 2020, 0, 1007, 4, 1], 256),
    ([511, 1, 512, 513, 33, 32, 31, 496, 1024], 384),     # 512-position tile seams
    ([8200], 128),
])
def test_tokblk_small_ragged_from_quantized_activations(counts, H):
    m = need_gpu()
    counts = np.array(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    x = synth.expert_activations(tokens=T, hidden=H, seed=int(T + H + 1))
    packed, sb = mxfp4.quantize_packed(F.bf16_bits_to_f32(x))
    check_tokblk(m, packed, sb, off, H)


def test_tokblk_random_scales_wide_shifts():
    """Uniformly random code bytes and scale bytes in [80, 200]: shifts inside
    a block of 128 tokens reach 120 (values far below the E4M3 range)."""
    m = need_gpu()
    H = 640
    counts = np.array([300, 1, 0, 129, 77, 1000])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    packed, sb = synth.random_mxfp4(int(off[-1]), H, seed=12, scale_lo=80, scale_hi=200)
    check_tokblk(m, packed, sb, off, H)


def test_tokblk_many_empty_experts_between_blocks():
    """Experts with no tokens take no 128-position slot in the dense layout,
    so long runs of them share one start: 80 empty experts between two
    blocks of one tile, empty experts at both ends, and one-token experts
    that each fill a slot."""
    m = need_gpu()
    H = 256
    counts = np.zeros(600, np.int64)
    counts[[5, 86, 87, 300, 598]] = [100, 60, 1, 129, 3]
    counts[400:470] = 1                                   # 70 one-token experts, 70 slots
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    packed, sb = synth.random_mxfp4(int(off[-1]), H, seed=21)
    check_tokblk(m, packed, sb, off, H)


@pytest.mark.parametrize("E", [2047, 2048, 2600])
def test_tokblk_expert_table_in_lds_and_in_global_memory(E):
    m = need_gpu()
    H = 384
    rng = np.random.default_rng(E + 1)
    counts = rng.integers(0, 7, size=E)
    counts[rng.choice(E, 12, replace=False)] = rng.integers(200, 600, size=12)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    packed, sb = synth.random_mxfp4(int(off[-1]), H, seed=E + 1)
    check_tokblk(m, packed, sb, off, H)


@pytest.mark.parametrize("off", [
    [0, 50, 20, 90, 90],
    [-30, 10, 10, 600, 5000],
    [400, 100, 0, 600],
])
def test_tokblk_malformed_offsets_stay_in_bounds(off):
    """Offsets that are not ascending or leave [0, T] are clamped on the
    device: the call completes and nothing is written outside the outputs.
    Clamped offsets are nondecreasing-or-not values in [0, T], so every
    padded position stays below 128 (ceil(T / 128) + E) and every scale
    index below H (ceil(T / 128) + E)."""
    m = need_gpu()
    T, H = 600, 384
    packed, sb = synth.random_mxfp4(T, H, seed=10)
    convert_tokblk_gpu(m, packed, sb, np.array(off, np.int64), H)
