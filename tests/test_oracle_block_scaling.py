"""Pins of block scaling against the worked example of "weight precision
part 2" ("Sixteen values aren't enough", "Block scaling") -- CPU only."""
import numpy as np

from conftest import read_golden
from oracle import formats as F
from oracle import mxfp4, nvfp4

G = read_golden("block_scaling_example.txt")
W = np.array([float(t) for t in G["weights"]], dtype=np.float32)


def _f(key):
    return [float(t) for t in G[key]]


def test_straight_to_fp4_loses_every_weight():
    codes = F.e2m1_rtn(W)
    assert list(np.abs(F.e2m1_decode(codes))) == _f("straight_fp4")
    t = np.float32(float(G["zero_threshold"][0]))
    assert F.e2m1_decode(F.e2m1_rtn(t)) == 0.0
    assert F.e2m1_decode(F.e2m1_rtn(np.nextafter(t, np.float32(1)))) == 0.5


def test_block_of_four_with_unencoded_scale():
    amax = np.max(np.abs(W))
    assert round(float(amax), 4) == _f("block_absmax")[0]
    s = np.float32(amax / np.float32(6))
    assert round(float(s), 5) == _f("block_scale")[0]
    q = (W / s).astype(np.float32)
    assert [round(float(v), 2) for v in q] == _f("block_quotients")
    codes = F.e2m1_rtn(q)
    assert list(F.e2m1_decode(codes)) == _f("block_rounded")
    rec = F.e2m1_decode(codes) * float(s)
    assert [float(f"{v:.3g}") for v in rec] == _f("block_recovered")
    err = np.abs(rec - W.astype(np.float64)) / np.abs(W.astype(np.float64)) * 100
    assert [int(round(e)) for e in err] == [int(v) for v in _f("block_error_pct")]


def test_block_of_four_as_nvfp4_block_gives_same_codes():
    # the same four weights inside one 16-element NVFP4 block (rest zero),
    # tensor scale 1: the e4m3 scale is 0.00785 -> 4 * 2**-9 = 0.0078125
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, :4] = W
    codes, sc = nvfp4.quantize(x, np.float32(1.0))
    assert sc[0, 0] == 0x04 and F.e4m3_decode(sc[0, 0]) == 0.0078125
    assert list(F.e2m1_decode(codes[0, :4])) == _f("block_rounded")
    assert np.all(codes[0, 4:] == 0)


def test_one_scale_per_matrix_loses_the_block():
    amax = np.float32(_f("matrix_absmax")[0])
    s = np.float32(amax / np.float32(6))
    assert round(float(s), 4) == _f("matrix_scale")[0]
    q = (W / s).astype(np.float32)
    assert [round(float(v), 2) for v in q] == _f("matrix_quotients")
    assert list(np.abs(F.e2m1_decode(F.e2m1_rtn(q)))) == _f("matrix_rounded")


def test_bits_per_value_of_both_layouts():
    sizes = read_golden("format_sizes.txt")
    x = np.random.default_rng(0).normal(size=(8, 256)).astype(np.float32)
    p, sb = mxfp4.quantize_packed(x)
    assert (p.nbytes + sb.nbytes) * 8 / x.size == float(sizes["mxfp4_bits_per_value"][0])
    p, sb = nvfp4.quantize_packed(x, nvfp4.tensor_scale(x))
    assert (p.nbytes + sb.nbytes) * 8 / x.size == float(sizes["nvfp4_bits_per_value"][0])
