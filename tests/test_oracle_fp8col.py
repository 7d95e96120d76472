"""Pins of the MXFP4-row -> FP8-column and -> FP8-row converters (MoE
report, "核心技术贡献" items 1-3) -- CPU only."""
import numpy as np
import torch

import synth
from oracle import formats as F
from oracle import fp8col, mxfp4


def test_lossless_when_shift_at_most_8_and_layout():
    H = 256
    counts = np.array([3, 0, 5, 1, 0])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    rng = np.random.default_rng(0)
    packed = rng.integers(0, 256, size=(T, H // 2), dtype=np.uint8)
    sb = rng.integers(120, 129, size=(T, H // 32), dtype=np.uint8)   # d <= 8
    out, sc = fp8col.convert(packed, sb, off, H)
    codes = F.unpack_codes(packed)
    for e in range(counts.size):
        a, n = int(off[e]), int(counts[e])
        blk = out[H * a: H * (a + n)].reshape(H, n)
        scl = sc[(H // 128) * a: (H // 128) * (a + n)].reshape(H // 128, n)
        for t in range(n):
            for h in range(H):
                v_in = F.e2m1_decode(codes[a + t, h]) * 2.0 ** (int(sb[a + t, h // 32]) - 127)
                v_out = F.e4m3_decode(blk[h, t]) * float(scl[h // 128, t])
                assert v_in == v_out
                assert (blk[h, t] >> 7) == (codes[a + t, h] >> 3)


def test_all_code_shift_pairs_match_torch_rne():
    # every (code, d) with d = 0..254: value e2m1 * 2**-d rounded to e4m3
    H = 128
    rows = []
    for d in range(255):
        s = np.zeros(4, np.uint8)
        s[0] = 254                      # target 254 in sub-block 0
        s[1] = 254 - d                  # sub-block 1 shifted by d
        rows.append(s)
    sb = np.array(rows, np.uint8)
    T = sb.shape[0]
    codes = np.tile(np.arange(16, dtype=np.uint8), (T, H // 16))
    out, _ = fp8col.convert(F.pack_codes(codes), sb, np.array([0, T], np.int64), H)
    blk = out.reshape(H, T)
    for d in range(255):
        vals = F.e2m1_decode(np.arange(16)) * 2.0 ** -d
        ref = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = blk[32:48, d]             # sub-block 1, codes 0..15
        np.testing.assert_array_equal(got, ref)


def test_stepwise_equivalence_on_quantized_activations():
    counts, off = synth.expert_counts(tokens=300, experts=7, seed=9)
    x = synth.expert_activations(tokens=300, hidden=384, seed=9)
    packed, sb = mxfp4.quantize_packed(F.bf16_bits_to_f32(x))
    out, sc = fp8col.convert(packed, sb, off, 384)
    # stepwise: FP4 -> float -> (divide by the block target) -> FP8
    deq = mxfp4.dequantize_f32(F.unpack_codes(packed), sb).astype(np.float64)
    for e in range(7):
        a, b = int(off[e]), int(off[e + 1])
        n = b - a
        tgt = sb[a:b].reshape(n, 3, 4).max(axis=2).astype(np.float64)
        scale = np.repeat(np.exp2(tgt - 127), 128, axis=1)
        ref = torch.from_numpy((deq[a:b] / scale).astype(np.float32)).to(torch.float8_e4m3fn)
        ref = ref.view(torch.uint8).numpy().T.reshape(-1)
        np.testing.assert_array_equal(out[384 * a: 384 * b], ref)


def test_rows_are_the_columns_untransposed():
    """The row converter and the (separately pinned) column converter give
    the same FP8 bytes and scales, one per-expert transpose apart."""
    rng = np.random.default_rng(4)
    H = 384
    counts = np.array([7, 0, 1, 30, 2])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    packed = rng.integers(0, 256, size=(T, H // 2), dtype=np.uint8)
    sb = rng.integers(100, 140, size=(T, H // 32), dtype=np.uint8)
    ro, rs = fp8col.convert_rows(packed, sb, H)
    co, cs = fp8col.convert(packed, sb, off, H)
    assert ro.shape == (T, H) and rs.shape == (T, H // 128)
    for e in range(counts.size):
        a, n = int(off[e]), int(counts[e])
        np.testing.assert_array_equal(co[H * a: H * (a + n)].reshape(H, n), ro[a:a + n].T)
        np.testing.assert_array_equal(cs[(H // 128) * a: (H // 128) * (a + n)].reshape(H // 128, n),
                                      rs[a:a + n].T)


def test_rows_lossless_when_shift_at_most_8():
    """value * scale is unchanged for every element whose shift d <= 8."""
    rng = np.random.default_rng(5)
    T, H = 6, 256
    packed = rng.integers(0, 256, size=(T, H // 2), dtype=np.uint8)
    sb = rng.integers(120, 129, size=(T, H // 32), dtype=np.uint8)
    out, sc = fp8col.convert_rows(packed, sb, H)
    v_in = F.e2m1_decode(F.unpack_codes(packed)) * np.exp2(np.repeat(sb.astype(np.float64) - 127, 32, axis=1))
    v_out = F.e4m3_decode(out) * np.repeat(sc.astype(np.float64), 128, axis=1)
    np.testing.assert_array_equal(v_in, v_out)
    # FP8 rows with 4-byte scales per 128 values: (1 + 4/128) bytes per value,
    # the MoE report's 1.03 M K ("通信量")
    assert (out.nbytes + sc.nbytes) / (T * H) == 1 + 4 / 128


# ---- FP8 blocks along the tokens (the alternative FP8-column reading) ----

def _token_block_case(seed, H=128, counts=(0, 130, 5, 128, 1, 257, 0), lo=100, hi=141):
    counts = np.asarray(counts, np.int64)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, size=(T, H // 2), dtype=np.uint8)
    sb = rng.integers(lo, hi, size=(T, H // 32), dtype=np.uint8)
    return counts, off, packed, sb


def test_token_blocks_brute_force_against_torch_rne():
    # every value by explicit loops over (expert, channel, token block): the
    # target is the largest UE8M0 byte of the block's tokens for the channel's
    # 32-channel group, the value e2m1 * 2**-(target - own byte) is rounded by
    # torch's float8_e4m3fn cast, the scale is 2**(target - 127)
    H = 128
    counts, off, packed, sb = _token_block_case(3, H)
    out, sc, written = fp8col.convert_token_blocks(packed, sb, off, H)
    codes = F.unpack_codes(packed)
    E = counts.size
    for e in range(E):
        a, n = int(off[e]), int(counts[e])
        if n == 0:
            continue
        nb = (n + 127) // 128
        base = H * ((int(off[e]) + 127) // 128 + e)
        blk = out[H * a: H * (a + n)].reshape(H, n)
        for h in range(H):
            for j in range(nb):
                toks = range(128 * j, min(128 * j + 128, n))
                target = max(int(sb[a + u, h // 32]) for u in toks)
                assert sc[base + h * nb + j] == np.float32(2.0 ** (target - 127))
                assert written[base + h * nb + j]
                vals = np.array([F.e2m1_decode(codes[a + u, h]) * 2.0 ** -(target - int(sb[a + u, h // 32]))
                                 for u in toks], np.float32)
                ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                np.testing.assert_array_equal(blk[h, 128 * j: 128 * j + len(toks)], ref)
    assert written.sum() == sum(H * ((int(n) + 127) // 128) for n in counts)


def test_token_blocks_lossless_when_shift_at_most_8():
    H = 256
    counts, off, packed, sb = _token_block_case(4, H, counts=(200, 3, 0, 129), lo=120, hi=129)
    out, sc, _ = fp8col.convert_token_blocks(packed, sb, off, H)
    codes = F.unpack_codes(packed)
    for e in range(counts.size):
        a, n = int(off[e]), int(counts[e])
        if n == 0:
            continue
        nb = (n + 127) // 128
        base = H * ((a + 127) // 128 + e)
        blk = out[H * a: H * (a + n)].reshape(H, n)
        scl = sc[base: base + H * nb].reshape(H, nb)
        t = np.arange(n)
        for h in range(0, H, 7):
            v_in = F.e2m1_decode(codes[a + t, h]) * np.exp2(sb[a + t, h // 32].astype(np.float64) - 127)
            v_out = F.e4m3_decode(blk[h]) * scl[h, t // 128].astype(np.float64)
            np.testing.assert_array_equal(v_in, v_out)
            # the target is attained: some token of every block keeps its exponent (d = 0)
            for j in range(nb):
                seg = sb[a + 128 * j: a + min(128 * j + 128, n), h // 32]
                assert scl[h, j] == np.float32(2.0 ** (int(seg.max()) - 127))


def test_token_blocks_partial_block_sees_only_its_tokens():
    # a shard of 130 tokens: the last two form a block of their own, and a large
    # byte there must not reach the first block (which equals a shard of 128)
    H = 128
    counts, off, packed, sb = _token_block_case(5, H, counts=(130,), lo=110, hi=120)
    sb[129, :] = 200
    out, sc, _ = fp8col.convert_token_blocks(packed, sb, off, H)
    out128, sc128, _ = fp8col.convert_token_blocks(packed[:128], sb[:128], np.array([0, 128]), H)
    np.testing.assert_array_equal(out.reshape(H, 130)[:, :128], out128.reshape(H, 128))
    np.testing.assert_array_equal(sc[:H * 2].reshape(H, 2)[:, 0], sc128[:H])
    assert np.all(sc[:H * 2].reshape(H, 2)[:, 1] == np.float32(2.0 ** (200 - 127)))


def test_token_block_scale_matrices_are_disjoint_and_inside_the_buffer():
    H = 128
    rng = np.random.default_rng(6)
    for trial in range(200):
        E = int(rng.integers(1, 40))
        # a mix of empty, tiny and multi-block shards
        counts = np.where(rng.random(E) < 0.5, rng.integers(0, 4, size=E), rng.integers(0, 400, size=E))
        off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        T = int(off[-1])
        base = fp8col.token_block_scale_offset(off, H)
        size = H * ((T + 127) // 128 + E)
        ends = base[:-1] + H * ((counts + 127) // 128)
        assert base[0] == 0 and np.all(ends <= size)
        nz = counts > 0
        starts, stops = base[:-1][nz], ends[nz]
        assert np.all(stops[:-1] <= starts[1:]), (counts, base)
