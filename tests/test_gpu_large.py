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
    # the fp32 receiver too (16 GiB of output, quads past index 2^31)
    del y, x
    _need_memory(R * C * 4)
    yf = m.fp4_dequantize(p, s, R, C, "mxfp4", None, torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(yf[torch.tensor(ids, device="cuda")]).view(np.uint32),
                                  np.asarray(mxfp4.dequantize(rp, rs, "f32"), np.float32).view(np.uint32))


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


def test_fp8_rows_and_columns_past_2_32_output_bytes():
    """655,360 tokens x 7168 in 256 Zipf(1.1) experts: 4.7 GB of FP8 output,
    so the late experts' rows sit past byte 2^32; columns with FP8 blocks of
    128 channels and of 128 tokens, and rows."""
    import synth
    from oracle import fp8col
    m = need_gpu()
    T, H, E = 655360, 7168, 256
    _need_memory(T * H * (0.5 + 1 / 32 + 2 + 2 / 32))
    counts, off = synth.expert_counts(T, E, seed=7)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    packed = torch.randint(0, 256, (T, H // 2), generator=g, device="cuda", dtype=torch.uint8)
    sb = torch.randint(110, 141, (T, H // 32), generator=g, device="cuda", dtype=torch.uint8)
    off_d = torch.from_numpy(off).cuda()
    o, s = m.mxfp4_row_to_fp8_col(packed, sb, off_d, H)
    orow, srow = m.mxfp4_row_to_fp8_row(packed, sb, H)
    torch.cuda.synchronize()
    HB = H // 128
    assert H * int(off[E - 4]) > (1 << 32)
    for e in (0, E // 2, E - 4, E - 2, E - 1):
        a, b = int(off[e]), int(off[e + 1])
        n = b - a
        if n == 0:
            continue
        # token windows at the start, middle and end of the expert (the
        # conversion has no dependence across tokens)
        wins = sorted({(0, min(n, 512)), (max(0, n // 2 - 256), min(n, n // 2 + 256)), (max(0, n - 512), n)})
        for t0, t1 in wins:
            pk, sc = host(packed[a + t0:a + t1]), host(sb[a + t0:a + t1])
            for blk in (0, HB - 1):
                cols, scs = slice(blk * 64, blk * 64 + 64), slice(blk * 4, blk * 4 + 4)
                ro, rs = fp8col.convert(pk[:, cols], sc[:, scs], np.array([0, t1 - t0], np.int64), 128)
                rows = o[H * a: H * b].view(H, n)[blk * 128: blk * 128 + 128, t0:t1]
                np.testing.assert_array_equal(host(rows).reshape(-1), ro)
                gs = s[HB * a: HB * b].view(HB, n)[blk, t0:t1]
                np.testing.assert_array_equal(host(gs).view(np.uint32), rs.view(np.uint32))
            k = min(32, t1 - t0)                          # FP8 rows: the window's first tokens
            qo, qs = fp8col.convert_rows(pk[:k], sc[:k], H)
            np.testing.assert_array_equal(host(orow[a + t0:a + t0 + k]), qo)
            np.testing.assert_array_equal(host(srow[a + t0:a + t0 + k]).view(np.uint32),
                                          qs.view(np.uint32))
    # the same shards with FP8 blocks of 128 tokens, into the same FP8 buffer
    del orow, srow
    st = torch.empty(m.tokblk_scale_count(T, E, H), dtype=torch.float32, device="cuda")
    m.mxfp4_row_to_fp8_col_tokblk(packed, sb, off_d, H, o, st)
    torch.cuda.synchronize()
    base = fp8col.token_block_scale_offset(off, H)
    for e in (0, E // 2, E - 4, E - 2, E - 1):
        a, b = int(off[e]), int(off[e + 1])
        n = b - a
        if n == 0:
            continue
        nb = (n + 127) // 128
        # windows starting on 128-token blocks (a block depends only on its tokens)
        wins = sorted({(0, min(n, 512)), (128 * max(0, (n // 2 - 256) // 128), min(n, 128 * max(0, (n // 2 - 256) // 128) + 512)),
                       (128 * max(0, (n - 512) // 128), n)})
        for t0, t1 in wins:
            pk, sc = host(packed[a + t0:a + t1]), host(sb[a + t0:a + t1])
            wb = (t1 - t0 + 127) // 128
            for blk in (0, HB - 1):
                cols, scs = slice(blk * 64, blk * 64 + 64), slice(blk * 4, blk * 4 + 4)
                ro, rs, _ = fp8col.convert_token_blocks(pk[:, cols], sc[:, scs], np.array([0, t1 - t0], np.int64), 128)
                rows = o[H * a: H * b].view(H, n)[blk * 128: blk * 128 + 128, t0:t1]
                np.testing.assert_array_equal(host(rows).reshape(-1), ro)
                gs = st[int(base[e]): int(base[e]) + H * nb].view(H, nb)[blk * 128: blk * 128 + 128, t0 // 128: t0 // 128 + wb]
                np.testing.assert_array_equal(host(gs).view(np.uint32), rs[:128 * wb].reshape(128, wb).view(np.uint32))


def test_errfeedback_past_2_32_elements():
    """fp32 x and residual of 2^32 + 98,304 elements each (16 GiB), SR with a
    given S_t, in one step: W and the new residual of sampled rows, including
    the last, bit for bit."""
    m = need_gpu()
    R, C = (1 << 17) + 3, 1 << 15
    _need_memory(R * C * (4 + 4 + 2))
    xb = _fill(R, C, 13)
    x = xb.float()
    del xb
    r = torch.zeros((R, C), dtype=torch.float32, device="cuda")
    r[R - 1] = 1e-3                                      # a non-zero residual on the last row
    w = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    st = np.float32(5.0 / 2688)
    ts = torch.tensor([st], dtype=torch.float32, device="cuda")
    ids = [0, R // 2, R - 2, R - 1]
    xs = host(x[torch.tensor(ids, device="cuda")])
    rs = host(r[torch.tensor(ids, device="cuda")])
    m.fp4_errfeedback_qdq(x, r, w, None, "sr", 21, 3, "given", ts)
    torch.cuda.synchronize()
    oy, orr, _, _, _ = nvfp4.errfeedback_qdq(xs, rs, st, "sr", seed=21, step=3, row_ids=ids)
    np.testing.assert_array_equal(host_bf16(w[torch.tensor(ids, device="cuda")]), oy)
    np.testing.assert_array_equal(host(r[torch.tensor(ids, device="cuda")]).view(np.uint32),
                                  orr.view(np.uint32))


def test_fp4quant_past_2_32_elements():
    """FP4Quant G = 256 over 2^32 + 98,304 bf16 elements: sampled rows of the
    codes and scales within the transform's tolerance.  Then the oracle's
    codes and scales of those rows are written into the encoded tensor and
    the whole tensor is decoded: the sampled rows (the last past element
    2^32) agree with the oracle's decode of its own codes within 1e-6 of each
    output."""
    from oracle import fp4quant as Q
    from test_gpu_fp4quant import code_tol, grid_pos, s2_rtol
    m = need_gpu()
    R, C, G = (1 << 17) + 3, 1 << 15, 256
    _need_memory(R * C * (2 + 0.5 + 4) + 2 * R * C // G * 4)
    x = _fill(R, C, 14)
    p, s1, s2 = m.fp4quant_encode(x, G)
    torch.cuda.synchronize()
    ids = [0, R // 2, R - 1]
    t = torch.tensor(ids, device="cuda")
    xs = _rows(x, ids)
    del x
    ph, h1, h2 = host(p[t]), host(s1[t]), host(s2[t])
    rc, r1, r2 = Q.encode(xs, G)
    codes = F.unpack_codes(ph)
    d = np.abs(grid_pos(codes) - grid_pos(rc))
    assert d.max() <= 1 and np.mean(d > 0) < 1e-4
    assert np.all(F.e2m1_rtn_margin(Q.ratios(xs, G))[d > 0] <= code_tol(G))
    np.testing.assert_allclose(h1, r1, rtol=1e-6, atol=0)
    np.testing.assert_allclose(h2, r2, rtol=s2_rtol(G), atol=0)
    p[t] = torch.from_numpy(F.pack_codes(rc)).cuda()
    s1[t] = torch.from_numpy(r1).cuda()
    s2[t] = torch.from_numpy(r2).cuda()
    y = m.fp4quant_decode(p, s1, s2, R, C, G, torch.float32)
    torch.cuda.synchronize()
    ref = Q.decode64(rc, r1, r2, G)
    assert np.all(np.abs(host(y[t]).astype(np.float64) - ref) <= 1e-6 * np.abs(ref) + 2.0 ** -148)


def test_fp4quant_sr_counters_past_2_34_elements():
    """The FP4Quant SR variant over 2^34 + 2^21 bf16 elements (G = 256): the
    draws of the last rows use Philox counters with a non-zero high word.
    Sampled rows, including the last, within the SR tolerance."""
    from oracle import fp4quant as Q
    from test_gpu_fp4quant import check_encode_sr
    m = need_gpu()
    R, C, G = (1 << 19) + 64, 1 << 15, 256
    _need_memory(R * C * (2 + 0.5) + 2 * R * C // G * 4)
    x = _fill(R, C, 15)
    seed, step = 0x0123456789ABCDEF, (1 << 33) + 5
    p, s1, s2 = m.fp4quant_encode_ex(x, G, "sr", seed, step)
    torch.cuda.synchronize()
    ids = [0, R // 3, R - 65, R - 64, R - 1]            # the last 64 rows lie past 2^34
    t = torch.tensor(ids, device="cuda")
    check_encode_sr(host(p[t]), host(s1[t]), host(s2[t]), _rows(x, ids), G, seed, step, row_ids=ids)


def test_mxfp4_sr_from_fp32_past_2_34_elements():
    """MXFP4 stochastic rounding from fp32 over 2^34 + 2^21 elements (64 GiB):
    the four-element lanes of the last rows draw from Philox counters with a
    non-zero high word.  Sampled rows, including the last, bit-exact."""
    m = need_gpu()
    R, C = (1 << 19) + 64, 1 << 15
    _need_memory(R * C * (4 + 0.5 + 1 / 32))
    x = torch.empty((R, C), dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(16)
    x.normal_(0.0, 2.0, generator=g)
    seed, step = 0x0FEDCBA987654321, (1 << 35) + 9
    p, s, _ = m.fp4_quantize(x, "mxfp4", "sr", seed=seed, step=step)
    torch.cuda.synchronize()
    ids = [0, R // 3, R - 65, R - 64, R - 1]            # the last 64 rows lie past 2^34
    t = torch.tensor(ids, device="cuda")
    xs = host(x[t])
    rp, rs = mxfp4.quantize_packed(xs, "sr", seed=seed, step=step, row_ids=ids)
    np.testing.assert_array_equal(host(s[t]), rs)
    np.testing.assert_array_equal(host(p[t]), rp)


def test_nvfp4_sr_and_errfeedback_from_fp32_past_2_34_elements():
    """NVFP4 stochastic rounding from fp32, then error feedback from fp32 x
    with an fp32 residual, over 2^34 + 2^21 elements (x and r 64 GiB each):
    the four-element lanes of the last rows draw from Philox counters with a
    non-zero high word.  Codes and scales of the quantize, W and the new
    residual of the error-feedback step, on sampled rows including the last,
    bit for bit."""
    m = need_gpu()
    R, C = (1 << 19) + 64, 1 << 15
    _need_memory(R * C * (4 + 4 + 2))
    x = torch.empty((R, C), dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(17)
    x.normal_(0.0, 1.5, generator=g)
    st = np.float32(6.0 / 2688)
    ts = torch.tensor([st], dtype=torch.float32, device="cuda")
    seed, step = 0x00C0FFEE12345678, (1 << 34) + 3
    ids = [0, R // 3, R - 65, R - 64, R - 1]            # the last 64 rows lie past 2^34
    t = torch.tensor(ids, device="cuda")
    xs = host(x[t])
    p, s, _ = m.fp4_quantize(x, "nvfp4", "sr", seed=seed, step=step, tscale="given", tensor_scale=ts)
    torch.cuda.synchronize()
    rp, rs = nvfp4.quantize_packed(xs, st, "sr", seed=seed, step=step, row_ids=ids)
    np.testing.assert_array_equal(host(s[t]), rs)
    np.testing.assert_array_equal(host(p[t]), rp)
    del p, s
    torch.cuda.empty_cache()
    r = torch.empty((R, C), dtype=torch.float32, device="cuda")
    r.normal_(0.0, 0.05, generator=g)
    rs_in = host(r[t])
    w = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    m.fp4_errfeedback_qdq(x, r, w, None, "sr", seed, step + 1, "given", ts)
    torch.cuda.synchronize()
    oy, orr, _, _, _ = nvfp4.errfeedback_qdq(xs, rs_in, st, "sr", seed=seed, step=step + 1, row_ids=ids)
    np.testing.assert_array_equal(host_bf16(w[t]), oy)
    np.testing.assert_array_equal(host(r[t]).view(np.uint32), orr.view(np.uint32))


def test_errfeedback_bf16_in_place_past_2_34_elements():
    """In-place error feedback of a bf16 weight of 2^34 + 2^21 elements with
    an fp32 residual (one lane per octet: more than 2^31 work-items, so the
    grid is issued in slices), SR with Philox counters past 2^32: W and the
    new residual of sampled rows, including the last, bit for bit."""
    m = need_gpu()
    R, C = (1 << 19) + 64, 1 << 15
    _need_memory(R * C * (2 + 4))
    w = _fill(R, C, 18)
    r = torch.empty((R, C), dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(19)
    r.normal_(0.0, 0.05, generator=g)
    st = np.float32(4.5 / 2688)
    ts = torch.tensor([st], dtype=torch.float32, device="cuda")
    seed, step = 0x1357924680ABCDEF, (1 << 36) + 1
    ids = [0, R // 3, R - 65, R - 64, R - 1]            # the last 64 rows lie past 2^34
    t = torch.tensor(ids, device="cuda")
    ws, rs_in = _rows(w, ids), host(r[t])
    m.fp4_errfeedback_qdq(w, r, w, None, "sr", seed, step, "given", ts)
    torch.cuda.synchronize()
    oy, orr, _, _, _ = nvfp4.errfeedback_qdq(ws, rs_in, st, "sr", seed=seed, step=step, row_ids=ids)
    np.testing.assert_array_equal(host_bf16(w[t]), oy)
    np.testing.assert_array_equal(host(r[t]).view(np.uint32), orr.view(np.uint32))
