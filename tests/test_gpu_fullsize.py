"""Whole-output GPU parity at the five full-size workloads, in the launch
configurations the bench times.

Every output element of every workload is compared with the oracle: the
oracle runs over the whole tensor in a pool of CPU worker processes
(oracle_pool.py, fullsize_tasks.py) and each test prints its mismatch
counts.  Bars: bit-exact for NVFP4 and MXFP4 codes, scale bytes, tensor
scales, dequantized values, error-feedback weights and residuals and both
FP8 receivers; for FP4Quant, fewer than 1e-4 of the codes differ, each by one
grid step and only where the oracle's z / s2 is within the fp32 transform's
error of the decision point, both scales within 1e-6 relative, and the
decoder within 1e-6 relative per element."""
import numpy as np
import pytest
import torch

import fullsize_tasks as T
import synth
from gpu_util import Guarded, dev_bf16, dev_f32, dev_i64, dev_u8, host, host_bf16, need_gpu
from oracle import formats as F
from oracle import nvfp4
from oracle_pool import OraclePool, first_bad, spans, total

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def pool():
    need_gpu()
    with OraclePool() as p:
        print(f"\n[oracle pool: {p.n} worker processes]", flush=True)
        yield p


def _tasks(pool, n_rows, per_worker=4, **common):
    return [dict(common, a=a, b=b) for a, b in spans(n_rows, per_worker * pool.n)]


def _report(name, res, keys):
    n = total(res, "n")
    parts = [f"{k} {total(res, k)}" for k in keys]
    print(f"[{name}] {n} elements compared; mismatches: " + ", ".join(parts), flush=True)
    for k in keys:
        assert total(res, k) == 0, f"{name}: {total(res, k)} {k} mismatches, first at {first_bad(res, k)}"


def _quantize(m, x_dev, fmt, rounding="rtn", seed=0, step=0, tscale="compute", ts=None):
    rows, cols = x_dev.shape
    blk = 32 if fmt == "mxfp4" else 16
    gp, gs = Guarded(rows * cols // 2), Guarded(rows * cols // blk)
    if fmt == "nvfp4" and ts is None:
        ts = torch.empty(1, dtype=torch.float32, device="cuda")
    p, s, ts = m.fp4_quantize(x_dev, fmt, rounding, seed, step, tscale, ts,
                              gp.view(torch.uint8, (rows, cols // 2)),
                              gs.view(torch.uint8, (rows, cols // blk)))
    torch.cuda.synchronize()
    gp.check()
    gs.check()
    return p, s, ts


def _dequantize_bf16(m, p, s, rows, cols, fmt, ts=None):
    gy = Guarded(rows * cols * 2)
    y = m.fp4_dequantize(p, s, rows, cols, fmt, ts, torch.bfloat16, gy.view(torch.bfloat16, (rows, cols)))
    torch.cuda.synchronize()
    gy.check()
    return host_bf16(y)


# ------------------------------------------------ NVFP4 8192 x 8192 RTN
def test_nvfp4_rtn_8192x8192_whole_tensor(pool):
    """NVFP4 RTN round trip of an 8192 x 8192 bf16 weight (N(0, 0.02^2),
    0.1% outliers x50) with the tensor scale computed on the GPU: S_t, every
    code, scale byte and dequantized value."""
    m = need_gpu()
    xb = synth.weight_block(8192, 8192, seed=11)
    R, C = xb.shape
    p, s, ts = _quantize(m, dev_bf16(xb), "nvfp4")
    st = nvfp4.tensor_scale(F.bf16_bits_to_f32(xb))
    gpu_st = host(ts)[0]
    print(f"[nvfp4 8192x8192] S_t gpu {gpu_st!r} oracle {st!r}", flush=True)
    assert np.float32(gpu_st).view(np.uint32) == np.float32(st).view(np.uint32)
    y = _dequantize_bf16(m, p, s, R, C, "nvfp4", ts)
    paths = dict(x=pool.put("x", xb), p=pool.put("p", host(p)), s=pool.put("s", host(s)),
                 y=pool.put("y", y))
    res = pool.map(T.nvfp4_rows, _tasks(pool, R, dtype="bf16", st=float(st), rounding="rtn",
                                        seed=0, step=0, **paths))
    pool.drop(*paths.values())
    _report("nvfp4 8192x8192 RTN", res, ["packed", "scales", "dequant"])


# ------------------------------------------------ MXFP4 4096 x 7168 RTN
def test_mxfp4_moe_dispatch_whole_tensor(pool):
    """MXFP4 RTN quantize and dequantize of the 4096 x 7168 bf16 MoE dispatch
    activation (Student-t(4) * 0.5, 8 hot channels x30): every code, scale
    byte and dequantized value."""
    m = need_gpu()
    xb = synth.moe_dispatch()
    R, C = xb.shape
    p, s, _ = _quantize(m, dev_bf16(xb), "mxfp4")
    y = _dequantize_bf16(m, p, s, R, C, "mxfp4")
    paths = dict(x=pool.put("x", xb), p=pool.put("p", host(p)), s=pool.put("s", host(s)),
                 y=pool.put("y", y))
    res = pool.map(T.mxfp4_rows, _tasks(pool, R, dtype="bf16", rounding="rtn", seed=0, step=0,
                                        **paths))
    pool.drop(*paths.values())
    _report("mxfp4 4096x7168 RTN", res, ["packed", "scales", "dequant"])


def test_mxfp4_moe_dispatch_whole_tensor_sr(pool):
    """The same activation with stochastic rounding (seed and step with
    non-zero high words): every code and scale byte."""
    m = need_gpu()
    xb = synth.moe_dispatch()
    R, C = xb.shape
    seed, step = 0x9E3779B97F4A7C15, (1 << 33) + 7
    p, s, _ = _quantize(m, dev_bf16(xb), "mxfp4", "sr", seed, step)
    paths = dict(x=pool.put("x", xb), p=pool.put("p", host(p)), s=pool.put("s", host(s)))
    res = pool.map(T.mxfp4_rows, _tasks(pool, R, dtype="bf16", rounding="sr", seed=seed, step=step,
                                        **paths))
    pool.drop(*paths.values())
    _report("mxfp4 4096x7168 SR", res, ["packed", "scales"])


# ------------------------------------------------ FP4Quant 8192 x 4096
FQ_CODE_FRAC = 1e-4
FQ_SCALE_RTOL = 1e-6
FQ_RECON_RTOL = 1e-6


def _wht_code_tol(G):
    """How far the oracle's z / s2 may lie from a decision point for an fp32
    evaluation to round the other way: each transform output is a depth
    log2 G tree sum of +-x, so its error is at most eta max|Hx| with
    eta = gamma_log2G sqrt(G); z / s2 then moves by at most 6 (2 eta + 4u)."""
    n = int(np.log2(G))
    eta = n * U32 / (1 - n * U32) * np.sqrt(G)
    return 6.0 * (2 * eta / (1 - eta) + 4 * U32) + 1e-12


@pytest.mark.parametrize("rounding", ["rtn", "sr"])
@pytest.mark.parametrize("G", [64, 256])
def test_fp4quant_tp_tensor_whole_tensor(pool, G, rounding):
    """FP4Quant encode of the 8192 x 4096 bf16 TP tensor (N(0,1), 1% of
    columns x20), then decode of the oracle's own codes and scales (fp32 and
    bf16 outputs): every code, both scales of every group, every output."""
    m = need_gpu()
    xb = synth.tp_tensor()
    R, C = xb.shape
    seed, step = 12345, 77
    x_dev = dev_bf16(xb)
    if rounding == "rtn":
        p, s1, s2 = m.fp4quant_encode(x_dev, G)
    else:
        p, s1, s2 = m.fp4quant_encode_ex(x_dev, G, "sr", seed, step)
    torch.cuda.synchronize()
    ng = C // G
    paths = dict(x=pool.put("x", xb), p=pool.put("p", host(p)), s1=pool.put("s1", host(s1)),
                 s2=pool.put("s2", host(s2)),
                 o_p=pool.new("o_p", (R, C // 2), np.uint8), o_s1=pool.new("o_s1", (R, ng), np.float32),
                 o_s2=pool.new("o_s2", (R, ng), np.float32))
    res = pool.map(T.fp4quant_encode_rows, _tasks(pool, R, G=G, dtype="bf16", rounding=rounding,
                                                  seed=seed, step=step, **paths))
    n, ndiff = total(res, "n"), total(res, "code_diff")
    dmax = max(r["code_dmax"] for r in res)
    mmax = max(r["code_margin_max"] for r in res)
    d2q = max(r["code_d2_q_max"] for r in res)
    s1_rel, s2_rel = max(r["s1_rel"] for r in res), max(r["s2_rel"] for r in res)
    print(f"[fp4quant G{G} {rounding}] {n} codes, {ndiff} differ ({ndiff / n:.2e}), max grid "
          f"distance {dmax}, max decision margin of a differing code {mmax:.3g} (bound "
          f"{_wht_code_tol(G):.3g}); s1 max rel err {s1_rel:.3g}, s2 max rel err {s2_rel:.3g}",
          flush=True)
    assert dmax <= (1 if rounding == "rtn" else 2)
    assert mmax <= _wht_code_tol(G)
    assert d2q <= _wht_code_tol(G)        # a two-step change only as a sign flip around 0 (SR)
    assert ndiff / n < FQ_CODE_FRAC
    assert s1_rel <= FQ_SCALE_RTOL and s2_rel <= FQ_SCALE_RTOL
    for k in ("s1_small", "s1_zero", "s2_small", "s2_zero"):
        assert total(res, k) == 0, k
    if rounding == "sr":
        pool.drop(*paths.values())
        return
    # decode of the oracle's codes and scales on the GPU
    op = np.load(paths["o_p"])
    os1, os2 = np.load(paths["o_s1"]), np.load(paths["o_s2"])
    pk, g1, g2 = dev_u8(op), dev_f32(os1), dev_f32(os2)
    yf = m.fp4quant_decode(pk, g1, g2, R, C, G, torch.float32)
    yb = m.fp4quant_decode(pk, g1, g2, R, C, G, torch.bfloat16)
    torch.cuda.synchronize()
    dpaths = dict(yf=pool.put("yf", host(yf)), yb=pool.put("yb", host_bf16(yb)))
    del yf, yb
    res = pool.map(T.fp4quant_decode_rows, _tasks(pool, R, G=G, rtol=FQ_RECON_RTOL, o_p=paths["o_p"],
                                                  o_s1=paths["o_s1"], o_s2=paths["o_s2"], **dpaths))
    pool.drop(*paths.values(), *dpaths.values())
    rel = max(r["f32_rel"] for r in res)
    print(f"[fp4quant G{G} decode] {total(res, 'n')} outputs; fp32 max rel err {rel:.3g}; "
          f"bf16 outputs not the RNE of the exact value: {total(res, 'bf16_not_rne_of_ref')}", flush=True)
    _report(f"fp4quant G{G} decode", res, ["f32_bad", "bf16_bad"])


# ------------------------------------------------ NVFP4 SR + EF, 10 steps
def test_errfeedback_8192x8192_ten_steps_whole_tensor(pool):
    """The in-place NVFP4 weight loop at 8192 x 8192: W0 ~ N(0, 0.02^2) bf16;
    at step t the fp32 input is x = fl32(W + fl32(1e-4 g_t)), and
    fp4_errfeedback_qdq(x, r, y=W, SR, seed 4, step t, computed S_t) updates
    W and the fp32 residual r in place.  The oracle runs the same ten steps
    on its own state; S_t, every weight and every residual element is
    compared after each step."""
    m = need_gpu()
    R = C = 8192
    wb = synth.ef_weight(R, C, seed=4)
    w_dev = dev_bf16(wb)
    r_dev = torch.zeros((R, C), dtype=torch.float32, device="cuda")
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    w_o = F.bf16_bits_to_f32(wb)                           # the oracle's state
    r_path = pool.put("r0", np.zeros((R, C), np.float32))
    for step in range(10):
        u = synth.ef_update(R, C, seed=4, step=step)
        x_dev = w_dev.float() + dev_f32(u)                 # fl32(W + u): one fp32 add
        m.fp4_errfeedback_qdq(x_dev, r_dev, w_dev, None, "sr", 4, step, "compute", ts)
        torch.cuda.synchronize()
        del x_dev
        x_o = (w_o + u).astype(np.float32)
        del u
        r_o = np.load(r_path, mmap_mode="r")
        st = nvfp4.tensor_scale((x_o + r_o).astype(np.float32))
        del r_o
        gpu_st = host(ts)[0]
        assert np.float32(gpu_st).view(np.uint32) == st.view(np.uint32), (step, gpu_st, st)
        paths = dict(x=pool.put("x", x_o), r=r_path, w_gpu=pool.put("w_gpu", host_bf16(w_dev)),
                     r_gpu=pool.put("r_gpu", host(r_dev)),
                     w_out=pool.new(f"w{step + 1}", (R, C), np.uint16),
                     r_out=pool.new(f"r{step + 1}", (R, C), np.float32))
        del x_o
        res = pool.map(T.ef_rows, _tasks(pool, R, st=float(st), rounding="sr", seed=4, step=step,
                                         **paths))
        _report(f"errfeedback step {step} (S_t {float(st)!r})", res, ["w", "r"])
        w_o = F.bf16_bits_to_f32(np.load(paths["w_out"]))
        pool.drop(paths["x"], paths["w_gpu"], paths["r_gpu"], paths["w_out"], r_path)
        r_path = paths["r_out"]
    pool.drop(r_path)


# ------------------------------------------------ MXFP4 rows -> FP8 (C5)
def _expert_windows(off, width=1024):
    wins = []
    for e in range(off.size - 1):
        n = int(off[e + 1] - off[e])
        for u0 in range(0, n, width):
            wins.append((e, u0, min(n, u0 + width)))
    return wins


def _fp8_inputs_from_activations(pool, Tn, H, seed=5):
    """N(0,1) activations -> bf16 -> MXFP4 by the oracle (in the pool)."""
    xb = synth.expert_activations(tokens=Tn, hidden=H, seed=seed)
    xp = pool.put("acts", xb)
    del xb
    pp, sp = pool.new("mx_p", (Tn, H // 2), np.uint8), pool.new("mx_s", (Tn, H // 32), np.uint8)
    pool.map(T.mxfp4_quantize_into, _tasks(pool, Tn, x=xp, p_out=pp, s_out=sp))
    pool.drop(xp)
    return pp, sp


def _check_fp8col(m, pool, pp, sp, off, H, name):
    Tn = int(off[-1])
    packed, sb = np.load(pp), np.load(sp)
    go, gs = Guarded(Tn * H), Guarded(Tn * H // 128 * 4)
    o, s = m.mxfp4_row_to_fp8_col(dev_u8(packed), dev_u8(sb), dev_i64(off), H,
                                  go.view(torch.uint8, (Tn * H,)), gs.view(torch.float32, (Tn * H // 128,)))
    torch.cuda.synchronize()
    go.check()
    gs.check()
    del packed, sb
    op, sp2 = pool.put("fp8", host(o)), pool.put("fp8s", host(s))
    del o, s, go, gs
    wins = _expert_windows(off)
    chunks = [wins[i::4 * pool.n] for i in range(4 * pool.n)]
    res = pool.map(T.fp8col_windows, [dict(p=pp, s=sp, o=op, sc=sp2, off=off.tolist(), H=H, windows=c)
                                      for c in chunks if c])
    pool.drop(op, sp2)
    _report(name, res, ["fp8", "scale"])


def _check_fp8col_tokblk(m, pool, pp, sp, off, H, name):
    Tn, E = int(off[-1]), off.size - 1
    nsc = m.tokblk_scale_count(Tn, E, H)
    packed, sb = np.load(pp), np.load(sp)
    go, gs = Guarded(Tn * H), Guarded(nsc * 4)
    o, s = m.mxfp4_row_to_fp8_col_tokblk(dev_u8(packed), dev_u8(sb), dev_i64(off), H,
                                         go.view(torch.uint8, (Tn * H,)), gs.view(torch.float32, (nsc,)))
    torch.cuda.synchronize()
    go.check()
    gs.check()
    del packed, sb
    op, sp2 = pool.put("fp8t", host(o)), pool.put("fp8ts", host(s))
    del o, s, go, gs
    wins = _expert_windows(off)
    chunks = [wins[i::4 * pool.n] for i in range(4 * pool.n)]
    res = pool.map(T.fp8col_tokblk_windows, [dict(p=pp, s=sp, o=op, sc=sp2, off=off.tolist(), H=H, windows=c)
                                             for c in chunks if c])
    pool.drop(op, sp2)
    _report(name, res, ["fp8", "scale"])


def _check_fp8row(m, pool, pp, sp, Tn, H, name):
    packed, sb = np.load(pp), np.load(sp)
    o, s = m.mxfp4_row_to_fp8_row(dev_u8(packed), dev_u8(sb), H)
    torch.cuda.synchronize()
    del packed, sb
    op, sp2 = pool.put("fp8r", host(o)), pool.put("fp8rs", host(s))
    del o, s
    res = pool.map(T.fp8row_rows, _tasks(pool, Tn, H=H, p=pp, s=sp, o=op, sc=sp2))
    pool.drop(op, sp2)
    _report(name, res, ["fp8", "scale"])


def test_fp8_receivers_zipf_shards_whole_output(pool):
    """65,536 tokens x 7168 in 256 experts with Zipf(1.1) multinomial counts;
    the MXFP4 rows are the oracle's quantization of N(0,1) bf16 activations.
    FP8 columns (per expert, transposed) and FP8 rows: every output byte and
    every fp32 block scale."""
    m = need_gpu()
    Tn, H, E = 65536, 7168, 256
    counts, off = synth.expert_counts(Tn, E, seed=5)
    pp, sp = _fp8_inputs_from_activations(pool, Tn, H)
    _check_fp8col(m, pool, pp, sp, off, H, "fp8 columns 65536x7168, 256 Zipf experts")
    _check_fp8col_tokblk(m, pool, pp, sp, off, H, "fp8 columns, 128-token blocks, 65536x7168, 256 Zipf experts")
    _check_fp8row(m, pool, pp, sp, Tn, H, "fp8 rows 65536x7168")
    pool.drop(pp, sp)


def test_fp8_receivers_random_rows_whole_output(pool):
    """The same shards with uniformly random code bytes and scale bytes in
    [105, 140], so that shifts between sub-block scales reach 35 (values
    shifted below the E4M3 range): every output byte and scale."""
    m = need_gpu()
    Tn, H, E = 65536, 7168, 256
    counts, off = synth.expert_counts(Tn, E, seed=5)
    packed, sb = synth.random_mxfp4(Tn, H, seed=6, scale_lo=105, scale_hi=140)
    pp, sp = pool.put("mx_p", packed), pool.put("mx_s", sb)
    del packed, sb
    _check_fp8col(m, pool, pp, sp, off, H, "fp8 columns 65536x7168 random rows")
    _check_fp8col_tokblk(m, pool, pp, sp, off, H, "fp8 columns, 128-token blocks, 65536x7168 random rows")
    _check_fp8row(m, pool, pp, sp, Tn, H, "fp8 rows 65536x7168 random rows")
    pool.drop(pp, sp)
