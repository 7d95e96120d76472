"""Oracle tasks that the worker pool (oracle_pool.py) runs on chunks of the
full-size workloads.  Each task reads its rows or tokens from memory-mapped
.npy files, runs the oracle on them, compares the result with the HIP
library's output (also read from .npy files) and returns mismatch counts
with the first mismatching index.  Imports numpy and the oracle only."""
import numpy as np

from oracle import formats as F
from oracle import fp4quant as Q
from oracle import fp8col, mxfp4, nvfp4
from oracle.philox import sr_uniform

SUBNORMAL = 2.0 ** -149
NORMAL_MIN = 2.0 ** -126


def _rows(path, a, b):
    return np.array(np.load(path, mmap_mode="r")[a:b])


def _write(path, a, b, value):
    out = np.load(path, mmap_mode="r+")
    out[a:b] = value
    out.flush()
    del out


def _bits(v):
    v = np.ascontiguousarray(v)
    if v.dtype == np.float32:
        return v.view(np.uint32)
    return v


def _diff(got, ref, row0=0):
    """(number of differing elements, index of the first one with its row
    offset by row0) -- float32 arrays compared as bit patterns."""
    bad = _bits(got) != _bits(ref)
    n = int(bad.sum())
    if not n:
        return 0, None
    idx = [int(i) for i in np.argwhere(bad)[0]]
    idx[0] += row0
    return n, tuple(idx)


def _put(res, key, got, ref, row0=0):
    res[key], res[key + "_at"] = _diff(got, ref, row0)


# ------------------------------------------------- NVFP4 / MXFP4 round trips
def nvfp4_rows(t):
    """Rows [a, b) of an NVFP4 quantize (and dequantize) against the oracle,
    bit for bit: codes, scale bytes and the bf16 dequantized values."""
    a, b = t["a"], t["b"]
    x = F.to_f32(_rows(t["x"], a, b), t["dtype"])
    st = np.float32(t["st"])
    rp, rs = nvfp4.quantize_packed(x, st, t["rounding"], t["seed"], t["step"],
                                   row_ids=np.arange(a, b, dtype=np.int64))
    res = {"n": int(x.size)}
    _put(res, "packed", _rows(t["p"], a, b), rp, a)
    _put(res, "scales", _rows(t["s"], a, b), rs, a)
    if t.get("y"):
        _put(res, "dequant", _rows(t["y"], a, b), nvfp4.dequantize(rp, rs, st, "bf16"), a)
    return res


def mxfp4_rows(t):
    """Rows [a, b) of an MXFP4 quantize (and dequantize) against the oracle."""
    a, b = t["a"], t["b"]
    x = F.to_f32(_rows(t["x"], a, b), t["dtype"])
    rp, rs = mxfp4.quantize_packed(x, t["rounding"], t["seed"], t["step"],
                                   row_ids=np.arange(a, b, dtype=np.int64))
    res = {"n": int(x.size)}
    _put(res, "packed", _rows(t["p"], a, b), rp, a)
    _put(res, "scales", _rows(t["s"], a, b), rs, a)
    if t.get("y"):
        _put(res, "dequant", _rows(t["y"], a, b), mxfp4.dequantize(rp, rs, "bf16"), a)
    return res


def mxfp4_quantize_into(t):
    """The oracle's MXFP4 RTN rows of bf16 activations rows [a, b), written
    into the packed and scale files (inputs of the FP8 receivers)."""
    a, b = t["a"], t["b"]
    x = F.bf16_bits_to_f32(_rows(t["x"], a, b))
    rp, rs = mxfp4.quantize_packed(x)
    _write(t["p_out"], a, b, rp)
    _write(t["s_out"], a, b, rs)
    return {"n": int(x.size)}


# ------------------------------------------------------- error feedback
def ef_rows(t):
    """Rows [a, b) of one error-feedback step: the oracle's step on its own
    state (x, r), written to the next-state files, and compared bit for bit
    with the library's W (bf16) and residual."""
    a, b = t["a"], t["b"]
    x = _rows(t["x"], a, b)
    r = _rows(t["r"], a, b)
    ob, rn, _, _, _ = nvfp4.errfeedback_qdq(x, r, np.float32(t["st"]), t["rounding"], t["seed"],
                                            t["step"], out="bf16",
                                            row_ids=np.arange(a, b, dtype=np.int64))
    _write(t["w_out"], a, b, ob)
    _write(t["r_out"], a, b, rn)
    res = {"n": int(x.size)}
    _put(res, "w", _rows(t["w_gpu"], a, b), ob, a)
    _put(res, "r", _rows(t["r_gpu"], a, b), rn, a)
    return res


# ------------------------------------------------------------- FP4Quant
def grid_pos(codes):
    """Signed position of a code on the grid -6 .. -0.5, 0, 0.5 .. 6 (+-0
    merged), as an integer -7 .. 7."""
    c = np.asarray(codes).astype(np.int64)
    mag = c & 7
    return np.where(mag == 0, 0, np.where((c & 8) != 0, -mag, mag))


def _rel(got, ref):
    """Largest |got - ref| / |ref| over ref >= the smallest normal, and the
    number of elements with |ref| below it that differ by more than one
    subnormal step (both float64)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    big = np.abs(ref) >= NORMAL_MIN
    rel = float(np.max(np.abs(got[big] - ref[big]) / np.abs(ref[big]))) if big.any() else 0.0
    small_bad = int(np.sum(np.abs(got[~big] - ref[~big]) > SUBNORMAL))
    return rel, small_bad


def fp4quant_encode_rows(t):
    """Rows [a, b) of an FP4Quant encode.  The oracle's codes and scales are
    written to o_p / o_s1 / o_s2 (they are the input of the decode check);
    the library's codes are compared by grid distance and by how far the
    oracle's z / s2 lies from the rounding decision point (RTN: the nearest
    midpoint; SR: the element's threshold for its draw u), its scales by
    relative error."""
    a, b, G = t["a"], t["b"], t["G"]
    x = F.to_f32(_rows(t["x"], a, b), t["dtype"])
    rows = np.arange(a, b, dtype=np.int64)
    rc, r1, r2 = Q.encode(x, G, t["rounding"], t["seed"], t["step"], row_ids=rows)
    _write(t["o_p"], a, b, F.pack_codes(rc))
    _write(t["o_s1"], a, b, r1)
    _write(t["o_s2"], a, b, r2)
    codes = F.unpack_codes(_rows(t["p"], a, b))
    d = np.abs(grid_pos(codes) - grid_pos(rc))
    q = Q.ratios(x, G)
    if t["rounding"] == "rtn":
        margin = F.e2m1_rtn_margin(q)
    else:
        C = x.shape[1]
        u = sr_uniform(rows[:, None] * C + np.arange(C, dtype=np.int64)[None, :], t["seed"], t["step"])
        margin = F.e2m1_sr_margin(q, u)
    diff = d > 0
    s1 = _rows(t["s1"], a, b)
    s2 = _rows(t["s2"], a, b)
    s1_rel, s1_small = _rel(s1, r1)
    s2_rel, s2_small = _rel(s2, r2)
    return {
        "n": int(x.size), "groups": int(r1.size),
        "code_diff": int(diff.sum()), "code_dmax": int(d.max()),
        "code_margin_max": float(margin[diff].max()) if diff.any() else 0.0,
        "code_d2_q_max": float(np.abs(q)[d == 2].max()) if (d == 2).any() else 0.0,
        "s1_rel": s1_rel, "s1_small": s1_small, "s1_zero": int(np.sum((s1 == 0) != (r1 == 0))),
        "s2_rel": s2_rel, "s2_small": s2_small, "s2_zero": int(np.sum((s2 == 0) != (r2 == 0))),
    }


def fp4quant_decode_rows(t):
    """Rows [a, b) of the decoder run on the oracle's own codes and scales:
    the library's fp32 output against the oracle's float64 decode,
    elementwise (relative error, with one subnormal step of slack below the
    normal range), and its bf16 output against the bf16 roundings of the
    interval ref -+ tol."""
    a, b, G = t["a"], t["b"], t["G"]
    codes = F.unpack_codes(_rows(t["o_p"], a, b))
    ref = Q.decode64(codes, _rows(t["o_s1"], a, b), _rows(t["o_s2"], a, b), G)
    yf = _rows(t["yf"], a, b).astype(np.float64)
    tol = t["rtol"] * np.abs(ref) + 2 * SUBNORMAL
    bad_f = np.abs(yf - ref) > tol
    big = np.abs(ref) >= NORMAL_MIN
    rel = float(np.max(np.abs(yf[big] - ref[big]) / np.abs(ref[big]))) if big.any() else 0.0
    yb = F.bf16_bits_to_f32(_rows(t["yb"], a, b)).astype(np.float64)
    lo = F.bf16_bits_to_f32(F.f32_to_bf16_bits((ref - tol).astype(np.float32))).astype(np.float64)
    hi = F.bf16_bits_to_f32(F.f32_to_bf16_bits((ref + tol).astype(np.float32))).astype(np.float64)
    bad_b = ~((yb >= np.minimum(lo, hi)) & (yb <= np.maximum(lo, hi)))
    exact_b = int(np.sum(_rows(t["yb"], a, b) != F.f32_to_bf16_bits(ref.astype(np.float32))))
    res = {"n": int(ref.size), "f32_rel": rel, "bf16_not_rne_of_ref": exact_b}
    res["f32_bad"], res["f32_bad_at"] = int(bad_f.sum()), (
        tuple(int(i) + (a if k == 0 else 0) for k, i in enumerate(np.argwhere(bad_f)[0])) if bad_f.any() else None)
    res["bf16_bad"], res["bf16_bad_at"] = int(bad_b.sum()), (
        tuple(int(i) + (a if k == 0 else 0) for k, i in enumerate(np.argwhere(bad_b)[0])) if bad_b.any() else None)
    return res


# ------------------------------------------------------- FP8 receivers
def fp8col_windows(t):
    """Token windows of expert shards: for each (e, u0, u1), tokens
    off[e] + u0 .. off[e] + u1 - 1 of expert e converted by the oracle as a
    shard of their own (each output column depends on its token's row
    only), compared with columns u0 .. u1 - 1 of the library's [H, n_e]
    matrix and [H/128, n_e] scales."""
    H = t["H"]
    HB = H // 128
    off = np.asarray(t["off"], np.int64)
    out = np.load(t["o"], mmap_mode="r")
    sc = np.load(t["sc"], mmap_mode="r")
    packed = np.load(t["p"], mmap_mode="r")
    sb = np.load(t["s"], mmap_mode="r")
    res = {"n": 0, "fp8": 0, "fp8_at": None, "scale": 0, "scale_at": None}
    for e, u0, u1 in t["windows"]:
        a, n = int(off[e]), int(off[e + 1] - off[e])
        w = u1 - u0
        ro, rs = fp8col.convert(np.array(packed[a + u0:a + u1]), np.array(sb[a + u0:a + u1]),
                                np.array([0, w], np.int64), H)
        got = np.array(out[H * a:H * (a + n)]).reshape(H, n)[:, u0:u1]
        gs = np.array(sc[HB * a:HB * (a + n)]).reshape(HB, n)[:, u0:u1]
        k, at = _diff(got, ro.reshape(H, w))
        if k:
            res["fp8"] += k
            res["fp8_at"] = res["fp8_at"] or (e, at[0], at[1] + u0)
        k, at = _diff(gs, rs.reshape(HB, w))
        if k:
            res["scale"] += k
            res["scale_at"] = res["scale_at"] or (e, at[0], at[1] + u0)
        res["n"] += H * w
    return res


def fp8col_tokblk_windows(t):
    """Token windows (starting on multiples of 128 tokens) of expert shards
    for the token-block FP8 columns: window (e, u0, u1) converted by the
    oracle as a shard of its own (a 128-token block depends only on its own
    tokens) against columns u0 .. u1 - 1 of the library's [H, n_e] matrix and
    columns u0/128 .. of expert e's [H, ceil(n_e/128)] scale matrix."""
    H = t["H"]
    off = np.asarray(t["off"], np.int64)
    base = fp8col.token_block_scale_offset(off, H)
    out = np.load(t["o"], mmap_mode="r")
    sc = np.load(t["sc"], mmap_mode="r")
    packed = np.load(t["p"], mmap_mode="r")
    sb = np.load(t["s"], mmap_mode="r")
    res = {"n": 0, "fp8": 0, "fp8_at": None, "scale": 0, "scale_at": None}
    for e, u0, u1 in t["windows"]:
        assert u0 % 128 == 0
        a, n = int(off[e]), int(off[e + 1] - off[e])
        w, nb = u1 - u0, (n + 127) // 128
        ro, rs, _ = fp8col.convert_token_blocks(np.array(packed[a + u0:a + u1]), np.array(sb[a + u0:a + u1]),
                                                np.array([0, w], np.int64), H)
        got = np.array(out[H * a:H * (a + n)]).reshape(H, n)[:, u0:u1]
        k, at = _diff(got, ro.reshape(H, w))
        if k:
            res["fp8"] += k
            res["fp8_at"] = res["fp8_at"] or (e, at[0], at[1] + u0)
        wb = (w + 127) // 128
        gs = np.array(sc[base[e]:base[e] + H * nb]).reshape(H, nb)[:, u0 // 128:u0 // 128 + wb]
        k, at = _diff(gs, rs[:H * wb].reshape(H, wb))
        if k:
            res["scale"] += k
            res["scale_at"] = res["scale_at"] or (e, at[0], at[1] + u0 // 128)
        res["n"] += H * w
    return res


def fp8row_rows(t):
    """Tokens [a, b) of the FP8 row receiver against the oracle."""
    a, b, H = t["a"], t["b"], t["H"]
    ro, rs = fp8col.convert_rows(_rows(t["p"], a, b), _rows(t["s"], a, b), H)
    res = {"n": int(ro.size)}
    _put(res, "fp8", _rows(t["o"], a, b), ro, a)
    _put(res, "scale", _rows(t["sc"], a, b), rs, a)
    return res
