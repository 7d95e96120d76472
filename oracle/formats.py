"""Element formats used by the codec (oracle; test infrastructure only).

E2M1: "weight precision part 2", section "What FP4 can hold" -- the table of
the eight non-negative FP4 values (sign, 2 exponent bits, 1 mantissa bit) and
their negative copies.
E4M3: "fp4-train", section "How it works" (block scale encoded to e4m3) and
"Requirements and limits" (software e4m3 conversion).  The bit layout is the
OCP FP8 E4M3FN format [external]: bias 7, max 448, subnormals, no infinity,
0x7F / 0xFF are NaN.
UE8M0: "weight precision part 2", "Block scaling" (MXFP4's 8-bit
power-of-two scale); byte b means 2**(b-127), 0xFF is NaN (OCP MX) [external].
bf16: round-to-nearest-even from fp32 [external, IEEE].
"""
import numpy as np

# The eight non-negative E2M1 values, indexed by the 3 magnitude bits
# (exponent bits then mantissa bit), as tabulated on the page.
E2M1_TABLE = {
    (0b00, 0): 0.0, (0b00, 1): 0.5,
    (0b01, 0): 1.0, (0b01, 1): 1.5,
    (0b10, 0): 2.0, (0b10, 1): 3.0,
    (0b11, 0): 4.0, (0b11, 1): 6.0,
}
E2M1_MAG = np.array([E2M1_TABLE[(m >> 1, m & 1)] for m in range(8)], dtype=np.float64)
E2M1_MAX = 6.0


def e2m1_decode(codes):
    """4-bit code (bit 3 = sign, bits 2..0 = magnitude) -> float64 value.

    A code with the sign bit and magnitude 0 decodes to -0.0 [reading: the
    sign bit is kept on zeros]."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAG[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def _signbit_code(q):
    return np.where(np.signbit(q), 8, 0).astype(np.uint8)


def e2m1_rtn(q):
    """Round-to-nearest onto the E2M1 grid, ties to the even code.

    "fp4-train" ("How it works") rounds each scaled element to the e2m1 grid;
    "weight precision part 2" ("Block scaling", step 4) rounds to the nearest
    FP4 value.  [reading] Ties go to the even magnitude code (IEEE
    round-half-even) and magnitudes above 6 saturate to 6, since E2M1 has no
    infinity.  Definition used: the grid value at minimum distance; on an
    exact tie the one with even code.  Input may be float32 or float64.
    NaN is outside the contract and raises.
    """
    q = np.asarray(q)
    if np.isnan(q).any():
        raise ValueError("NaN is outside the codec's contract")
    a = np.minimum(np.abs(q.astype(np.float64)), E2M1_MAX)   # inf -> 6
    dist = np.abs(a[..., None] - E2M1_MAG)                   # exact in fp64
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best
    idx = np.arange(8)
    # among the (at most two, adjacent) nearest, prefer the even index
    score = np.where(cand, np.where(idx % 2 == 0, 0, 1), 99)
    m3 = np.argmin(score, axis=-1).astype(np.uint8)
    return (m3 | _signbit_code(q)).astype(np.uint8)


# Where RTN changes its decision between adjacent grid magnitudes: the
# midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.
E2M1_MIDPOINTS = (E2M1_MAG[:-1] + E2M1_MAG[1:]) / 2


def e2m1_rtn_margin(q):
    """Distance from |q| to the nearest midpoint of adjacent E2M1 magnitudes,
    i.e. how far q may move before e2m1_rtn picks another grid magnitude
    (the sign of a zero aside; magnitudes beyond 5 only ever round to 6, so
    their margin is |q| - 5 as well).  float64."""
    a = np.abs(np.asarray(q, dtype=np.float64))
    return np.abs(a[..., None] - E2M1_MIDPOINTS).min(axis=-1)


def e2m1_sr_margin(q, u):
    """Distance from |q| to the nearest point where e2m1_sr(., u) changes its
    decision for this u: the thresholds g_k + u (g_{k+1} - g_k) between
    adjacent grid magnitudes g_k < g_{k+1} (at u = 0 the first one is 0,
    where the sign of a non-zero code flips).  float64."""
    a = np.abs(np.asarray(q, dtype=np.float64))
    u = np.asarray(u, dtype=np.float64)
    thr = E2M1_MAG[:-1] + u[..., None] * (E2M1_MAG[1:] - E2M1_MAG[:-1])
    return np.abs(a[..., None] - thr).min(axis=-1)


def e2m1_sr(q, u):
    """Stochastic rounding onto the E2M1 grid.

    "fp4-train", "How it works": a value lying between two neighbouring grid
    points rounds up with a probability proportional to how far it sits above
    the lower point, which makes the rounding unbiased.  [reading] Work on the
    magnitude |q|: lo = largest grid value <= |q|, hi = the next one; the
    result is hi iff u < (|q| - lo) / (hi - lo), with u in [0, 1) supplied by
    the caller; |q| >= 6 gives 6.  The sign is copied from q.
    """
    q = np.asarray(q)
    if np.isnan(q).any():
        raise ValueError("NaN is outside the codec's contract")
    u = np.asarray(u, dtype=np.float64)
    a = np.abs(q.astype(np.float64))
    lo_idx = np.searchsorted(E2M1_MAG, a, side="right") - 1   # largest grid <= a
    lo_idx = np.clip(lo_idx, 0, 7)
    sat = a >= E2M1_MAX
    hi_idx = np.minimum(lo_idx + 1, 7)
    lo = E2M1_MAG[lo_idx]
    hi = E2M1_MAG[hi_idx]
    width = np.where(sat, 1.0, hi - lo)
    frac = np.where(sat, 0.0, (a - lo) / width)
    m3 = np.where(sat, 7, np.where(u < frac, hi_idx, lo_idx)).astype(np.uint8)
    return (m3 | _signbit_code(q)).astype(np.uint8)


def pack_codes(codes):
    """Two 4-bit codes per byte along the last axis.

    "fp4-train" ("How it works") and the FP4Quant article ("Making
    compression cheap enough to help") store two codes per byte.  [reading:
    no page fixes the order] element 2j goes to the low nibble and element
    2j+1 to the high nibble of byte j, the order of the fp4x2 storage type
    of ROCm's hip_fp4.h (pinned against its host conversion in the tests)."""
    c = np.asarray(codes).astype(np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_codes(packed):
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ----------------------------------------------------------------- E4M3 (FN)
def e4m3_decode(codes):
    """OCP E4M3FN byte -> float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return s * mag


_E4M3_POS = e4m3_decode(np.arange(0x7F))     # 0x00..0x7E, increasing
E4M3_MAX = 448.0


def e4m3_encode(x):
    """float -> OCP E4M3FN byte, round-to-nearest-even, saturating at 448.

    [reading] "fp4-train" only says the block scale is converted to e4m3 in
    software; IEEE nearest-even with saturation to the largest finite value
    (E4M3FN has no infinity) is taken.  Definition used: the representable
    magnitude at minimum distance, ties to the even code, magnitudes above
    448 give 448; the sign bit is copied (so -0 -> 0x80).  NaN raises.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN is outside the codec's contract")
    a = np.minimum(np.abs(x), E4M3_MAX)
    # the representable magnitudes lo <= a < hi around a (lo = hi = 448 at the top)
    k = np.searchsorted(_E4M3_POS, a, side="right")
    lo = np.clip(k - 1, 0, _E4M3_POS.size - 1)
    hi = np.clip(k, 0, _E4M3_POS.size - 1)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    # the nearer one; on an exact tie the one with the even code
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (hi % 2 == 0))
    out = np.where(take_hi, hi, lo).astype(np.uint8)
    out = out.reshape(a.shape)
    return (out | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


# ------------------------------------------------------------------ UE8M0
def e8m0_decode(b):
    """UE8M0 byte -> float64 2**(b-127); 0xFF is NaN."""
    b = np.asarray(b).astype(np.int64)
    return np.where(b == 0xFF, np.nan, np.exp2(b - 127.0))


# ------------------------------------------------------------------- bf16
def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32)


def f32_to_bf16_bits(x):
    """float32 -> bf16 bits, IEEE round-to-nearest-even on the 16 dropped
    mantissa bits (NaN stays NaN, overflow goes to infinity)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)
    return r.astype(np.uint16)


def to_f32(x, dtype):
    """Input tensor (numpy) in the codec's input dtype -> float32 values.
    dtype 'bf16' means x holds uint16 bf16 bit patterns."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    return np.asarray(x, dtype=np.float32)
