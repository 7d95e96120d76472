"""FP4Quant group codec (oracle; test infrastructure only).

Follows "FP4Quant speeds up GPU communication, with a measurable accuracy
trade-off": section "Why four bits need more than rounding" (split the
tensor into small contiguous groups; a group scale from the root-mean-square
magnitude; a normalized Walsh-Hadamard transform built from additions and
subtractions; a second scale from the largest absolute transformed value
that fits the group into the four-bit range; both scales travel with the
codes; the transform is reversible, the rounding is not) and section
"Making compression cheap enough to help" (receiver: unpack, dequantize,
inverse transform).  Group sizes 64 and 256 are the ones the results section
measures.

Arithmetic is float64 throughout; the two scales are emitted as float32.
The transform is a matrix product with scipy's Sylvester-ordered Hadamard
matrix, a library routine.
"""
import numpy as np
import scipy.linalg

from . import formats as F
from .philox import sr_uniform


def hadamard(G):
    """Sylvester (natural) order: H[i, j] = (-1)**popcount(i & j)."""
    return scipy.linalg.hadamard(G).astype(np.float64)


def _ratios(x, G):
    """The steps of the encoder up to the rounding (see encode); returns
    (q = z / s2 per element [R, C], s1, s2, zero) with s1, s2, zero per
    group, all float64."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    R, C = x.shape
    assert C % G == 0
    xg = x.reshape(-1, G)
    H = hadamard(G)
    s1 = np.sqrt(np.mean(xg * xg, axis=1))
    zero = s1 == 0
    s1_safe = np.where(zero, 1.0, s1)
    y = xg / s1_safe[:, None]
    z = (y @ H.T) / np.sqrt(G)
    s2 = np.max(np.abs(z), axis=1) / 6.0
    s2_safe = np.where(zero | (s2 == 0), 1.0, s2)
    q = z / s2_safe[:, None]
    q[zero] = 0.0
    s1 = np.where(zero, 0.0, s1)
    s2 = np.where(zero, 0.0, s2)
    return q.reshape(R, C), s1, s2, zero


def encode(x, G, rounding="rtn", seed=0, step=0, row_ids=None):
    """x: float32 [R, C] (C % G == 0, G a power of two).

    Per group g (G contiguous elements of a row):
      s1 = sqrt(mean(x**2))      [reading] no epsilon; s1 == 0 -> zeros
      y  = x / s1
      z  = H y / sqrt(G)         [reading] orthonormal "normalized" WHT
      s2 = max|z| / 6            [reading] absmax-to-6, E2M1's largest value
      code = E2M1 RTN(z / s2)    the article's rounding
    rounding="sr" is a variant the article does not describe: "fp4-train"'s
    stochastic rounding ("How it works") applied to z / s2, the draw of
    each transformed element keyed by (seed, step, its row-major index in
    the tensor) exactly as for NVFP4; row_ids names the tensor rows x holds
    when it is a sample of them.
    Returns (codes uint8 [R, C], s1 float32 [R, C/G], s2 float32 [R, C/G])."""
    q, s1, s2, zero = _ratios(x, G)
    R, C = q.shape
    if rounding == "rtn":
        codes = F.e2m1_rtn(q).reshape(-1, G)
    else:
        rows = np.arange(R, dtype=np.int64) if row_ids is None else np.asarray(row_ids, np.int64)
        index = rows[:, None] * C + np.arange(C, dtype=np.int64)[None, :]
        codes = F.e2m1_sr(q, sr_uniform(index, seed, step)).reshape(-1, G)
    codes[zero] = 0
    return (codes.reshape(R, C), s1.astype(np.float32).reshape(R, C // G),
            s2.astype(np.float32).reshape(R, C // G))


def ratios(x, G):
    """The value each code rounds, z / s2 in float64 (0 in zero groups).  A
    float32 implementation may round a code differently from the oracle only
    where this value lies within its arithmetic error of an E2M1 rounding
    boundary (formats.e2m1_rtn_margin)."""
    return _ratios(x, G)[0]


def decode64(codes, s1, s2, G):
    """Receiver in float64: z' = e2m1 * s2; y' = H z' / sqrt(G); x' = y' * s1.
    (H / sqrt(G) is its own inverse.)  Scales are the emitted float32 ones."""
    codes = np.asarray(codes)
    R, C = codes.shape
    zq = F.e2m1_decode(codes).reshape(-1, G) * np.asarray(s2, np.float64).reshape(-1, 1)
    y = (zq @ hadamard(G).T) / np.sqrt(G)
    return (y * np.asarray(s1, np.float64).reshape(-1, 1)).reshape(R, C)


def encode_packed(x, G, rounding="rtn", seed=0, step=0, row_ids=None):
    codes, s1, s2 = encode(x, G, rounding, seed, step, row_ids)
    return F.pack_codes(codes), s1, s2
