"""Philox4x32-10 counter-based generator (oracle; test infrastructure only).

"fp4-train", "How it works": stochastic rounding draws from a counter-based
RNG keyed by (seed, step, global index).  [reading] The generator is
Philox4x32 with 10 rounds as published by Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11) [external]:
  round:  (c0,c1,c2,c3) -> (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2),
                            hi(M0*c0) ^ c3 ^ k1, lo(M0*c0))
  key schedule between rounds: k0 += W0, k1 += W1 (mod 2**32)
with the paper's multipliers and Weyl constants.

Stream layout [reading]: element with global row-major index i uses
counter = (lo32(i>>2), hi32(i>>2), lo32(step), hi32(step)),
key = (lo32(seed), hi32(seed)), output word (i & 3), and
u = (word >> 8) * 2**-24 in [0, 1).
"""
import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  All inputs are uint32-valued arrays or
    scalars (broadcast); returns four uint32 arrays."""
    c0, c1, c2, c3 = (np.asarray(v, dtype=np.uint64) & _MASK for v in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK
        p0 = np.uint64(PHILOX_M0) * c0          # < 2**64, exact in uint64
        p1 = np.uint64(PHILOX_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return tuple(v.astype(np.uint32) for v in (c0, c1, c2, c3))


def sr_uniform(index, seed, step):
    """u in [0,1) (float64, exactly a multiple of 2**-24) for each global
    element index (int64 array), per the stream layout in the module doc."""
    i = np.asarray(index, dtype=np.uint64)
    blk = i >> np.uint64(2)
    seed = np.uint64(seed)
    step = np.uint64(step)
    w = philox4x32_10(blk & _MASK, blk >> np.uint64(32),
                      step & _MASK, step >> np.uint64(32),
                      seed & _MASK, seed >> np.uint64(32))
    words = np.stack(w, axis=-1)                       # [..., 4]
    sel = (i & np.uint64(3)).astype(np.int64)
    word = np.take_along_axis(words, sel[..., None], axis=-1)[..., 0]
    return (word >> np.uint32(8)).astype(np.float64) * 2.0 ** -24
