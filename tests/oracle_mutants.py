"""Deliberate mistakes planted in the oracle, one at a time, to show that the
CPU pins catch them (tests/test_oracle_mutants.py runs the pins against each).

Each entry: (name, oracle module, exact source text, its wrong replacement).
The text must occur exactly once in the module.  Together they cover every
oracle function with a plausible slip: a wrong table entry, constant, offset,
rounding tie, sign, index, operand order, normalisation or missing transpose.
The nibble order inside a packed byte is left out: no page fixes it (it is
the one "parity unpinned" function), so no pin can catch a swap of it."""

MUTANTS = [
    # formats: E2M1, E4M3, bf16, stochastic rounding, the RTN margin
    ("e2m1 table entry 3 -> 2.5", "oracle.formats", "(0b10, 1): 3.0", "(0b10, 1): 2.5"),
    ("e2m1 RTN ties to odd", "oracle.formats",
     "    score = np.where(cand, np.where(idx % 2 == 0, 0, 1), 99)\n    m3",
     "    score = np.where(cand, np.where(idx % 2 == 1, 0, 1), 99)\n    m3"),
    ("e2m1 RTN saturates at 4", "oracle.formats",
     "a = np.minimum(np.abs(q.astype(np.float64)), E2M1_MAX)",
     "a = np.minimum(np.abs(q.astype(np.float64)), 4.0)"),
    ("e2m1 SR picks the upper point with probability 1 - frac", "oracle.formats",
     "np.where(u < frac, hi_idx, lo_idx)", "np.where(u < frac, lo_idx, hi_idx)"),
    ("e4m3 RNE ties to odd", "oracle.formats",
     "        score = np.where(cand, np.where(idx % 2 == 0, 0, 1), 99)",
     "        score = np.where(cand, np.where(idx % 2 == 1, 0, 1), 99)"),
    ("e4m3 exponent bias 8", "oracle.formats", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    ("e4m3 subnormal step 2^-10", "oracle.formats", "m * 2.0 ** -9", "m * 2.0 ** -10"),
    ("bf16 rounds half up", "oracle.formats", "(u + 0x7FFF + lsb)", "(u + 0x8000)"),
    ("e8m0 bias 128", "oracle.formats", "np.exp2(b - 127.0)", "np.exp2(b - 128.0)"),
    ("RTN margin: farthest midpoint", "oracle.formats",
     "np.abs(a[..., None] - E2M1_MIDPOINTS).min(axis=-1)",
     "np.abs(a[..., None] - E2M1_MIDPOINTS).max(axis=-1)"),
    # philox
    ("philox 9 rounds", "oracle.philox", "for r in range(10):", "for r in range(9):"),
    ("philox multiplier", "oracle.philox", "PHILOX_M1 = 0xCD9E8D57", "PHILOX_M1 = 0xCD9E8D59"),
    ("philox key schedule", "oracle.philox", "(k1 + np.uint64(PHILOX_W1))", "(k1 + np.uint64(PHILOX_W0))"),
    ("philox output permutation", "oracle.philox",
     "c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0",
     "c0, c1, c2, c3 = hi0 ^ c1 ^ k0, lo1, hi1 ^ c3 ^ k1, lo0"),
    ("SR stream: one call per element", "oracle.philox", "blk = i >> np.uint64(2)", "blk = i"),
    ("SR stream: 23-bit uniforms", "oracle.philox", "(word >> np.uint32(8))", "(word >> np.uint32(9))"),
    ("SR stream: seed and step swapped", "oracle.philox",
     "step & _MASK, step >> np.uint64(32),\n                      seed & _MASK, seed >> np.uint64(32)",
     "seed & _MASK, seed >> np.uint64(32),\n                      step & _MASK, step >> np.uint64(32)"),
    # nvfp4
    ("S_t = amax / 1536", "oracle.nvfp4", "a / np.float32(E2M1_MAX * E4M3_MAX)",
     "a / np.float32(E2M1_MAX * 256.0)"),
    ("block scale absmax / 4", "oracle.nvfp4", "r = (absmax / np.float32(6.0))",
     "r = (absmax / np.float32(4.0))"),
    ("decoded scale divides by S_t", "oracle.nvfp4",
     "* np.float32(st)).astype(np.float32)", "/ np.float32(st)).astype(np.float32)"),
    ("element quotient multiplies", "oracle.nvfp4", "q = (x / s_dec)", "q = (x * s_dec)"),
    ("global index with a row pitch of C + 1", "oracle.nvfp4",
     "rows[:, None] * C + np.arange", "rows[:, None] * (C + 1) + np.arange"),
    ("EF residual sign", "oracle.nvfp4", "(v - of).astype", "(of - v).astype"),
    ("EF residual against the fp32 value", "oracle.nvfp4", "(v - of).astype", "(v - y).astype"),
    # mxfp4
    ("UE8M0 exponent offset 1", "oracle.mxfp4", "- 1 - 2", "- 1 - 1"),
    ("MXFP4 SR index transposed", "oracle.mxfp4", "rows[:, None] * C + np.arange(C, dtype=np.int64)[None, :]",
     "rows[:, None] + R * np.arange(C, dtype=np.int64)[None, :]"),
    # fp4quant
    ("WHT in reversed row order", "oracle.fp4quant", "scipy.linalg.hadamard(G).astype", "scipy.linalg.hadamard(G)[::-1].astype"),
    ("RMS without the mean", "oracle.fp4quant", "np.sqrt(np.mean(xg * xg, axis=1))", "np.sqrt(np.sum(xg * xg, axis=1))"),
    ("absmax to 4", "oracle.fp4quant", "s2 = np.max(np.abs(z), axis=1) / 6.0", "s2 = np.max(np.abs(z), axis=1) / 4.0"),
    ("transform normalised by G", "oracle.fp4quant", "z = (y @ H.T) / np.sqrt(G)", "z = (y @ H.T) / G"),
    ("decode divides by s1", "oracle.fp4quant", "(y * np.asarray(s1, np.float64)", "(y / np.asarray(s1, np.float64)"),
    # fp8col
    ("FP8 target scale is the minimum", "oracle.fp8col",
     "tgt = sub.reshape(n, H // 128, 4).max(axis=2)", "tgt = sub.reshape(n, H // 128, 4).min(axis=2)"),
    ("FP8 shift in the wrong direction", "oracle.fp8col",
     "reshape(n, H // 32, 32) * np.exp2(-d", "reshape(n, H // 32, 32) * np.exp2(d"),
    ("FP8 columns not transposed", "oracle.fp8col", "out[H * a: H * b] = fp8.T.reshape(-1)",
     "out[H * a: H * b] = fp8.reshape(-1)"),
    ("FP8 rows: target scale is the minimum", "oracle.fp8col",
     "tgt = sb.reshape(T, H // 128, 4).max(axis=2)", "tgt = sb.reshape(T, H // 128, 4).min(axis=2)"),
]
