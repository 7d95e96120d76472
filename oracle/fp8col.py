"""MXFP4 rows -> FP8 E4M3 columns, per ragged expert shard, and MXFP4 rows
-> FP8 E4M3 rows (oracle; test infrastructure only).

Follows the report on "Practical FP4 Training for Large-Scale MoE Models on
Hopper GPUs": "核心技术贡献" item 1 (direct FP4-to-FP8 conversion: 32-element
MXFP4 blocks and 128-element FP8 blocks; the target scale of an FP8 block is
the maximum of its four source block scales and each value's exponent is
compensated by the difference, keeping the value), item 2 (FP4RowToFP8Col:
dequantize, transpose and requantize in one pass) and item 3 (ragged expert
shards addressed through precomputed offsets), and "通信量" (FP8 traffic about
1.03 M K bytes, i.e. 4-byte scales per 128 elements).

Definition used here (the value-level meaning of the bit remap):
  for expert e with tokens [off[e], off[e+1]), token t, FP8 block b
  (hidden channels 128b .. 128b+127 of that token = four MXFP4 blocks):
    S_tgt = max of the four UE8M0 bytes;   d = S_tgt - S_sub >= 0
    out[h, t - off[e]] = e4m3_RNE_sat( e2m1(code[t, h]) * 2**-d )   (float64)
    fp32 scale[b, t - off[e]] = 2**(S_tgt - 127)
[reading] "FP8 column": after the per-expert transpose to [H, n_e] a block is
128 consecutive rows of one column.  The fp8 output of expert e starts at
byte H*off[e]; its scales start at element (H/128)*off[e].
"""
import numpy as np

from . import formats as F


def convert(packed, scale_bytes, offsets, H):
    """packed uint8 [T, H/2]; scale_bytes uint8 [T, H/32]; offsets int64 [E+1].
    Returns (fp8 bytes uint8 [T*H], fp32 scales float32 [T*H/128])."""
    packed = np.asarray(packed, dtype=np.uint8)
    sb = np.asarray(scale_bytes, dtype=np.uint8).astype(np.int64)
    off = np.asarray(offsets, dtype=np.int64)
    T = packed.shape[0]
    assert H % 128 == 0 and packed.shape[1] * 2 == H and sb.shape == (T, H // 32)
    if (sb == 0xFF).any():
        raise ValueError("UE8M0 NaN scale is outside the contract")
    out = np.zeros(T * H, dtype=np.uint8)
    sc_out = np.zeros(T * (H // 128), dtype=np.float32)
    for e in range(off.size - 1):
        a, b = int(off[e]), int(off[e + 1])
        n = b - a
        if n == 0:
            continue
        codes = F.unpack_codes(packed[a:b])                      # [n, H]
        sub = sb[a:b]                                            # [n, H/32]
        tgt = sub.reshape(n, H // 128, 4).max(axis=2)            # [n, H/128]
        d = np.repeat(tgt, 4, axis=1) - sub                      # [n, H/32]
        val = F.e2m1_decode(codes).reshape(n, H // 32, 32) * np.exp2(-d[..., None].astype(np.float64))
        fp8 = F.e4m3_encode(val.reshape(n, H))                   # [n, H]
        out[H * a: H * b] = fp8.T.reshape(-1)                    # [H, n]
        sc = np.exp2(tgt.astype(np.float64) - 127.0).astype(np.float32)  # [n, H/128]
        sc_out[(H // 128) * a: (H // 128) * b] = sc.T.reshape(-1)
    return out, sc_out


def convert_rows(packed, scale_bytes, H):
    """MXFP4 rows -> FP8 E4M3 rows, no transpose: the receiver that the MoE
    report names FP4RowToFP8Row beside FP4RowToFP8Col ("核心技术贡献" items
    1-2), with the same value-level remap as convert():
      S_tgt = max of the four UE8M0 bytes of each 128-channel block;
      out[t, h] = e4m3_RNE_sat( e2m1(code[t, h]) * 2**-(S_tgt - S_sub) );
      fp32 scale[t, b] = 2**(S_tgt - 127).
    packed uint8 [T, H/2]; scale_bytes uint8 [T, H/32].
    Returns (fp8 bytes uint8 [T, H], fp32 scales float32 [T, H/128])."""
    packed = np.asarray(packed, dtype=np.uint8)
    sb = np.asarray(scale_bytes, dtype=np.uint8).astype(np.int64)
    T = packed.shape[0]
    assert H % 128 == 0 and packed.shape[1] * 2 == H and sb.shape == (T, H // 32)
    if (sb == 0xFF).any():
        raise ValueError("UE8M0 NaN scale is outside the contract")
    codes = F.unpack_codes(packed)                               # [T, H]
    tgt = sb.reshape(T, H // 128, 4).max(axis=2)                 # [T, H/128]
    d = np.repeat(tgt, 4, axis=1) - sb                           # [T, H/32]
    val = F.e2m1_decode(codes).reshape(T, H // 32, 32) * np.exp2(-d[..., None].astype(np.float64))
    out = F.e4m3_encode(val.reshape(T, H))
    sc = np.exp2(tgt.astype(np.float64) - 127.0).astype(np.float32)
    return out.astype(np.uint8), sc


def token_block_scale_offset(offsets, H):
    """First fp32 element of each expert's scales in convert_token_blocks:
    expert e's [H, ceil(n_e / 128)] matrix starts at H * (ceil(off[e] / 128) + e)
    (a closed form of off[e] and e, so no prefix sum over the experts; the
    matrices never overlap because ceil(off[e+1]/128) + 1 - ceil(off[e]/128)
    >= ceil(n_e / 128)).  The whole scale buffer holds H * (ceil(T/128) + E)
    floats; entries between the matrices are not written."""
    off = np.asarray(offsets, dtype=np.int64)
    e = np.arange(off.size, dtype=np.int64)
    return H * (-(-off // 128) + e)


def convert_token_blocks(packed, scale_bytes, offsets, H):
    """MXFP4 rows -> FP8 E4M3 columns with FP8 blocks along the tokens: the
    alternative reading of the MoE report's FP8 column ("核心技术贡献" items 1
    and 2: the FP8 copy feeds the backward pass, whose weight gradient
    contracts over the tokens, so after the per-expert transpose a block is
    128 consecutive tokens of one hidden channel; "方法概述": the backward
    pass stays in FP8).  The target scale of a block is again the largest of
    its source block scales -- here the UE8M0 bytes of the block's tokens for
    the channel's 32-channel group -- and each value keeps its magnitude by
    the exponent shift d = S_tgt - S_sub.  A shard whose token count is not a
    multiple of 128 ends in a partial block, whose target comes from the
    tokens it has.

      for expert e with tokens [off[e], off[e+1]), n = n_e, channel h,
      token block j (local tokens 128 j .. min(128 j + 128, n) - 1):
        S_tgt(j, h) = max over those tokens t of sb[t, h // 32]
        out[h, t - off[e]] = e4m3_RNE_sat( e2m1(code[t, h]) * 2**-(S_tgt - sb[t, h//32]) )
        fp32 scale[h, j] = 2**(S_tgt - 127), in expert e's [H, ceil(n / 128)]
        matrix at token_block_scale_offset(off, H)[e]

    packed uint8 [T, H/2]; scale_bytes uint8 [T, H/32]; offsets int64 [E+1].
    Returns (fp8 bytes uint8 [T*H], fp32 scales float32 [H*(ceil(T/128)+E)],
    bool mask of the scale entries written)."""
    packed = np.asarray(packed, dtype=np.uint8)
    sb = np.asarray(scale_bytes, dtype=np.uint8).astype(np.int64)
    off = np.asarray(offsets, dtype=np.int64)
    T = packed.shape[0]
    E = off.size - 1
    assert H % 128 == 0 and packed.shape[1] * 2 == H and sb.shape == (T, H // 32)
    if (sb == 0xFF).any():
        raise ValueError("UE8M0 NaN scale is outside the contract")
    base = token_block_scale_offset(off, H)
    out = np.zeros(T * H, dtype=np.uint8)
    sc_out = np.zeros(H * (-(-T // 128) + E), dtype=np.float32)
    written = np.zeros(sc_out.size, dtype=bool)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        n = b - a
        if n == 0:
            continue
        nb = -(-n // 128)
        codes = F.unpack_codes(packed[a:b])                      # [n, H]
        sub = sb[a:b]                                            # [n, H/32]
        # a partial last block is padded with byte 0, which never raises a maximum
        padded = np.zeros((nb * 128, H // 32), dtype=np.int64)
        padded[:n] = sub
        tgt = padded.reshape(nb, 128, H // 32).max(axis=1)       # [nb, H/32]
        d = tgt[np.arange(n) // 128] - sub                       # [n, H/32]
        val = F.e2m1_decode(codes).reshape(n, H // 32, 32) * np.exp2(-d[..., None].astype(np.float64))
        fp8 = F.e4m3_encode(val.reshape(n, H))                   # [n, H]
        out[H * a: H * b] = fp8.T.reshape(-1)                    # [H, n]
        sc = np.exp2(np.repeat(tgt, 32, axis=1).astype(np.float64) - 127.0).astype(np.float32)  # [nb, H]
        sc_out[base[e]: base[e] + H * nb] = sc.T.reshape(-1)     # [H, nb]
        written[base[e]: base[e] + H * nb] = True
    return out, sc_out, written
