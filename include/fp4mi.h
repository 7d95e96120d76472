/*
 * fp4mi.h -- block-scaled FP4 codec for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfp4mi.so.  Every entry point is asynchronous on the HIP stream
 * it is given ("stream" is a hipStream_t passed as void*; NULL means the
 * null stream) and returns an int status (FP4_OK = 0 or an FP4_E* code).
 *
 * Ownership: every tensor argument is caller-owned device memory (for
 * example a torch tensor's data_ptr()).  Except where an entry point says
 * otherwise, the library allocates no device memory and keeps no state
 * between calls; calls are re-entrant.
 *
 * Errors: argument validation happens on the host before any launch.  On a
 * validation error nothing is launched and no output is written.  FP4_EHIP
 * reports a launch failure; faults inside a kernel surface through HIP at
 * the next synchronisation.  A call on an empty tensor (rows*cols == 0, or
 * total_tokens == 0) is a no-op that returns FP4_OK and writes nothing.
 * Element counts rows*cols of 2^46 or more are FP4_ESHAPE; below that, any
 * size that fits in device memory is accepted (grids of more than 2^31
 * work-items are issued in slices).
 *
 * Layout conventions: tensors are dense row-major [rows, cols]; blocks and
 * groups are contiguous runs along cols.  An E2M1 code is 4 bits: bit 3 is
 * the sign, bits 2..0 index the magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
 * Codes are packed two per byte: element 2j in the low nibble of byte j,
 * element 2j+1 in the high nibble ([rows, cols/2] bytes).
 *
 * Values that are NaN, and infinite inputs, are outside the contract: the
 * outputs are then unspecified but every access stays in bounds.
 */
#ifndef FP4MI_H
#define FP4MI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define FP4_OK        0  /* success                                          */
#define FP4_EINVAL    1  /* null pointer, bad enum, bad group size           */
#define FP4_ESHAPE    2  /* negative size or a size that breaks a block rule */
#define FP4_EALIGN    3  /* a pointer is not aligned as documented           */
#define FP4_EDTYPE    4  /* unknown element dtype                            */
#define FP4_EHIP      5  /* a HIP launch failed                              */
#define FP4_EOVERLAP  6  /* an output overlaps an input it may not alias     */

/* ---- enums ------------------------------------------------------------- */
#define FP4_DTYPE_F32   0   /* IEEE float32                                  */
#define FP4_DTYPE_BF16  1   /* bfloat16                                      */

#define FP4_FMT_NVFP4   0   /* 16-element blocks, E4M3 scale, fp32 tensor scale */
#define FP4_FMT_MXFP4   1   /* 32-element blocks, UE8M0 power-of-two scale     */

#define FP4_ROUND_RTN   0   /* round to nearest, ties to the even code        */
#define FP4_ROUND_SR    1   /* stochastic rounding, Philox4x32-10 keyed by    */
                            /* (seed, step, global row-major element index)   */

#define FP4_TSCALE_COMPUTE 0 /* NVFP4: compute S_t from the data, write it    */
#define FP4_TSCALE_GIVEN   1 /* NVFP4: read S_t from *tensor_scale            */

#define FP4MI_ABI_VERSION 1

/*
 * fp4_quantize -- block-scaled FP4 quantize and pack.
 *
 * Follows "fp4-train" (sections "Usage": quantize(W, stochastic, seed, step)
 * -> (packed, scale); "How it works": per-block scale absmax/6, elements
 * divided by the decoded scale and rounded onto the e2m1 grid by RTN or by
 * counter-based stochastic rounding; "Requirements and limits": fp32 or
 * bf16 input) and "weight precision part 2" (section "Block scaling": MXFP4
 * 32-element power-of-two scale, NVFP4 16-element FP8 scale plus one fp32
 * scale per matrix); the MoE report's BF16ToFP4Row kernel is the MXFP4 case.
 *
 *  x            [rows, cols] input, dtype FP4_DTYPE_F32 or _BF16; 16-byte aligned
 *  rows, cols   rows >= 0; cols % 16 == 0 (NVFP4) or cols % 32 == 0 (MXFP4)
 *  fmt          FP4_FMT_NVFP4 or FP4_FMT_MXFP4
 *  rounding     FP4_ROUND_RTN or FP4_ROUND_SR; seed and step key the SR stream
 *  tscale_mode  NVFP4 only.  COMPUTE: S_t = max|x| / 2688 (1 if that is 0) is
 *               computed and written to *tensor_scale (a pass over x before
 *               the codes; the packed output holds its partial maxima until
 *               the codes overwrite them).  GIVEN: *tensor_scale (a positive
 *               finite fp32) is read.  Ignored for MXFP4.
 *  tensor_scale device fp32, 4-byte aligned; may be NULL for MXFP4
 *  packed       out [rows, cols/2] bytes, 4-byte aligned
 *  scales       out: NVFP4 [rows, cols/16] E4M3 bytes, MXFP4 [rows, cols/32]
 *               UE8M0 bytes (value 2^(b-127))
 * Outputs must not overlap x (FP4_EOVERLAP).
 */
int fp4_quantize(const void* x, int dtype, int64_t rows, int64_t cols,
                 int fmt, int rounding, uint64_t seed, uint64_t step,
                 int tscale_mode, float* tensor_scale,
                 uint8_t* packed, uint8_t* scales, void* stream);

/*
 * fp4_dequantize -- unpack and rescale ("fp4-train", "Usage":
 * dequantize(packed, scale, rows, cols)).
 *
 * NVFP4: y = e2m1(code) * fl32(e4m3(scale) * S_t), rounded once to fp32;
 * MXFP4: y = e2m1(code) * 2^(b-127) (exact; UE8M0 0xFF gives NaN).
 * bf16 output is the round-to-nearest-even of that fp32 value.
 *
 *  packed        [rows, cols/2], 4-byte aligned
 *  scales        as written by fp4_quantize
 *  tensor_scale  device fp32 S_t (NVFP4; may be NULL for MXFP4)
 *  y             out [rows, cols] in out_dtype, 16-byte aligned; must not
 *                overlap the inputs
 */
int fp4_dequantize(const uint8_t* packed, const uint8_t* scales,
                   const float* tensor_scale, int64_t rows, int64_t cols,
                   int fmt, void* y, int out_dtype, void* stream);

/*
 * fp4quant_encode -- FP4Quant group encoder ("FP4Quant speeds up GPU
 * communication, with a measurable accuracy trade-off", sections "Why four
 * bits need more than rounding" and "Making compression cheap enough to
 * help").
 *
 * Per group of G contiguous elements along a row:
 *   s1 = sqrt(mean x^2); z = H_G (x / s1) / sqrt(G)  (Sylvester-ordered
 *   Walsh-Hadamard, its own inverse); s2 = max|z| / 6; code = RTN(z / s2).
 * An all-zero group gives codes 0 and s1 = s2 = 0.
 *
 *  x        [rows, cols], f32 or bf16, 16-byte aligned
 *  group    G: a power of two, 16 <= G <= 1024, cols % G == 0
 *  packed   out [rows, cols/2] codes, 4-byte aligned
 *  s_rms    out fp32 s1 [rows, cols/G], 4-byte aligned
 *  s_abs    out fp32 s2 [rows, cols/G], 4-byte aligned
 * Arithmetic is fp32 (the scales and codes agree with an exact evaluation
 * to within fp32 rounding).  Outputs must not overlap x.
 */
int fp4quant_encode(const void* x, int dtype, int64_t rows, int64_t cols,
                    int32_t group, uint8_t* packed, float* s_rms, float* s_abs,
                    void* stream);

/*
 * fp4quant_encode_ex -- fp4quant_encode with a choice of rounding.
 *
 * FP4_ROUND_RTN is fp4quant_encode.  FP4_ROUND_SR is a variant the FP4Quant
 * article does not describe: "fp4-train"'s stochastic rounding (section "How
 * it works": round up to the next grid point with probability
 * (|q| - lo) / (hi - lo), otherwise down) applied to z / s2, the draw of each
 * transformed element keyed by (seed, step, its row-major index in the
 * tensor) with the same Philox4x32-10 stream layout as fp4_quantize.  Scales
 * are those of RTN.  Arguments as fp4quant_encode; rounding outside
 * {RTN, SR} is FP4_EINVAL.
 */
int fp4quant_encode_ex(const void* x, int dtype, int64_t rows, int64_t cols,
                       int32_t group, int rounding, uint64_t seed, uint64_t step,
                       uint8_t* packed, float* s_rms, float* s_abs, void* stream);

/*
 * fp4quant_decode -- FP4Quant receiver: unpack, dequantize, inverse WHT
 * (same page, section "Making compression cheap enough to help"):
 *   x' = s1 * H_G (e2m1(code) * s2) / sqrt(G).
 *  y   out [rows, cols] in out_dtype, 16-byte aligned; must not overlap inputs
 */
int fp4quant_decode(const uint8_t* packed, const float* s_rms, const float* s_abs,
                    int64_t rows, int64_t cols, int32_t group,
                    void* y, int out_dtype, void* stream);

/*
 * fp4_errfeedback_qdq -- NVFP4 quantize-dequantize with a per-element fp32
 * error-feedback residual ("fp4-train", "Usage": ErrorFeedback.qdq(name, x,
 * step); "How it works": the residual x - dequant(quantize(x)) is carried
 * into the next quantization).
 *
 *   v = fl32(x + r)          (r = 0 when residual is NULL: a plain qdq)
 *   S_t from max|v| (COMPUTE) or *tensor_scale (GIVEN)
 *   quantize v (RTN or SR, as fp4_quantize with fmt NVFP4)
 *   y = e2m1 * s_dec in out_dtype;  r <- fl32(v - y)   (residual against the
 *   value actually returned)
 *
 *  x, dtype      [rows, cols] input, 16-byte aligned, cols % 16 == 0
 *  residual      fp32 [rows, cols] in/out, 16-byte aligned, or NULL
 *  y, out_dtype  output [rows, cols], 16-byte aligned; y may be x itself when
 *                out_dtype == dtype (in-place weight update); otherwise no
 *                overlap with the inputs
 *  packed,scales optional outputs (NULL to skip), layouts as fp4_quantize
 *  tensor_scale  device fp32, written (COMPUTE) or read (GIVEN); COMPUTE
 *                keeps partial maxima in an output before the codes are
 *                written: packed when given, else y unless y == x (then a
 *                device atomic on *tensor_scale)
 */
int fp4_errfeedback_qdq(const void* x, int dtype, int64_t rows, int64_t cols,
                        float* residual, void* y, int out_dtype,
                        int rounding, uint64_t seed, uint64_t step,
                        int tscale_mode, float* tensor_scale,
                        uint8_t* packed, uint8_t* scales, void* stream);

/*
 * mxfp4_row_to_fp8_col -- fused MXFP4-row -> FP8-E4M3-column conversion over
 * ragged expert shards (MoE report "Practical FP4 Training for Large-Scale
 * MoE Models on Hopper GPUs", section "核心技术贡献": item 1 direct FP4->FP8
 * exponent remap with 4-to-1 scale alignment, item 2 FP4RowToFP8Col fused
 * dequantize-transpose-requantize, item 3 precomputed shard offsets).
 *
 * For expert e with tokens [off[e], off[e+1]), token t and FP8 block b
 * (hidden channels 128b..128b+127 = four MXFP4 blocks):
 *   S_tgt = max of the four UE8M0 bytes; d = S_tgt - S_sub;
 *   out[h, t-off[e]] = E4M3_RNE_sat(e2m1(code[t,h]) * 2^-d);
 *   fp8_scales[b, t-off[e]] = 2^(S_tgt - 127) (fp32).
 *
 *  packed         [T, H/2] MXFP4 codes (row per token), 16-byte aligned
 *  scales_e8m0    [T, H/32] UE8M0 bytes (0xFF outside the contract), 4-byte aligned
 *  token_offsets  device int64 [E+1]: off[0] = 0, nondecreasing, off[E] = T,
 *                 8-byte aligned (contents are not validated on the host)
 *  num_experts    1 <= E < 2^26 (FP4_EINVAL below 1, FP4_ESHAPE from 2^26);
 *                 total_tokens 0 <= T < 2^26;  hidden 0 < H < 2^21, H % 128 == 0
 *  fp8_out        out bytes [T*H], 4-byte aligned; expert e occupies
 *                 [H*off[e], H*off[e+1]) as a dense [H, n_e] matrix
 *  fp8_scales     out fp32 [T*H/128]; expert e occupies
 *                 [(H/128)*off[e], (H/128)*off[e+1]) as [H/128, n_e]; 4-byte aligned
 * Outputs must not overlap inputs (FP4_EOVERLAP).  Malformed offsets (not
 * ascending, outside [0, T]) are clamped on the device: the outputs are then
 * unspecified but every access stays inside the buffers.
 */
int mxfp4_row_to_fp8_col(const uint8_t* packed, const uint8_t* scales_e8m0,
                         const int64_t* token_offsets, int32_t num_experts,
                         int64_t total_tokens, int64_t hidden,
                         uint8_t* fp8_out, float* fp8_scales, void* stream);

/*
 * mxfp4_row_to_fp8_col_tokblk -- the fused MXFP4-row -> FP8-E4M3-column
 * conversion with FP8 blocks along the tokens: the FP8 copy that feeds the
 * backward pass, whose weight gradient contracts over the tokens (MoE report
 * "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs",
 * section "核心技术贡献" items 1-3; section "方法概述": the backward pass stays
 * in FP8).  After the per-expert transpose to [H, n_e], block j of channel h
 * is the expert's tokens 128j .. 128j+127 (the last block of a shard may be
 * partial), and its target scale is the largest source scale of the block:
 *   S_tgt(h, j) = max over the block's tokens t of UE8M0[t, h/32];
 *   out[h, t-off[e]] = E4M3_RNE_sat(e2m1(code[t,h]) * 2^-(S_tgt - UE8M0[t, h/32]));
 *   scale[h, j] = 2^(S_tgt - 127) (fp32).
 *
 *  packed, scales_e8m0, token_offsets, hidden, fp8_out: as mxfp4_row_to_fp8_col
 *  num_experts    1 <= E < 2^23 (FP4_EINVAL below 1, FP4_ESHAPE from 2^23);
 *                 total_tokens 0 <= T < 2^26;  hidden 0 < H < 2^21, H % 128 == 0
 *  fp8_scales     out fp32 [H * (ceil(T/128) + E)], 4-byte aligned; expert e's
 *                 [H, ceil(n_e/128)] matrix starts at element
 *                 H * (ceil(off[e]/128) + e) (a closed form of the offsets;
 *                 the matrices never overlap; elements between them are not
 *                 written)
 * Outputs must not overlap inputs or each other (FP4_EOVERLAP).  Malformed
 * offsets are clamped on the device as for mxfp4_row_to_fp8_col.
 */
int mxfp4_row_to_fp8_col_tokblk(const uint8_t* packed, const uint8_t* scales_e8m0,
                                const int64_t* token_offsets, int32_t num_experts,
                                int64_t total_tokens, int64_t hidden,
                                uint8_t* fp8_out, float* fp8_scales, void* stream);

/*
 * mxfp4_row_to_fp8_row -- MXFP4 rows -> FP8 E4M3 rows, no transpose: the
 * forward receiver that the MoE report names FP4RowToFP8Row beside
 * FP4RowToFP8Col ("Practical FP4 Training for Large-Scale MoE Models on
 * Hopper GPUs", section "核心技术贡献", items 1 and 2), with the same
 * per-value exponent remap and 4-to-1 scale alignment:
 *   S_tgt = max of the four UE8M0 bytes of a 128-channel block;
 *   out[t, h] = E4M3_RNE_sat(e2m1(code[t,h]) * 2^-(S_tgt - S_sub));
 *   fp8_scales[t, b] = 2^(S_tgt - 127) (fp32).
 *
 *  packed         [T, H/2] MXFP4 codes, 16-byte aligned
 *  scales_e8m0    [T, H/32] UE8M0 bytes (0xFF outside the contract), 4-byte aligned
 *  total_tokens   T >= 0;  hidden H > 0, H % 128 == 0
 *  fp8_out        out [T, H] E4M3 bytes, 16-byte aligned
 *  fp8_scales     out fp32 [T, H/128], 4-byte aligned
 * Outputs must not overlap inputs or each other.
 */
int mxfp4_row_to_fp8_row(const uint8_t* packed, const uint8_t* scales_e8m0,
                         int64_t total_tokens, int64_t hidden,
                         uint8_t* fp8_out, float* fp8_scales, void* stream);

/* Human-readable name of a status code (static string). */
const char* fp4_status_string(int status);

/* FP4MI_ABI_VERSION of the library. */
int fp4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4MI_H */
