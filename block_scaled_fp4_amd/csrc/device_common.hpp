// Device helpers shared by the codec kernels (gfx950, wave64).
//
// Element formats: E2M1 (4-bit: sign, 2 exponent bits with bias 1, one
// mantissa bit; magnitudes 0 .5 1 1.5 2 3 4 6), OCP E4M3FN (bias 7, max 448,
// no infinity), UE8M0 (2^(b-127)).  All conversions here are exact integer /
// IEEE-fp32 sequences whose rounding is round-to-nearest-even by
// construction; none relies on a rounding-mode register.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4mi {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

// ------------------------------------------------------------------ memory
__device__ __forceinline__ u32x4 ld_u32x4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
// A plain (cached) load, for data that a later kernel reads again.
__device__ __forceinline__ u32x4 ld_u32x4_keep(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st_u32x4(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st_u32(void* p, uint32_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

// ------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN keeps its top bits and is quieted.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return (f != f) ? ((u >> 16) | 0x40u) : r;
}
// Two fp32 -> two bf16 (RNE) with the gfx950 converter (v_cvt_pk_bf16_f32),
// which agrees with f32_to_bf16_rne on every non-NaN fp32 (checked
// exhaustively on the GPU); NaN stays NaN with an unspecified payload.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Load 8 consecutive elements (element index 8*i .. 8*i+7) as fp32.
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t i, float (&v)[8]) {
  if constexpr (BF16) {
    u32x4 w = ld_u32x4(static_cast<const uint8_t*>(base) + i * 16);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  } else {
    const uint8_t* p = static_cast<const uint8_t*>(base) + i * 32;
    u32x4 a = ld_u32x4(p), b = ld_u32x4(p + 16);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
}

// Store 8 consecutive fp32 values as f32 or bf16 (RNE).
template <bool BF16>
__device__ __forceinline__ void store8(void* base, int64_t i, const float (&v)[8]) {
  if constexpr (BF16) {
    u32x4 w;
    w.x = pack_bf16x2(v[0], v[1]); w.y = pack_bf16x2(v[2], v[3]);
    w.z = pack_bf16x2(v[4], v[5]); w.w = pack_bf16x2(v[6], v[7]);
    st_u32x4(static_cast<uint8_t*>(base) + i * 16, w);
  } else {
    uint8_t* p = static_cast<uint8_t*>(base) + i * 32;
    u32x4 a, b;
    a.x = __float_as_uint(v[0]); a.y = __float_as_uint(v[1]);
    a.z = __float_as_uint(v[2]); a.w = __float_as_uint(v[3]);
    b.x = __float_as_uint(v[4]); b.y = __float_as_uint(v[5]);
    b.z = __float_as_uint(v[6]); b.w = __float_as_uint(v[7]);
    st_u32x4(p, a);
    st_u32x4(p + 16, b);
  }
}

// ------------------------------------------------------- cross-lane (DPP)
// quad_perm [1,0,3,2]: value of lane ^ 1;  quad_perm [2,3,0,1]: lane ^ 2.
__device__ __forceinline__ float lane_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ int lane_xor1_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ int lane_xor2_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
}

// -------------------------------------------------------------------- E2M1
// Magnitude code of RTN(a) for a = |q| >= 0 (a may be +inf).
// With E = clamp(floor(log2 a), 0, 2) the grid spacing around a is 2^(E-1),
// so k = rne(a * 2^(1-E)) is the rounded value in units of that spacing and
// the magnitude code is k + 2E; everything above 6 saturates to code 7.
// Integer ties in rne are ties to the even code because k and k + 2E share
// their parity.
__device__ __forceinline__ uint32_t e2m1_rtn_mag(float a) {
  int eb = (int)((__float_as_uint(a) >> 23) & 0xFFu);   // biased exponent (0 for subnormal)
  int E = min(max(eb - 127, 0), 2);
  float s = __builtin_amdgcn_ldexpf(a, 1 - E);            // exact scaling by 2, 1 or 1/2
  float k = __builtin_rintf(fminf(s, 8.0f));              // round half to even
  uint32_t m = (uint32_t)k + (uint32_t)(2 * E);
  return min(m, 7u);
}

__device__ __forceinline__ uint32_t sign_nibble(float q) {
  return (__float_as_uint(q) >> 28) & 8u;
}

__device__ __forceinline__ uint32_t e2m1_rtn(float q) {
  return e2m1_rtn_mag(fabsf(q)) | sign_nibble(q);
}

// Stochastic rounding of a = |q| with uniform u24 in [0, 2^24): with lo the
// largest grid value <= a and hi the next, the result is hi iff
// u24 * 2^-24 < (a - lo) / (hi - lo).  In units of the local spacing
// s = a * 2^(1-E): lo = floor(s), frac = s - floor(s) (both exact).
// extra_up lets the caller force the "u = 0 and the exact a is positive"
// case when a has underflowed to zero on its way here.
__device__ __forceinline__ uint32_t e2m1_sr_mag(float a, uint32_t u24, bool extra_up) {
  a = fminf(a, 6.0f);                                    // >= 6 (and inf) pins to code 7
  int eb = (int)((__float_as_uint(a) >> 23) & 0xFFu);
  int E = min(max(eb - 127, 0), 2);
  float s = __builtin_amdgcn_ldexpf(a, 1 - E);           // exact; in [0, 4) or [2, 3]
  float k = __builtin_floorf(s);
  float frac = s - k;
  bool up = ((float)u24 * 0x1p-24f < frac) || extra_up;
  uint32_t m = (uint32_t)k + (uint32_t)(2 * E) + (up ? 1u : 0u);
  return min(m, 7u);
}

// ------------------------------------------- gfx950 scaled FP4 converts
// v_cvt_scalef32_pk_fp4_{f32,bf16}: two inputs divided by a scale and
// rounded to E2M1 (nearest even, saturating), written to byte SEL of `old`
// (first input in the low nibble).  Checked bit-for-bit against e2m1_rtn on
// all 2^32 fp32 inputs at scale 1, and on every bf16 input at every scale
// 2^k, k in [-127, 127]; only those uses appear in this library.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2_f32(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2_bf16(uint32_t old, uint32_t two_bf16, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(bf16x2_t, two_bf16),
                                                   scale, SEL);
}
// Eight E2M1 codes of a word -> eight fp32 values times a power-of-two
// scale (v_cvt_scalef32_pk_f32_fp4; exact at every normal power-of-two
// scale, checked exhaustively on the GPU).
__device__ __forceinline__ void e2m1x8_to_f32(uint32_t w, float scale, float (&v)[8]) {
  const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 0);
  const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 1);
  const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 2);
  const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 3);
  v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
  v[4] = c.x; v[5] = c.y; v[6] = d.x; v[7] = d.y;
}

// Eight fp32 values at unit scale -> eight RTN codes in one word.
__device__ __forceinline__ uint32_t rtn8_unit(const float (&q)[8]) {
  uint32_t w = cvt_fp4x2_f32<0>(0u, q[0], q[1], 1.0f);
  w = cvt_fp4x2_f32<1>(w, q[2], q[3], 1.0f);
  w = cvt_fp4x2_f32<2>(w, q[4], q[5], 1.0f);
  return cvt_fp4x2_f32<3>(w, q[6], q[7], 1.0f);
}

// E2M1 code -> fp32 value (magnitudes built from the bit fields: exponent
// field 0 is the 0 / 0.5 subnormal pair, otherwise 2^(e-1) * (1 + m/2)).
__device__ __forceinline__ float e2m1_value(uint32_t code) {
  uint32_t m3 = code & 7u;
  uint32_t e = m3 >> 1, mb = m3 & 1u;
  float mag = e ? __uint_as_float(((e + 126u) << 23) | (mb << 22)) : 0.5f * (float)mb;
  return __uint_as_float(__float_as_uint(mag) | ((code & 8u) << 28));
}

// -------------------------------------------------------------------- E4M3
// r >= 0 (may be +inf) -> OCP E4M3FN byte, round to nearest even, saturating
// at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode_sat(float r) {
  if (!(r < 448.0f)) return 0x7Eu;
  if (r < 0x1p-6f) {                                      // subnormal range: units of 2^-9
    return (uint32_t)__builtin_rintf(r * 512.0f);         // 8 -> 0x08 = 2^-6 (exact)
  }
  uint32_t u = __float_as_uint(r);
  u += 0x7FFFFu + ((u >> 20) & 1u);                       // RNE to 3 mantissa bits
  uint32_t e = (u >> 23) - 120u;                          // rebias 127 -> 7
  return (e << 3) | ((u >> 20) & 7u);
}

// The same encoding through the gfx950 fp8 converter: v_cvt_pk_fp8_f32 rounds
// to nearest even and agrees with e4m3_encode_sat on every non-negative fp32
// below 464 (checked exhaustively on the GPU); clamping at 448 first makes
// it saturate like e4m3_encode_sat above that.
__device__ __forceinline__ uint32_t e4m3_encode_sat_hw(float r) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(r, 448.0f), 0.0f, 0, false) & 0xFFu;
}

// E4M3FN byte (finite, sign ignored) -> fp32 magnitude.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}
// The same decode through the gfx950 converter (v_cvt_f32_fp8, OCP E4M3FN);
// agrees with e4m3_value on every finite byte (checked exhaustively on the
// GPU).  For bytes 0..0x7E.
__device__ __forceinline__ float e4m3_value_hw(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}
// E4M3FN byte -> fp32 value with sign; 0x7F / 0xFF give NaN.
__device__ __forceinline__ float e4m3_value_signed(uint32_t c) {
  float v = __uint_as_float(__float_as_uint(e4m3_value(c)) | ((c & 0x80u) << 24));
  return ((c & 0x7Fu) == 0x7Fu) ? __builtin_nanf("") : v;
}

// ------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror & Shaw (SC'11): ten rounds of two 32x32->64 products
// with the key bumped by the Weyl constants between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                              uint32_t& c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
}

// Eight uniform 24-bit draws for elements 8*i .. 8*i+7 of the stream keyed by
// (seed, step): element j uses counter (j>>2, step) and output word j & 3.
// WIDE = false promises 2 i + 1 < 2^32 (the counter's second word is then 0,
// so the first rounds' second products depend only on seed and step and are
// computed once per wave on the scalar unit).
template <bool WIDE = true>
__device__ __forceinline__ void sr_draws8(int64_t i, uint64_t seed, uint64_t step,
                                          uint32_t (&u)[8]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint64_t blk = (uint64_t)i * 2u + (uint64_t)h;
    uint32_t c0 = (uint32_t)blk, c1 = WIDE ? (uint32_t)(blk >> 32) : 0u;
    uint32_t c2 = (uint32_t)step, c3 = (uint32_t)(step >> 32);
    philox4x32_10(c0, c1, c2, c3, (uint32_t)seed, (uint32_t)(seed >> 32));
    u[4 * h + 0] = c0 >> 8; u[4 * h + 1] = c1 >> 8;
    u[4 * h + 2] = c2 >> 8; u[4 * h + 3] = c3 >> 8;
  }
}

// Workgroups for an exact grid in which each thread owns `per_thread` items.
inline int64_t blocks_for(int64_t items, int per_thread) {
  const int64_t per_block = (int64_t)kThreads * per_thread;
  return (items + per_block - 1) / per_block;
}

// A dispatch packet holds a grid's size in work-items as a 32-bit count, so
// a larger 1-D grid would wrap.  launch_1d issues `blocks` workgroups of
// `threads` in slices of at most 2^31 work-items and passes each slice's
// first workgroup index as the kernel's last argument (blk0), which the
// kernel adds to blockIdx.x; below that size it is one launch.
constexpr int64_t kSliceItems = int64_t(1) << 31;
template <typename... P, typename... A>
inline void launch_1d(void (*kernel)(P...), int64_t blocks, int threads, hipStream_t st, A... args) {
  const int64_t per = kSliceItems / threads;
  for (int64_t b0 = 0; b0 < blocks; b0 += per) {
    const int64_t nb = blocks - b0 < per ? blocks - b0 : per;
    hipLaunchKernelGGL(kernel, dim3((unsigned)nb), dim3((unsigned)threads), 0, st, args..., b0);
  }
}

// Grid size for a grid-stride loop over `items` work items of one thread each.
inline unsigned grid_for(int64_t items, int64_t cap = 256 * 16) {
  int64_t b = (items + kThreads - 1) / kThreads;
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (unsigned)b;
}

}  // namespace fp4mi
