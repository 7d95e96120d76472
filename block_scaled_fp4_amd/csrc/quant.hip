// NVFP4 / MXFP4 quantize, dequantize and error-feedback qdq for gfx950.
//
// "fp4-train" ("How it works", "Usage") and "weight precision part 2"
// ("Block scaling") define the operations; the MoE report's BF16ToFP4Row is
// the MXFP4 quantizer.
//
// Work decomposition: one thread owns one "octet" of 8 consecutive elements
// (one 16-byte bf16 load or two 16-byte fp32 loads, one 4-byte store of
// packed codes).  An NVFP4 block (16) is a lane pair, an MXFP4 block (32) a
// lane quad; block maxima are combined with DPP quad permutes, so no LDS is
// used.  Grid-stride loops with strides that are multiples of 256 keep every
// pair / quad either wholly active or wholly inactive.
#include "device_common.hpp"
#include "host_common.hpp"

namespace fp4mi {
namespace {

// Octets per thread: enough independent 16-byte loads in flight per lane to
// cover HBM latency (64 bytes of input per thread for either dtype).
template <bool BF16> constexpr int kOctets = BF16 ? 4 : 2;

// ----------------------------------------------------------- block scales
struct NvScale {
  uint32_t code;   // E4M3 byte
  float sdec;      // fl32(e4m3 * S_t)
};

// fl32(fl32(absmax / 6) / S_t) -> E4M3 (RNE, saturating); s_dec = fl32(e4m3 * S_t).
__device__ __forceinline__ NvScale nv_block_scale_exact(float absmax, float st) {
  float r = absmax / 6.0f;
  r = r / st;
  NvScale s;
  s.code = e4m3_encode_sat_hw(r);
  s.sdec = e4m3_value(s.code) * st;
  return s;
}

// ------------------------------------------- NVFP4 quotients without division
// Three quotients decide the NVFP4 codes: fl32(absmax / 6), fl32(that / S_t)
// and fl32(x / s_dec).  Each is taken as q0 = a * y with y = fl32(1 / b),
// followed by one correction, q1 = fma(-fma(q0, b, -a), y, q0) (residual
// then refined quotient).  On the GPU, for every fp32 significand of b:
//  - recip_rn(b) = fma(fma(-b, r, 1), r, r), r = v_rcp_f32(b), equals the
//    IEEE quotient 1 / b (exponents -100 .. 100 checked);
//  - div_rn(a, 6, fl32(1/6)) equals the IEEE a / 6 for every significand
//    of a;
//  - div_rn(a, b, fl32(1/b)) equals the IEEE a / b for every a within 48
//    ulps of t * b, for each E2M1 rounding threshold t and each value t
//    with at most five significant bits (which includes every E4M3 rounding
//    boundary).
// E2M1 codes and E4M3 bytes change only at those points, so wherever the
// operands and quotients are normal numbers (where scaling by powers of two
// changes nothing) the codes and bytes taken from q1 are those of the IEEE
// quotients.  The residual is negated (fma(q0, b, -a)) so that a zero a
// keeps its sign.
__device__ __forceinline__ float recip_rn(float b) {
  const float r = __builtin_amdgcn_rcpf(b);
  return __builtin_fmaf(__builtin_fmaf(-b, r, 1.0f), r, r);
}
__device__ __forceinline__ float div_rn(float a, float b, float y) {
  const float q0 = a * y;
  return __builtin_fmaf(-__builtin_fmaf(q0, b, -a), y, q0);
}
constexpr float kInv6 = 0x1.555556p-3f;          // fl32(1 / 6)

// S_t range in which the division-free chain holds for every block: all
// s_dec = e4m3 * S_t (2^-9 <= e4m3 <= 448) and their reciprocals are normal.
__device__ __forceinline__ bool nv_newton_range(float st) {
  return st >= 0x1p-100f && st <= 0x1p+100f;
}

// Block scale by the division-free chain; rst = fl32(1 / S_t).  *ok is
// cleared when the raw quotient r is 2^120 or more (a saturated scale so far
// off that element quotients could overflow); the exact scale and codes
// must then be taken.  An absmax below 2^-120 gives r < 2^-22 (byte 0)
// whatever the rounding of absmax / 6, so the chain stays exact there too.
__device__ __forceinline__ NvScale nv_block_scale_newton(float absmax, float st, float rst,
                                                         bool* ok) {
  const float r = div_rn(div_rn(absmax, 6.0f, kInv6), st, rst);
  *ok = r < 0x1p+120f;
  const uint32_t c = e4m3_encode_sat_hw(r);
  return NvScale{c, e4m3_value_hw(c) * st};
}

// MXFP4: UE8M0 byte = clamp(floor(log2 absmax) - 2 + 127, 0, 254), read from
// the exponent field; subnormal and zero maxima give 0.
__device__ __forceinline__ uint32_t mx_scale_byte(float absmax) {
  int eb = (int)((__float_as_uint(absmax) >> 23) & 0xFFu);
  return (uint32_t)max(eb - 2, 0);
}

// Largest magnitude of eight bf16 values as a 16-bit pattern: for finite
// values the patterns with the sign cleared order like the magnitudes, and
// packed 16-bit integer maxima need none of the float maximum's NaN
// handling (v_pk_max_u16).
__device__ __forceinline__ uint32_t absmax_bits_bf16x8(const u32x4& w) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint32_t m = 0x7FFF7FFFu;
  const u16x2 a = __builtin_bit_cast(u16x2, w.x & m), b = __builtin_bit_cast(u16x2, w.y & m);
  const u16x2 c = __builtin_bit_cast(u16x2, w.z & m), d = __builtin_bit_cast(u16x2, w.w & m);
  const u16x2 r = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max((uint32_t)r.x, (uint32_t)r.y);
}

__device__ __forceinline__ float absmax8(const float (&v)[8]) {
  float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  float b = fmaxf(fmaxf(fabsf(v[4]), fabsf(v[5])), fmaxf(fabsf(v[6]), fabsf(v[7])));
  return fmaxf(a, b);
}

__device__ __forceinline__ void unpack_bf16x8(const u32x4& w, float (&v)[8]) {
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void unpack_f32x8(const u32x4& a, const u32x4& b, float (&v)[8]) {
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
  v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
  v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
  v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}

template <bool BF16>
__device__ __forceinline__ void load_octet(const void* x, int64_t i, float (&v)[8]) {
  if constexpr (BF16) {
    unpack_bf16x8(ld_u32x4(static_cast<const uint8_t*>(x) + i * 16), v);
  } else {
    const uint8_t* p = static_cast<const uint8_t*>(x) + i * 32;
    unpack_f32x8(ld_u32x4(p), ld_u32x4(p + 16), v);
  }
}

// Codes of one octet under a decided block scale (software rounding; exact).
template <bool MX, bool SR, bool WIDE = true>
__device__ __forceinline__ uint32_t encode_octet_sw(const float (&v)[8], float sdec, int mx_shift,
                                                    int64_t i, uint64_t seed, uint64_t step) {
  uint32_t u[8];
  if constexpr (SR) sr_draws8<WIDE>(i, seed, step, u);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float q;
    if constexpr (MX) {
      q = __builtin_amdgcn_ldexpf(v[j], mx_shift);     // exact unless it lands below 2^-126
    } else {
      q = (sdec == 0.0f) ? __builtin_copysignf(0.0f, v[j]) : v[j] / sdec;  // IEEE division
    }
    uint32_t c;
    if constexpr (SR) {
      // MX: an exactly positive scaled value that underflowed still rounds up when u = 0.
      bool extra = MX && (q == 0.0f) && (v[j] != 0.0f) && (u[j] == 0u);
      c = e2m1_sr_mag(fabsf(q), u[j], extra) | sign_nibble(v[j]);
    } else {
      c = e2m1_rtn_mag(fabsf(q)) | sign_nibble(v[j]);
    }
    word |= c << (4 * j);
  }
  return word;
}

// NVFP4 RTN codes of fl32(v / sdec) from division-free quotients (exact for
// sdec in [2^-109, 2^109] or 0; see recip_rn / div_rn).  sdec = 0 gives
// y = 0 and sign-only codes.
__device__ __forceinline__ uint32_t encode_octet_nv_rtn(const float (&v)[8], float sdec) {
  const float y = (sdec == 0.0f) ? 0.0f : recip_rn(sdec);
  float q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) q[j] = div_rn(v[j], sdec, y);
  return rtn8_unit(q);
}

// NVFP4 SR codes of q = fl32(v / sdec) (sdec != 0) from the division-free
// quotient.  With y = fl32(1 / sdec), a one-fma correction of fl32(v y) is
// the IEEE quotient whenever neither the quotient nor the residual
// underflows (Markstein's correction theorem); on the GPU it matched the
// IEEE division for every bf16 numerator significand against every fp32
// divisor significand, at exponent pairs spanning |v| >= 2^-100, |q| in
// [2^-100, 2^114] and sdec in [2^-109, 2^109].  The SR decision reads every
// bit of q, so elements outside that range (|v| or |q| below 2^-100, zero
// excepted) take the IEEE division.
template <bool WIDE>
__device__ __forceinline__ uint32_t encode_octet_nv_sr_newton(const float (&v)[8], float sdec,
                                                              int64_t i, uint64_t seed,
                                                              uint64_t step) {
  uint32_t u[8];
  sr_draws8<WIDE>(i, seed, step, u);
  const float y = recip_rn(sdec);
  // |v| >= 2^-100 and |v / sdec| >= 2^-100  <=>  |v| >= 2^-100 max(1, sdec)
  // (a power-of-two multiple of sdec, exact); twice the magnitude bits
  // minus 2 maps a zero to the top of the unsigned range
  const uint32_t lim = (__float_as_uint(0x1p-100f * fmaxf(1.0f, sdec)) << 1) - 2u;
  float q[8];
  uint32_t small = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    q[j] = div_rn(v[j], sdec, y);
    small = min(small, (__float_as_uint(v[j]) << 1) - 2u);
  }
  if (small < lim) {                                   // rare: IEEE quotients
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = v[j] / sdec;
  }
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    word |= (e2m1_sr_mag(fabsf(q[j]), u[j], false) | sign_nibble(v[j])) << (4 * j);
  return word;
}

// MXFP4 RTN codes: divide by 2^e and round in the converter (bf16 words go
// in unexpanded; fp32 values are scaled exactly first and converted at unit
// scale).
template <bool BF16>
__device__ __forceinline__ uint32_t encode_octet_mx_rtn(const u32x4& raw, const float (&v)[8],
                                                        uint32_t sbyte) {
  if constexpr (BF16) {
    const float scale = __builtin_amdgcn_ldexpf(1.0f, (int)sbyte - 127);
    uint32_t w = cvt_fp4x2_bf16<0>(0u, raw.x, scale);
    w = cvt_fp4x2_bf16<1>(w, raw.y, scale);
    w = cvt_fp4x2_bf16<2>(w, raw.z, scale);
    return cvt_fp4x2_bf16<3>(w, raw.w, scale);
  } else {
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = __builtin_amdgcn_ldexpf(v[j], 127 - (int)sbyte);
    return rtn8_unit(q);
  }
}

// ------------------------------------------------------------- quantize
// Thread t of workgroup b owns octets b*256*U + t + 256*k, k < U: every
// load and store instruction of a wave covers 64 consecutive octets, and
// the U loads are issued before any of them is consumed.
template <bool BF16, bool MX, bool SR, int U = kOctets<BF16>, bool WIDE = true>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const void* __restrict__ x, int64_t n_oct, const float* __restrict__ st_ptr, uint64_t seed,
    uint64_t step, uint32_t* __restrict__ packed, uint8_t* __restrict__ scales, int64_t blk0) {
  const float st = MX ? 1.0f : *st_ptr;
  const bool newton = !MX && nv_newton_range(st);
  const float rst = newton ? 1.0f / st : 0.0f;
  const int64_t base = ((int64_t)blockIdx.x + blk0) * (kThreads * U) + threadIdx.x;
  u32x4 ra[U], rb[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t i = base + (int64_t)k * kThreads;
    const bool ok = i < n_oct;
    if constexpr (BF16) {
      ra[k] = ok ? ld_u32x4(static_cast<const uint8_t*>(x) + i * 16) : u32x4{0u, 0u, 0u, 0u};
    } else {
      const uint8_t* p = static_cast<const uint8_t*>(x) + i * 32;
      // MXFP4 reads the two halves of an fp32 octet with plain loads (the
      // line stays in L2 between the two instructions)
      ra[k] = ok ? (MX ? ld_u32x4_keep(p) : ld_u32x4(p)) : u32x4{0u, 0u, 0u, 0u};
      rb[k] = ok ? (MX ? ld_u32x4_keep(p + 16) : ld_u32x4(p + 16)) : u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t i = base + (int64_t)k * kThreads;
    float v[8];
    if constexpr (BF16) unpack_bf16x8(ra[k], v);
    else unpack_f32x8(ra[k], rb[k], v);
    float am = 0.0f;
    if constexpr (BF16) {
      // from bf16: the block maximum as a bf16 pattern, widened to the fp32
      // value (MXFP4 quantize 0.7% faster on 4096 x 7168)
      uint32_t mb = absmax_bits_bf16x8(ra[k]);
      mb = max(mb, (uint32_t)lane_xor1_i((int)mb));
      if constexpr (MX) mb = max(mb, (uint32_t)lane_xor2_i((int)mb));
      am = __uint_as_float(mb << 16);
    } else {
      am = absmax8(v);
      am = fmaxf(am, lane_xor1(am));
      if constexpr (MX) am = fmaxf(am, lane_xor2(am));
    }
    uint32_t scode, word;
    if constexpr (MX) {
      scode = mx_scale_byte(am);
      if constexpr (SR)
        word = encode_octet_sw<true, true, WIDE>(v, 0.0f, 127 - (int)scode, i, seed, step);
      else word = encode_octet_mx_rtn<BF16>(ra[k], v, scode);
    } else if constexpr (SR) {
      // bf16 blocks whose scale came from the division-free chain (S_t in
      // range, raw quotient below 2^120) take division-free element quotients
      bool ok = false;
      NvScale s{0u, 0.0f};
      if (newton) s = nv_block_scale_newton(am, st, rst, &ok);
      if (!ok) s = nv_block_scale_exact(am, st);
      scode = s.code;
      if (BF16 && ok && s.sdec != 0.0f)
        word = encode_octet_nv_sr_newton<WIDE>(v, s.sdec, i, seed, step);
      else
        word = encode_octet_sw<false, true, WIDE>(v, s.sdec, 0, i, seed, step);
    } else {
      static_assert(MX || SR, "NVFP4 RTN has its own kernel");
    }
    if (i < n_oct) {
      st_u32(packed + i, word);
      if ((i & (MX ? 3 : 1)) == 0) scales[i >> (MX ? 2 : 1)] = (uint8_t)scode;
    }
  }
}

// ------------------------------------------------ MXFP4 from fp32
// Thread t of workgroup b handles quads q = b 256 U + t + 256 k (k < U) of
// four elements: 16 input bytes at 16 q (one contiguous 1 KiB per load
// instruction of a wave), two code bytes at 2 q.  A 32-element block is 8
// consecutive lanes; its absmax takes three exchanges.  Codes as in
// quantize_kernel: q = x * 2^(127 - b) exactly, then the scaled converter
// (RTN) or e2m1_sr_mag with the draws of elements 4 q .. 4 q + 3, which are
// the four words of Philox counter q.
template <bool SR, bool WIDE, int U = 2>
__global__ __launch_bounds__(kThreads) void mx_quantize_f32_kernel(
    const float* __restrict__ x, int64_t n_quad, uint64_t seed, uint64_t step,
    uint16_t* __restrict__ packed, uint8_t* __restrict__ scales, int64_t blk0) {
  const int64_t base = ((int64_t)blockIdx.x + blk0) * (kThreads * U) + threadIdx.x;
  u32x4 a[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t q = base + (int64_t)k * kThreads;
    a[k] = q < n_quad ? ld_u32x4(x + 4 * q) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t q = base + (int64_t)k * kThreads;
    const float v[4] = {__uint_as_float(a[k].x), __uint_as_float(a[k].y), __uint_as_float(a[k].z),
                        __uint_as_float(a[k].w)};
    float am = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    am = fmaxf(am, lane_xor1(am));                  // every lane takes part in the exchanges
    am = fmaxf(am, lane_xor2(am));
    am = fmaxf(am, __shfl_xor(am, 4));
    const uint32_t scode = mx_scale_byte(am);
    const int shift = 127 - (int)scode;
    uint32_t code;
    if constexpr (SR) {
      uint32_t c0 = (uint32_t)q, c1 = WIDE ? (uint32_t)((uint64_t)q >> 32) : 0u;
      uint32_t c2 = (uint32_t)step, c3 = (uint32_t)(step >> 32);
      philox4x32_10(c0, c1, c2, c3, (uint32_t)seed, (uint32_t)(seed >> 32));
      const uint32_t u[4] = {c0 >> 8, c1 >> 8, c2 >> 8, c3 >> 8};
      code = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float qv = __builtin_amdgcn_ldexpf(v[j], shift);
        // an exactly positive scaled value that underflowed still rounds up when u = 0
        const bool extra = (qv == 0.0f) && (v[j] != 0.0f) && (u[j] == 0u);
        code |= (e2m1_sr_mag(fabsf(qv), u[j], extra) | sign_nibble(v[j])) << (4 * j);
      }
    } else {
      const float q0 = __builtin_amdgcn_ldexpf(v[0], shift), q1 = __builtin_amdgcn_ldexpf(v[1], shift);
      const float q2 = __builtin_amdgcn_ldexpf(v[2], shift), q3 = __builtin_amdgcn_ldexpf(v[3], shift);
      code = cvt_fp4x2_f32<1>(cvt_fp4x2_f32<0>(0u, q0, q1, 1.0f), q2, q3, 1.0f);
    }
    if (q < n_quad) {
      packed[q] = (uint16_t)code;
      if ((q & 7) == 0) scales[q >> 3] = (uint8_t)scode;
    }
  }
}

// ------------------------------------------------ NVFP4 RTN quantize
// Scale and codes from the division-free quotients, which are exact
// wherever S_t lies in [2^-100, 2^100] and the block's raw scale quotient is
// below 2^120; other blocks (a wave-uniform branch, taken only for extreme
// inputs) use IEEE divisions.
// Thread t of workgroup b owns octets b*256*U + t + 256*k, k < U.
template <bool BF16, int U = kOctets<BF16>>
__global__ __launch_bounds__(kThreads) void nv_rtn_quantize_kernel(
    const void* __restrict__ x, int64_t n_oct, const float* __restrict__ st_ptr,
    uint32_t* __restrict__ packed, uint8_t* __restrict__ scales, int64_t blk0) {
  const float st = *st_ptr;
  const bool newton = nv_newton_range(st);
  const float rst = newton ? 1.0f / st : 0.0f;
  const int64_t base = ((int64_t)blockIdx.x + blk0) * (kThreads * U) + threadIdx.x;
  u32x4 ra[U], rb[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t i = base + (int64_t)k * kThreads;
    const bool ok = i < n_oct;
    if constexpr (BF16) {
      ra[k] = ok ? ld_u32x4(static_cast<const uint8_t*>(x) + i * 16) : u32x4{0u, 0u, 0u, 0u};
    } else {
      const uint8_t* p = static_cast<const uint8_t*>(x) + i * 32;
      ra[k] = ok ? ld_u32x4(p) : u32x4{0u, 0u, 0u, 0u};
      rb[k] = ok ? ld_u32x4(p + 16) : u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t i = base + (int64_t)k * kThreads;
    float v[8];
    if constexpr (BF16) unpack_bf16x8(ra[k], v);
    else unpack_f32x8(ra[k], rb[k], v);
    // block absmax: a non-negative float orders like its bit pattern
    uint32_t amb = BF16 ? absmax_bits_bf16x8(ra[k]) << 16 : __float_as_uint(absmax8(v));
    amb = max(amb, (uint32_t)lane_xor1_i((int)amb));
    const float am = __uint_as_float(amb);
    bool ok;
    NvScale s = nv_block_scale_newton(am, st, rst, &ok);
    ok = ok && newton;
    uint32_t word = encode_octet_nv_rtn(v, s.sdec);
    if (__ballot(!ok)) {                            // wave-uniform; extreme inputs only
      if (!ok) {
        s = nv_block_scale_exact(am, st);
        word = encode_octet_sw<false, false>(v, s.sdec, 0, i, 0, 0);
      }
    }
    if (i < n_oct) {
      st_u32(packed + i, word);
      if ((i & 1) == 0) scales[i >> 1] = (uint8_t)s.code;
    }
  }
}

// ------------------------------------------------ NVFP4 from fp32
// Four elements per lane as in mx_quantize_f32_kernel (a 16-element block is
// 4 lanes: two DPP exchanges for its absmax); scale and codes as in
// nv_rtn_quantize_kernel, with the IEEE fallback behind the same wave-uniform
// branch.  SR: the four draws of a lane are the four words of Philox counter
// q (elements 4 q .. 4 q + 3), and the quotients are the division-free ones
// of encode_octet_nv_sr_newton, with IEEE divisions for a lane holding an
// element or quotient below 2^-100 or a block whose scale left the
// division-free chain.
template <bool SR, bool WIDE, int U = 2>
__global__ __launch_bounds__(kThreads) void nv_quantize_f32_kernel(
    const float* __restrict__ x, int64_t n_quad, const float* __restrict__ st_ptr, uint64_t seed,
    uint64_t step, uint16_t* __restrict__ packed, uint8_t* __restrict__ scales, int64_t blk0) {
  const float st = *st_ptr;
  const bool newton = nv_newton_range(st);
  const float rst = newton ? 1.0f / st : 0.0f;
  const int64_t base = ((int64_t)blockIdx.x + blk0) * (kThreads * U) + threadIdx.x;
  u32x4 a[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t q = base + (int64_t)k * kThreads;
    a[k] = q < n_quad ? ld_u32x4(x + 4 * q) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t q = base + (int64_t)k * kThreads;
    const float v[4] = {__uint_as_float(a[k].x), __uint_as_float(a[k].y), __uint_as_float(a[k].z),
                        __uint_as_float(a[k].w)};
    // block absmax: a non-negative float orders like its bit pattern
    uint32_t amb = __float_as_uint(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    amb = max(amb, (uint32_t)lane_xor1_i((int)amb));
    amb = max(amb, (uint32_t)lane_xor2_i((int)amb));
    const float am = __uint_as_float(amb);
    bool ok;
    NvScale s = nv_block_scale_newton(am, st, rst, &ok);
    ok = ok && newton;
    uint32_t code;
    if constexpr (SR) {
      uint32_t c0 = (uint32_t)q, c1 = WIDE ? (uint32_t)((uint64_t)q >> 32) : 0u;
      uint32_t c2 = (uint32_t)step, c3 = (uint32_t)(step >> 32);
      philox4x32_10(c0, c1, c2, c3, (uint32_t)seed, (uint32_t)(seed >> 32));
      const uint32_t u[4] = {c0 >> 8, c1 >> 8, c2 >> 8, c3 >> 8};
      if (!ok) s = nv_block_scale_exact(am, st);
      float qv[4];
      if (ok && s.sdec != 0.0f) {
        const float y = recip_rn(s.sdec);
        // |v| >= 2^-100 and |v / sdec| >= 2^-100 (zero excepted), as in encode_octet_nv_sr_newton
        const uint32_t lim = (__float_as_uint(0x1p-100f * fmaxf(1.0f, s.sdec)) << 1) - 2u;
        uint32_t small = 0xFFFFFFFFu;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qv[j] = div_rn(v[j], s.sdec, y);
          small = min(small, (__float_as_uint(v[j]) << 1) - 2u);
        }
        if (small < lim) {                              // rare: IEEE quotients
#pragma unroll
          for (int j = 0; j < 4; ++j) qv[j] = v[j] / s.sdec;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          qv[j] = (s.sdec == 0.0f) ? __builtin_copysignf(0.0f, v[j]) : v[j] / s.sdec;  // IEEE division
      }
      code = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) code |= (e2m1_sr_mag(fabsf(qv[j]), u[j], false) | sign_nibble(v[j])) << (4 * j);
    } else {
      const float y = (s.sdec == 0.0f) ? 0.0f : recip_rn(s.sdec);
      code = cvt_fp4x2_f32<1>(cvt_fp4x2_f32<0>(0u, div_rn(v[0], s.sdec, y), div_rn(v[1], s.sdec, y), 1.0f),
                              div_rn(v[2], s.sdec, y), div_rn(v[3], s.sdec, y), 1.0f);
      if (__ballot(!ok)) {                            // wave-uniform; extreme inputs only
        if (!ok) {
          s = nv_block_scale_exact(am, st);
          code = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float qv = (s.sdec == 0.0f) ? __builtin_copysignf(0.0f, v[j]) : v[j] / s.sdec;  // IEEE division
            code |= (e2m1_rtn_mag(fabsf(qv)) | sign_nibble(v[j])) << (4 * j);
          }
        }
      }
    }
    if (q < n_quad) {
      packed[q] = (uint16_t)code;
      if ((q & 3) == 0) scales[q >> 2] = (uint8_t)s.code;
    }
  }
}

// ----------------------------------------------------------- dequantize
// bf16 output of an MXFP4 octet with a normal scale byte (1 <= b <= 254).
__device__ __forceinline__ void mx_dequant_octet_hw(uint32_t w, uint32_t b, void* y, int64_t i) {
  // scale 2^(b-127) is a normal float whose exponent field is b
  const float scale = __uint_as_float(b << 23);
  u32x4 o;
  o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  st_u32x4(static_cast<uint8_t*>(y) + i * 16, o);
}

// bf16 output (fp32 output: dequantize_f32_kernel).
template <bool MX, int U = 1>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(
    const uint32_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const float* __restrict__ st_ptr, int64_t n_oct, void* __restrict__ y, int64_t blk0) {
  const float st = MX ? 1.0f : *st_ptr;
  const int64_t base = ((int64_t)blockIdx.x + blk0) * (kThreads * U) + threadIdx.x;
  uint32_t w[U], b[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t i = base + (int64_t)k * kThreads;
    const bool ok = i < n_oct;
    // plain (temporal) loads: for 4-byte code loads they stream faster than
    // non-temporal ones on gfx950
    w[k] = ok ? packed[i] : 0u;
    b[k] = ok ? scales[i >> (MX ? 2 : 1)] : 0u;
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t i = base + (int64_t)k * kThreads;
    if (i >= n_oct) continue;
    float v[8];
    if constexpr (MX) {
      if (b[k] - 1u < 254u) {
        mx_dequant_octet_hw(w[k], b[k], y, i);
        continue;
      }
      // UE8M0 0 (2^-127) and 0xFF (NaN) in software
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float e = e2m1_value((w[k] >> (4 * j)) & 15u);
        v[j] = (b[k] == 255u) ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(e, -127);
      }
    } else {
      const float sdec = e4m3_value_signed(b[k]) * st;
      e2m1x8_to_f32(w[k], 1.0f, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = v[j] * sdec;
    }
    store8<true>(y, i, v);
  }
}

// fp32 output: thread t of workgroup b handles quads q = b 256 U + t + 256 k
// (k < U) of four elements: their two code bytes at 2 q and 16 output bytes
// at 16 q, so every store instruction of a wave writes 1 KiB contiguously
// (an octet per lane writes 32 bytes in two instructions, each half-filling
// its lines).  The values are those of dequantize_kernel: the same scaled
// converter, and UE8M0 bytes 0 and 0xFF in software.
template <bool MX, int U = 2>
__global__ __launch_bounds__(kThreads) void dequantize_f32_kernel(
    const uint16_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const float* __restrict__ st_ptr, int64_t n_quad, float* __restrict__ y, int64_t blk0) {
  const float st = MX ? 1.0f : *st_ptr;
  const int64_t base = ((int64_t)blockIdx.x + blk0) * (kThreads * U) + threadIdx.x;
  uint32_t w[U], b[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t q = base + (int64_t)k * kThreads;
    const bool ok = q < n_quad;
    w[k] = ok ? (uint32_t)packed[q] : 0u;
    b[k] = ok ? scales[q >> (MX ? 3 : 2)] : 0u;
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t q = base + (int64_t)k * kThreads;
    if (q >= n_quad) continue;
    float v[4];
    if (!MX || b[k] - 1u < 254u) {
      // MXFP4: 2^(b-127) is the normal float with exponent field b
      const float scale = MX ? __uint_as_float(b[k] << 23) : 1.0f;
      const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], scale, 0);
      const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[k], scale, 1);
      v[0] = lo.x; v[1] = lo.y; v[2] = hi.x; v[3] = hi.y;
      if constexpr (!MX) {
        const float sdec = e4m3_value_signed(b[k]) * st;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = v[j] * sdec;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = e2m1_value((w[k] >> (4 * j)) & 15u);
        v[j] = (b[k] == 255u) ? __builtin_nanf("") : __builtin_amdgcn_ldexpf(e, -127);
      }
    }
    st_u32x4(y + 4 * q, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                              __float_as_uint(v[3])});
  }
}

// --------------------------------------------------- tensor amax (NVFP4)
__global__ void zero_u32_kernel(uint32_t* p) { *p = 0u; }

// max |x (+ r)| over the tensor.  The maximum of non-negative floats is
// taken on their bit patterns (which order like the values; bf16 magnitudes
// as 16-bit patterns).  At most kAmaxGrid large workgroups, each with U
// octets per thread in flight.  PART: workgroup b writes its maximum to
// out_bits[b] (a caller-side output buffer lent as scratch; a finalize
// kernel reduces them).  Otherwise each workgroup issues one atomic max on
// *out_bits, which must start at 0 (atomics on one word are serialised at
// the memory side, several ns each).
constexpr int kAmaxThreads = 1024;
constexpr int kAmaxGrid = 256;

template <bool BF16, bool RES, bool PART>
__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(const void* __restrict__ x,
                                                            const float* __restrict__ r,
                                                            int64_t n_oct,
                                                            uint32_t* __restrict__ out_bits) {
  constexpr int U = (BF16 && !RES) ? 4 : 2;
  __shared__ uint32_t part[kAmaxThreads / 64];
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kAmaxThreads * U;
  for (int64_t base = (int64_t)blockIdx.x * kAmaxThreads * U + threadIdx.x; base < n_oct;
       base += stride) {
    u32x4 a[U], b[U], c[U], d[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int64_t i = base + (int64_t)k * kAmaxThreads;
      const bool ok = i < n_oct;
      const u32x4 z = {0u, 0u, 0u, 0u};
      if constexpr (BF16) {
        a[k] = ok ? ld_u32x4_keep(static_cast<const uint8_t*>(x) + i * 16) : z;
      } else {
        a[k] = ok ? ld_u32x4_keep(static_cast<const uint8_t*>(x) + i * 32) : z;
        b[k] = ok ? ld_u32x4_keep(static_cast<const uint8_t*>(x) + i * 32 + 16) : z;
      }
      if constexpr (RES) {
        c[k] = ok ? ld_u32x4_keep(reinterpret_cast<const uint8_t*>(r) + i * 32) : z;
        d[k] = ok ? ld_u32x4_keep(reinterpret_cast<const uint8_t*>(r) + i * 32 + 16) : z;
      }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if constexpr (BF16 && !RES) {
        const uint32_t w0 = a[k].x & 0x7FFF7FFFu, w1 = a[k].y & 0x7FFF7FFFu;
        const uint32_t w2 = a[k].z & 0x7FFF7FFFu, w3 = a[k].w & 0x7FFF7FFFu;
        const uint32_t hi = max(max(w0 >> 16, w1 >> 16), max(w2 >> 16, w3 >> 16));
        const uint32_t lo = max(max(w0 & 0xFFFFu, w1 & 0xFFFFu), max(w2 & 0xFFFFu, w3 & 0xFFFFu));
        m = max(m, max(hi, lo) << 16);
      } else {
        float v[8];
        if constexpr (BF16) unpack_bf16x8(a[k], v);
        else unpack_f32x8(a[k], b[k], v);
        if constexpr (RES) {
          float rr[8];
          unpack_f32x8(c[k], d[k], rr);
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = v[j] + rr[j];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) m = max(m, __float_as_uint(v[j]) & 0x7FFFFFFFu);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t q = part[0];
    for (int w = 1; w < kAmaxThreads / 64; ++w) q = max(q, part[w]);
    if constexpr (PART) out_bits[blockIdx.x] = q;
    else atomicMax(out_bits, q);
  }
}

// S_t = fl32(A / 2688) (1 when that is 0) from the amax bits of `count`
// partial maxima; one workgroup of kAmaxGrid threads.
__global__ __launch_bounds__(kAmaxGrid) void tensor_scale_from_partials_kernel(
    const uint32_t* __restrict__ parts, int count, float* __restrict__ ts) {
  __shared__ uint32_t wmax[kAmaxGrid / 64];
  uint32_t m = threadIdx.x < (unsigned)count ? parts[threadIdx.x] : 0u;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t q = wmax[0];
    for (int w = 1; w < kAmaxGrid / 64; ++w) q = max(q, wmax[w]);
    const float s = __uint_as_float(q) / 2688.0f;
    *ts = (s == 0.0f) ? 1.0f : s;
  }
}

// S_t = fl32(A / 2688), 1 when that is 0; written over the amax in place.
__global__ void tensor_scale_finalize_kernel(float* ts) {
  float a = __uint_as_float(*reinterpret_cast<uint32_t*>(ts));
  float s = a / 2688.0f;
  *ts = (s == 0.0f) ? 1.0f : s;
}

// ------------------------------------------------- error-feedback qdq
// v = x + r, its NVFP4 codes under S_t, the dequantized W = codes * s_dec
// (rounded once to bf16 for bf16 output, the residual taken against the
// rounded value) and the new residual v - W.  Four elements per lane as in
// nv_quantize_f32_kernel (a 16-element block is 4 lanes): one 16-byte access
// of r and of an fp32 x or y per lane, 8 bytes of a bf16 one, so a wave
// instruction covers whole lines; the codes are those of that kernel.  Each
// lane reads its elements before it writes them, so x may be y and r is
// updated in place.  On 8192 x 8192 with a given S_t this took 145 us from
// fp32 x (160 us with an octet per lane, 152 us with two quads per lane,
// 167 us with two and plain loads) and 125 us from bf16 x in place (135 us
// with an octet per lane).
template <bool BF16IN, bool BF16OUT, bool RES, bool SR, bool CODES, bool WIDE, int U = 1>
__global__ __launch_bounds__(kThreads) void ef_qdq_kernel(
    const void* x, float* __restrict__ res, void* y, int64_t n_quad,
    const float* __restrict__ st_ptr, uint64_t seed, uint64_t step, uint16_t* __restrict__ packed,
    uint8_t* __restrict__ scales, int64_t blk0) {
  const float st = *st_ptr;
  const bool newton = nv_newton_range(st);
  const float rst = newton ? 1.0f / st : 0.0f;
  const int64_t base = ((int64_t)blockIdx.x + blk0) * (kThreads * U) + threadIdx.x;
  float v[U][4];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t q = base + (int64_t)k * kThreads;
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (q < n_quad) {
      if constexpr (BF16IN) {
        const u32x2 h = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(x) + 8 * q));
        a = u32x4{h.x << 16, h.x & 0xFFFF0000u, h.y << 16, h.y & 0xFFFF0000u};
      } else {
        a = ld_u32x4(static_cast<const float*>(x) + 4 * q);
      }
      if constexpr (RES) b = ld_u32x4(res + 4 * q);
    }
    v[k][0] = __uint_as_float(a.x); v[k][1] = __uint_as_float(a.y);
    v[k][2] = __uint_as_float(a.z); v[k][3] = __uint_as_float(a.w);
    if constexpr (RES) {
      v[k][0] = v[k][0] + __uint_as_float(b.x); v[k][1] = v[k][1] + __uint_as_float(b.y);
      v[k][2] = v[k][2] + __uint_as_float(b.z); v[k][3] = v[k][3] + __uint_as_float(b.w);
    }
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t q = base + (int64_t)k * kThreads;
    const float (&w)[4] = v[k];
    uint32_t amb = __float_as_uint(fmaxf(fmaxf(fabsf(w[0]), fabsf(w[1])), fmaxf(fabsf(w[2]), fabsf(w[3]))));
    amb = max(amb, (uint32_t)lane_xor1_i((int)amb));
    amb = max(amb, (uint32_t)lane_xor2_i((int)amb));
    const float am = __uint_as_float(amb);
    bool ok;
    NvScale s = nv_block_scale_newton(am, st, rst, &ok);
    ok = ok && newton;
    uint32_t code;
    if constexpr (SR) {
      uint32_t c0 = (uint32_t)q, c1 = WIDE ? (uint32_t)((uint64_t)q >> 32) : 0u;
      uint32_t c2 = (uint32_t)step, c3 = (uint32_t)(step >> 32);
      philox4x32_10(c0, c1, c2, c3, (uint32_t)seed, (uint32_t)(seed >> 32));
      const uint32_t u[4] = {c0 >> 8, c1 >> 8, c2 >> 8, c3 >> 8};
      if (!ok) s = nv_block_scale_exact(am, st);
      float qv[4];
      if (ok && s.sdec != 0.0f) {
        const float yr = recip_rn(s.sdec);
        const uint32_t lim = (__float_as_uint(0x1p-100f * fmaxf(1.0f, s.sdec)) << 1) - 2u;
        uint32_t small = 0xFFFFFFFFu;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qv[j] = div_rn(w[j], s.sdec, yr);
          small = min(small, (__float_as_uint(w[j]) << 1) - 2u);
        }
        if (small < lim) {                              // rare: IEEE quotients
#pragma unroll
          for (int j = 0; j < 4; ++j) qv[j] = w[j] / s.sdec;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          qv[j] = (s.sdec == 0.0f) ? __builtin_copysignf(0.0f, w[j]) : w[j] / s.sdec;  // IEEE division
      }
      code = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) code |= (e2m1_sr_mag(fabsf(qv[j]), u[j], false) | sign_nibble(w[j])) << (4 * j);
    } else {
      const float yr = (s.sdec == 0.0f) ? 0.0f : recip_rn(s.sdec);
      code = cvt_fp4x2_f32<1>(cvt_fp4x2_f32<0>(0u, div_rn(w[0], s.sdec, yr), div_rn(w[1], s.sdec, yr), 1.0f),
                              div_rn(w[2], s.sdec, yr), div_rn(w[3], s.sdec, yr), 1.0f);
      if (__ballot(!ok)) {                            // wave-uniform; extreme inputs only
        if (!ok) {
          s = nv_block_scale_exact(am, st);
          code = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float qv = (s.sdec == 0.0f) ? __builtin_copysignf(0.0f, w[j]) : w[j] / s.sdec;  // IEEE division
            code |= (e2m1_rtn_mag(fabsf(qv)) | sign_nibble(w[j])) << (4 * j);
          }
        }
      }
    }
    if (q >= n_quad) continue;
    const f32x2 d01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 0);
    const f32x2 d23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, 1.0f, 1);
    float o[4] = {d01.x * s.sdec, d01.y * s.sdec, d23.x * s.sdec, d23.y * s.sdec};
    if constexpr (BF16OUT) {
      // round to bf16 once; the residual is taken against the rounded values
      const uint32_t p0 = pack_bf16x2(o[0], o[1]), p1 = pack_bf16x2(o[2], o[3]);
      o[0] = __uint_as_float(p0 << 16); o[1] = __uint_as_float(p0 & 0xFFFF0000u);
      o[2] = __uint_as_float(p1 << 16); o[3] = __uint_as_float(p1 & 0xFFFF0000u);
      __builtin_nontemporal_store(u32x2{p0, p1}, reinterpret_cast<u32x2*>(static_cast<uint8_t*>(y) + q * 8));
    } else {
      st_u32x4(static_cast<float*>(y) + 4 * q,
               u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])});
    }
    if constexpr (RES)
      st_u32x4(res + 4 * q, u32x4{__float_as_uint(w[0] - o[0]), __float_as_uint(w[1] - o[1]),
                                  __float_as_uint(w[2] - o[2]), __float_as_uint(w[3] - o[3])});
    if constexpr (CODES) {
      packed[q] = (uint16_t)code;
      if ((q & 3) == 0) scales[q >> 2] = (uint8_t)s.code;
    }
  }
}

// ------------------------------------------------------------ launchers
// S_t into *ts.  With `scratch` (an output buffer of the call that is
// written only after S_t is known, of scratch_bytes bytes) the workgroups'
// maxima go there and one finalize kernel reduces them: two launches, no
// atomics.  Otherwise: zero, atomic maxima, finalize.
int launch_tensor_scale(const void* x, bool bf16, const float* res, int64_t n_oct, float* ts,
                        void* scratch, int64_t scratch_bytes, hipStream_t st) {
  const int u = (bf16 && !res) ? 4 : 2;
  int64_t g = (n_oct + (int64_t)kAmaxThreads * u - 1) / ((int64_t)kAmaxThreads * u);
  if (g > kAmaxGrid) g = kAmaxGrid;
  const dim3 grid((unsigned)g), blk(kAmaxThreads);
  const bool part = scratch != nullptr && scratch_bytes >= 4 * g;
  uint32_t* bits = part ? static_cast<uint32_t*>(scratch) : reinterpret_cast<uint32_t*>(ts);
  if (!part) hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(1), 0, st, bits);
#define FP4MI_AMAX(B, R, P) \
  hipLaunchKernelGGL((amax_kernel<B, R, P>), grid, blk, 0, st, x, res, n_oct, bits)
  if (part) {
    if (bf16) { if (res) FP4MI_AMAX(true, true, true); else FP4MI_AMAX(true, false, true); }
    else      { if (res) FP4MI_AMAX(false, true, true); else FP4MI_AMAX(false, false, true); }
    hipLaunchKernelGGL(tensor_scale_from_partials_kernel, dim3(1), dim3(kAmaxGrid), 0, st, bits,
                       (int)g, ts);
  } else {
    if (bf16) { if (res) FP4MI_AMAX(true, true, false); else FP4MI_AMAX(true, false, false); }
    else      { if (res) FP4MI_AMAX(false, true, false); else FP4MI_AMAX(false, false, false); }
    hipLaunchKernelGGL(tensor_scale_finalize_kernel, dim3(1), dim3(1), 0, st, ts);
  }
#undef FP4MI_AMAX
  return launch_status();
}

template <bool BF16, bool MX>
void launch_quantize_t(bool sr, const void* x, int64_t n_oct, const float* ts, uint64_t seed,
                       uint64_t step, uint32_t* packed, uint8_t* scales, hipStream_t st) {
  if constexpr (!BF16) {
    // fp32 input: one lane per four elements (MXFP4 both roundings, NVFP4 SR
    // and RTN), two quads per thread
    const int64_t n_quad = 2 * n_oct;
    const int64_t g4 = blocks_for(n_quad, 2);
    const float* xf = static_cast<const float*>(x);
    uint16_t* p16 = reinterpret_cast<uint16_t*>(packed);
    const bool wide = n_quad > (int64_t(1) << 32);   // SR counters q need their high word
    if constexpr (MX) {
      if (!sr) launch_1d(mx_quantize_f32_kernel<false, false>, g4, kThreads, st, xf, n_quad, seed, step, p16, scales);
      else if (!wide) launch_1d(mx_quantize_f32_kernel<true, false>, g4, kThreads, st, xf, n_quad, seed, step, p16, scales);
      else launch_1d(mx_quantize_f32_kernel<true, true>, g4, kThreads, st, xf, n_quad, seed, step, p16, scales);
    } else {
      if (!sr) launch_1d(nv_quantize_f32_kernel<false, false>, g4, kThreads, st, xf, n_quad, ts, seed, step, p16, scales);
      else if (!wide) launch_1d(nv_quantize_f32_kernel<true, false>, g4, kThreads, st, xf, n_quad, ts, seed, step, p16, scales);
      else launch_1d(nv_quantize_f32_kernel<true, true>, g4, kThreads, st, xf, n_quad, ts, seed, step, p16, scales);
    }
  } else {
    const int64_t g = blocks_for(n_oct, kOctets<BF16>);
    // SR counters 2 i + 1 below 2^32: their second word is 0 throughout
    if (sr && 2 * n_oct <= (int64_t(1) << 32))
      launch_1d(quantize_kernel<BF16, MX, true, kOctets<BF16>, false>, g, kThreads, st, x, n_oct, ts,
                seed, step, packed, scales);
    else if (sr)
      launch_1d(quantize_kernel<BF16, MX, true>, g, kThreads, st, x, n_oct, ts, seed, step, packed, scales);
    else if (MX)
      // three octets per thread: measured 1% faster than four on 4096 x 7168,
      // with the input in HBM or in the Infinity Cache
      launch_1d(quantize_kernel<BF16, true, false, 3>, blocks_for(n_oct, 3), kThreads, st, x, n_oct,
                ts, seed, step, packed, scales);
    else
      launch_1d(nv_rtn_quantize_kernel<BF16>, g, kThreads, st, x, n_oct, ts, packed, scales);
  }
}

template <bool BF16IN, bool BF16OUT>
void launch_ef_t(bool res, bool sr, bool codes, const void* x, float* r, void* y, int64_t n_oct,
                 const float* ts, uint64_t seed, uint64_t step, uint32_t* packed, uint8_t* scales,
                 hipStream_t st) {
  const int64_t n_quad = 2 * n_oct;
  const int64_t g4 = blocks_for(n_quad, 1);
  uint16_t* p16 = reinterpret_cast<uint16_t*>(packed);
  const bool wide = n_quad > (int64_t(1) << 32);     // SR counters q need their high word
#define FP4MI_EF(RES, SR, CODES, WIDE)                                                           \
  launch_1d(ef_qdq_kernel<BF16IN, BF16OUT, RES, SR, CODES, WIDE>, g4, kThreads, st, x, r, y, n_quad, \
            ts, seed, step, p16, scales)
#define FP4MI_EF_SR(RES, CODES) \
  do { if (wide) FP4MI_EF(RES, true, CODES, true); else FP4MI_EF(RES, true, CODES, false); } while (0)
  if (res) {
    if (sr) { if (codes) FP4MI_EF_SR(true, true); else FP4MI_EF_SR(true, false); }
    else    { if (codes) FP4MI_EF(true, false, true, false); else FP4MI_EF(true, false, false, false); }
  } else {
    if (sr) { if (codes) FP4MI_EF_SR(false, true); else FP4MI_EF_SR(false, false); }
    else    { if (codes) FP4MI_EF(false, false, true, false); else FP4MI_EF(false, false, false, false); }
  }
#undef FP4MI_EF_SR
#undef FP4MI_EF
}


}  // namespace
}  // namespace fp4mi

using namespace fp4mi;

extern "C" int fp4_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int fmt,
                            int rounding, uint64_t seed, uint64_t step, int tscale_mode,
                            float* tensor_scale, uint8_t* packed, uint8_t* scales, void* stream) {
  int es = dtype_size(dtype);
  if (!es) return FP4_EDTYPE;
  if (fmt != FP4_FMT_NVFP4 && fmt != FP4_FMT_MXFP4) return FP4_EINVAL;
  if (rounding != FP4_ROUND_RTN && rounding != FP4_ROUND_SR) return FP4_EINVAL;
  const bool mx = fmt == FP4_FMT_MXFP4;
  if (!mx && tscale_mode != FP4_TSCALE_COMPUTE && tscale_mode != FP4_TSCALE_GIVEN) return FP4_EINVAL;
  int64_t n;
  if (!checked_count(rows, cols, &n)) return FP4_ESHAPE;
  const int blk = mx ? 32 : 16;
  if (cols % blk) return FP4_ESHAPE;
  if (n == 0) return FP4_OK;
  if (!x || !packed || !scales || (!mx && !tensor_scale)) return FP4_EINVAL;
  if (!is_aligned(x, 16) || !is_aligned(packed, 4) || (!mx && !is_aligned(tensor_scale, 4)))
    return FP4_EALIGN;
  const int64_t xb = n * es, pb = n / 2, sb = n / blk;
  if (overlaps(packed, pb, x, xb) || overlaps(scales, sb, x, xb) || overlaps(packed, pb, scales, sb))
    return FP4_EOVERLAP;
  if (!mx && (overlaps(tensor_scale, 4, x, xb) || overlaps(tensor_scale, 4, packed, pb) ||
              overlaps(tensor_scale, 4, scales, sb)))
    return FP4_EOVERLAP;
  clear_stale_error();
  hipStream_t st = as_stream(stream);
  const bool bf16 = dtype == FP4_DTYPE_BF16, sr = rounding == FP4_ROUND_SR;
  const int64_t n_oct = n / 8;
  if (!mx && tscale_mode == FP4_TSCALE_COMPUTE) {
    // the packed codes are written only after S_t: their buffer holds the
    // amax pass's partial maxima meanwhile
    int rc = launch_tensor_scale(x, bf16, nullptr, n_oct, tensor_scale, packed, pb, st);
    if (rc) return rc;
  }
  uint32_t* pk = reinterpret_cast<uint32_t*>(packed);
  if (bf16) {
    if (mx) launch_quantize_t<true, true>(sr, x, n_oct, tensor_scale, seed, step, pk, scales, st);
    else    launch_quantize_t<true, false>(sr, x, n_oct, tensor_scale, seed, step, pk, scales, st);
  } else {
    if (mx) launch_quantize_t<false, true>(sr, x, n_oct, tensor_scale, seed, step, pk, scales, st);
    else    launch_quantize_t<false, false>(sr, x, n_oct, tensor_scale, seed, step, pk, scales, st);
  }
  return launch_status();
}

extern "C" int fp4_dequantize(const uint8_t* packed, const uint8_t* scales,
                              const float* tensor_scale, int64_t rows, int64_t cols, int fmt,
                              void* y, int out_dtype, void* stream) {
  int es = dtype_size(out_dtype);
  if (!es) return FP4_EDTYPE;
  if (fmt != FP4_FMT_NVFP4 && fmt != FP4_FMT_MXFP4) return FP4_EINVAL;
  const bool mx = fmt == FP4_FMT_MXFP4;
  int64_t n;
  if (!checked_count(rows, cols, &n)) return FP4_ESHAPE;
  const int blk = mx ? 32 : 16;
  if (cols % blk) return FP4_ESHAPE;
  if (n == 0) return FP4_OK;
  if (!packed || !scales || !y || (!mx && !tensor_scale)) return FP4_EINVAL;
  if (!is_aligned(y, 16) || !is_aligned(packed, 4) || (!mx && !is_aligned(tensor_scale, 4)))
    return FP4_EALIGN;
  const int64_t yb = n * es;
  if (overlaps(y, yb, packed, n / 2) || overlaps(y, yb, scales, n / blk) ||
      (!mx && overlaps(y, yb, tensor_scale, 4)))
    return FP4_EOVERLAP;
  clear_stale_error();
  hipStream_t st = as_stream(stream);
  const int64_t n_oct = n / 8;
  // two octets per thread: two code loads in flight per lane
  constexpr int U = 2;
  const uint32_t* pk = reinterpret_cast<const uint32_t*>(packed);
  if (out_dtype == FP4_DTYPE_BF16) {
    // MXFP4 to bf16: eight octets per thread, all eight code loads issued
    // before the first store.  With codes resident in HBM (4096 x 7168,
    // inputs rotating over 546 MB) this measured 13.2 us against 14.0 us
    // with two octets per thread; with codes still in the Infinity Cache two
    // octets are faster (11.6 us against 12.5 us).
    constexpr int UM = 8;
    if (mx) launch_1d(dequantize_kernel<true, UM>, blocks_for(n_oct, UM), kThreads, st, pk, scales, tensor_scale, n_oct, y);
    else    launch_1d(dequantize_kernel<false, U>, blocks_for(n_oct, U), kThreads, st, pk, scales, tensor_scale, n_oct, y);
  } else {
    const int64_t n_quad = 2 * n_oct;
    const int64_t g4 = blocks_for(n_quad, U);
    const uint16_t* p16 = reinterpret_cast<const uint16_t*>(packed);
    float* yf = static_cast<float*>(y);
    if (mx) launch_1d(dequantize_f32_kernel<true, U>, g4, kThreads, st, p16, scales, tensor_scale, n_quad, yf);
    else    launch_1d(dequantize_f32_kernel<false, U>, g4, kThreads, st, p16, scales, tensor_scale, n_quad, yf);
  }
  return launch_status();
}

extern "C" int fp4_errfeedback_qdq(const void* x, int dtype, int64_t rows, int64_t cols,
                                   float* residual, void* y, int out_dtype, int rounding,
                                   uint64_t seed, uint64_t step, int tscale_mode,
                                   float* tensor_scale, uint8_t* packed, uint8_t* scales,
                                   void* stream) {
  int es = dtype_size(dtype), eo = dtype_size(out_dtype);
  if (!es || !eo) return FP4_EDTYPE;
  if (rounding != FP4_ROUND_RTN && rounding != FP4_ROUND_SR) return FP4_EINVAL;
  if (tscale_mode != FP4_TSCALE_COMPUTE && tscale_mode != FP4_TSCALE_GIVEN) return FP4_EINVAL;
  int64_t n;
  if (!checked_count(rows, cols, &n)) return FP4_ESHAPE;
  if (cols % 16) return FP4_ESHAPE;
  if (n == 0) return FP4_OK;
  if (!x || !y || !tensor_scale) return FP4_EINVAL;
  if ((packed == nullptr) != (scales == nullptr)) return FP4_EINVAL;
  if (!is_aligned(x, 16) || !is_aligned(y, 16) || (residual && !is_aligned(residual, 16)) ||
      !is_aligned(tensor_scale, 4) || (packed && !is_aligned(packed, 4)))
    return FP4_EALIGN;
  const int64_t xb = n * es, yb = n * eo, rb = n * 4, pb = n / 2, sb = n / 16;
  const bool in_place = (y == x) && (dtype == out_dtype);
  if (!in_place && overlaps(y, yb, x, xb)) return FP4_EOVERLAP;
  if (residual && (overlaps(residual, rb, x, xb) || overlaps(residual, rb, y, yb))) return FP4_EOVERLAP;
  const void* outs[3] = {packed, scales, tensor_scale};
  const int64_t outn[3] = {pb, sb, 4};
  for (int k = 0; k < 3; ++k) {
    if (overlaps(outs[k], outn[k], x, xb) || overlaps(outs[k], outn[k], y, yb) ||
        (residual && overlaps(outs[k], outn[k], residual, rb)))
      return FP4_EOVERLAP;
    for (int l = k + 1; l < 3; ++l)
      if (overlaps(outs[k], outn[k], outs[l], outn[l])) return FP4_EOVERLAP;
  }
  clear_stale_error();
  hipStream_t st = as_stream(stream);
  const bool bf16 = dtype == FP4_DTYPE_BF16, obf16 = out_dtype == FP4_DTYPE_BF16;
  const bool sr = rounding == FP4_ROUND_SR, codes = packed != nullptr;
  const int64_t n_oct = n / 8;
  if (tscale_mode == FP4_TSCALE_COMPUTE) {
    // the amax partials go to an output the encode pass only writes: the
    // packed codes if requested, else y unless y is x
    void* scratch = packed ? static_cast<void*>(packed) : (in_place ? nullptr : y);
    const int64_t scratch_bytes = packed ? pb : (in_place ? 0 : yb);
    int rc = launch_tensor_scale(x, bf16, residual, n_oct, tensor_scale, scratch, scratch_bytes, st);
    if (rc) return rc;
  }
  uint32_t* pk = reinterpret_cast<uint32_t*>(packed);
  const bool res = residual != nullptr;
  if (bf16) {
    if (obf16) launch_ef_t<true, true>(res, sr, codes, x, residual, y, n_oct, tensor_scale, seed, step, pk, scales, st);
    else       launch_ef_t<true, false>(res, sr, codes, x, residual, y, n_oct, tensor_scale, seed, step, pk, scales, st);
  } else {
    if (obf16) launch_ef_t<false, true>(res, sr, codes, x, residual, y, n_oct, tensor_scale, seed, step, pk, scales, st);
    else       launch_ef_t<false, false>(res, sr, codes, x, residual, y, n_oct, tensor_scale, seed, step, pk, scales, st);
  }
  return launch_status();
}
