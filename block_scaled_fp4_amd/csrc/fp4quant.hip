// FP4Quant group codec for gfx950: RMS pre-scale, normalized Walsh-Hadamard
// transform, absmax-to-6 scale, E2M1 RTN, two codes per byte; and the
// receiver (unpack, dequantize, inverse transform).
//
// "FP4Quant speeds up GPU communication, with a measurable accuracy
// trade-off", sections "Why four bits need more than rounding" and "Making
// compression cheap enough to help".
//
// A group of G elements is held by LPG = G / EPL consecutive lanes of one
// wavefront, EPL (8 or 16) contiguous elements per lane.  The first log2(EPL)
// butterfly stages run in registers; the remaining log2(LPG) stages exchange
// with the partner lane (lane ^ m): DPP quad permutes for m = 1, 2 and
// ds_bpermute-based shuffles above that, so no LDS staging or barrier is
// needed for any G <= 64 * EPL.
//
// Encoder arithmetic.  With w = H x (unnormalised, fp32 butterflies):
//   z = H (x / s1) / sqrt(G) = w / (s1 sqrt(G)),  max|z| / 6 = s2,
//   z / s2 = 6 w / max|w|,   s2 = max|w| / (6 sqrt(G) s1),
// so the codes never depend on s1 and the transform runs on the raw input.
// Receiver arithmetic.  With c2 = 2 * e2m1(code) (integers in [-12, 12]),
//   x' = s1 * H(e2m1 * s2) / sqrt(G) = (H c2) * (s1 s2 / (2 sqrt(G))),
// and H c2 is computed exactly (integer-valued fp32 butterflies).
#include "device_common.hpp"
#include "host_common.hpp"

namespace fp4mi {
namespace {

template <int M>
__device__ __forceinline__ float xlane(float v) {
  if constexpr (M == 1) return lane_xor1(v);
  else if constexpr (M == 2) return lane_xor2(v);
  else return __shfl_xor(v, M);
}
// In-register butterflies over the EPL elements of a lane (natural order).
template <int EPL, typename T>
__device__ __forceinline__ void wht_local(T (&v)[EPL]) {
#pragma unroll
  for (int h = 1; h < EPL; h <<= 1) {
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      if ((j & h) == 0) {
        T a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

// Cross-lane butterfly stage with partner lane ^ M: the lower lane keeps
// a + b, the upper lane b' = a - b (its own value is b, the partner's a).
template <int M, int EPL>
__device__ __forceinline__ void wht_stage(float (&v)[EPL], bool upper) {
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    float p = xlane<M>(v[j]);
    v[j] = upper ? (p - v[j]) : (v[j] + p);
  }
}
template <int LPG, int EPL>
__device__ __forceinline__ void wht_cross(float (&v)[EPL], int lane) {
  if constexpr (LPG > 1) wht_stage<1, EPL>(v, lane & 1);
  if constexpr (LPG > 2) wht_stage<2, EPL>(v, lane & 2);
  if constexpr (LPG > 4) wht_stage<4, EPL>(v, lane & 4);
  if constexpr (LPG > 8) wht_stage<8, EPL>(v, lane & 8);
  if constexpr (LPG > 16) wht_stage<16, EPL>(v, lane & 16);
  if constexpr (LPG > 32) wht_stage<32, EPL>(v, lane & 32);
}
// Butterfly (pairwise) reductions across the LPG lanes of a group.
template <int LPG>
__device__ __forceinline__ float group_sum(float s) {
  if constexpr (LPG > 1) s = s + xlane<1>(s);
  if constexpr (LPG > 2) s = s + xlane<2>(s);
  if constexpr (LPG > 4) s = s + xlane<4>(s);
  if constexpr (LPG > 8) s = s + xlane<8>(s);
  if constexpr (LPG > 16) s = s + xlane<16>(s);
  if constexpr (LPG > 32) s = s + xlane<32>(s);
  return s;
}
template <int LPG>
__device__ __forceinline__ float group_max(float s) {
  if constexpr (LPG > 1) s = fmaxf(s, xlane<1>(s));
  if constexpr (LPG > 2) s = fmaxf(s, xlane<2>(s));
  if constexpr (LPG > 4) s = fmaxf(s, xlane<4>(s));
  if constexpr (LPG > 8) s = fmaxf(s, xlane<8>(s));
  if constexpr (LPG > 16) s = fmaxf(s, xlane<16>(s));
  if constexpr (LPG > 32) s = fmaxf(s, xlane<32>(s));
  return s;
}

// Pairwise sum of squares of a lane's elements.
template <int EPL>
__device__ __forceinline__ float sumsq(const float (&v)[EPL]) {
  float t[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) t[j] = v[j] * v[j];
#pragma unroll
  for (int h = 1; h < EPL; h <<= 1)
#pragma unroll
    for (int j = 0; j < EPL; j += 2 * h) t[j] = t[j] + t[j + h];
  return t[0];
}

// Per-group encode of the EPL elements a lane holds (all lanes of the wave
// take part: the cross-lane stages need every lane of the group).
template <int EPL, int LPG>
__device__ __forceinline__ void encode_lane(float (&v)[EPL], int lane, float inv_g, float c_s2,
                                            uint32_t (&words)[EPL / 8], float* s1o, float* s2o) {
  const float ss = group_sum<LPG>(sumsq<EPL>(v));
  wht_local<EPL>(v);
  wht_cross<LPG, EPL>(v, lane);
  float mx = 0.0f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) mx = fmaxf(mx, fabsf(v[j]));
  mx = group_max<LPG>(mx);
  const bool zero = (ss == 0.0f) || (mx == 0.0f);
  const float s1 = __builtin_sqrtf(ss * inv_g);
  const float rq = zero ? 0.0f : 6.0f / mx;
#pragma unroll
  for (int k = 0; k < EPL / 8; ++k) {
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = v[8 * k + j] * rq;     // +-0 when zero: code 0 or 8
    words[k] = zero ? 0u : rtn8_unit(q);
  }
  *s1o = zero ? 0.0f : s1;
  *s2o = zero ? 0.0f : (mx * c_s2) / s1;
}

// Thread t of workgroup b owns lane-items b*256*U + t + 256*k (k < U); each
// lane-item is EPL consecutive elements, LPG consecutive lane-items a group.
template <bool BF16, int EPL, int LPG>
__global__ __launch_bounds__(kThreads) void fp4quant_encode_kernel(
    const void* __restrict__ x, int64_t n_lane, float inv_g, float c_s2,
    uint32_t* __restrict__ packed, float* __restrict__ s_rms, float* __restrict__ s_abs) {
  constexpr int U = (EPL == 8) ? 2 : 1;
  constexpr int OCT = EPL / 8;
  const int lane = threadIdx.x & 63;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * U) + threadIdx.x;
  float v[U][EPL];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t t = base + (int64_t)k * kThreads;
#pragma unroll
    for (int o = 0; o < OCT; ++o) {
      float e[8];
      if (t < n_lane) load8<BF16>(x, t * OCT + o, e);
      else for (int j = 0; j < 8; ++j) e[j] = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[k][8 * o + j] = e[j];
    }
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t t = base + (int64_t)k * kThreads;
    uint32_t words[OCT];
    float s1, s2;
    encode_lane<EPL, LPG>(v[k], lane, inv_g, c_s2, words, &s1, &s2);
    if (t < n_lane) {
#pragma unroll
      for (int o = 0; o < OCT; ++o) st_u32(packed + t * OCT + o, words[o]);
      if ((lane & (LPG - 1)) == 0) {
        s_rms[t / LPG] = s1;
        s_abs[t / LPG] = s2;
      }
    }
  }
}

template <bool BF16OUT, int EPL, int LPG>
__global__ __launch_bounds__(kThreads) void fp4quant_decode_kernel(
    const uint32_t* __restrict__ packed, const float* __restrict__ s_rms,
    const float* __restrict__ s_abs, int64_t n_lane, float c_dec, void* __restrict__ y) {
  constexpr int U = (EPL == 8) ? 2 : 1;
  constexpr int OCT = EPL / 8;
  const int lane = threadIdx.x & 63;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * U) + threadIdx.x;
  uint32_t w[U][OCT];
  float f[U];
  // 2 * e2m1 values are integers in [-12, 12]; every partial sum of the
  // transform is an integer below 2^14, so fp32 butterflies on them are exact.
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t t = base + (int64_t)k * kThreads;
    const bool ok = t < n_lane;
#pragma unroll
    for (int o = 0; o < OCT; ++o) w[k][o] = ok ? packed[t * OCT + o] : 0u;
    f[k] = ok ? (s_rms[t / LPG] * s_abs[t / LPG]) * c_dec : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t t = base + (int64_t)k * kThreads;
    float c[EPL];
#pragma unroll
    for (int o = 0; o < OCT; ++o) {
      float e[8];
      e2m1x8_to_f32(w[k][o], 2.0f, e);
#pragma unroll
      for (int j = 0; j < 8; ++j) c[8 * o + j] = e[j];
    }
    wht_local<EPL>(c);
    wht_cross<LPG, EPL>(c, lane);
    if (t >= n_lane) continue;
#pragma unroll
    for (int o = 0; o < OCT; ++o) {
      float out[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) out[j] = c[8 * o + j] * f[k];
      store8<BF16OUT>(y, t * OCT + o, out);
    }
  }
}

template <bool BF16>
void launch_encode(int G, const void* x, int64_t n, uint32_t* pk, float* s1, float* s2,
                   hipStream_t st) {
  const float inv_g = 1.0f / (float)G;
  const float c_s2 = (float)(1.0 / (6.0 * __builtin_sqrt((double)G)));
#define FP4MI_ENC(EPL, LPG)                                                                   \
  {                                                                                           \
    int64_t nl = n / EPL;                                                                     \
    hipLaunchKernelGGL((fp4quant_encode_kernel<BF16, EPL, LPG>),                              \
                       dim3((unsigned)blocks_for(nl, EPL == 8 ? 2 : 1)),                      \
                       dim3(kThreads), 0, st, x, nl, inv_g, c_s2, pk, s1, s2);                 \
  }
  switch (G) {
    case 16: FP4MI_ENC(8, 2); break;
    case 32: FP4MI_ENC(8, 4); break;
    case 64: FP4MI_ENC(8, 8); break;
    case 128: FP4MI_ENC(8, 16); break;
    case 256: FP4MI_ENC(8, 32); break;
    case 512: FP4MI_ENC(8, 64); break;
    case 1024: FP4MI_ENC(16, 64); break;
  }
#undef FP4MI_ENC
}

template <bool BF16OUT>
void launch_decode(int G, const uint32_t* pk, const float* s1, const float* s2, int64_t n, void* y,
                   hipStream_t st) {
  const float c_dec = (float)(0.5 / __builtin_sqrt((double)G));
#define FP4MI_DEC(EPL, LPG)                                                                   \
  {                                                                                           \
    int64_t nl = n / EPL;                                                                     \
    hipLaunchKernelGGL((fp4quant_decode_kernel<BF16OUT, EPL, LPG>),                           \
                       dim3((unsigned)blocks_for(nl, EPL == 8 ? 2 : 1)),                      \
                       dim3(kThreads), 0, st, pk, s1, s2, nl, c_dec, y);                      \
  }
  switch (G) {
    case 16: FP4MI_DEC(8, 2); break;
    case 32: FP4MI_DEC(8, 4); break;
    case 64: FP4MI_DEC(8, 8); break;
    case 128: FP4MI_DEC(8, 16); break;
    case 256: FP4MI_DEC(8, 32); break;
    case 512: FP4MI_DEC(8, 64); break;
    case 1024: FP4MI_DEC(16, 64); break;
  }
#undef FP4MI_DEC
}

bool valid_group(int32_t G) { return G >= 16 && G <= 1024 && (G & (G - 1)) == 0; }

}  // namespace
}  // namespace fp4mi

using namespace fp4mi;

extern "C" int fp4quant_encode(const void* x, int dtype, int64_t rows, int64_t cols, int32_t group,
                               uint8_t* packed, float* s_rms, float* s_abs, void* stream) {
  int es = dtype_size(dtype);
  if (!es) return FP4_EDTYPE;
  if (!valid_group(group)) return FP4_EINVAL;
  int64_t n;
  if (!checked_count(rows, cols, &n)) return FP4_ESHAPE;
  if (cols % group) return FP4_ESHAPE;
  if (n == 0) return FP4_OK;
  if (!x || !packed || !s_rms || !s_abs) return FP4_EINVAL;
  if (!is_aligned(x, 16) || !is_aligned(packed, 4) || !is_aligned(s_rms, 4) || !is_aligned(s_abs, 4))
    return FP4_EALIGN;
  const int64_t xb = n * es, pb = n / 2, gb = (n / group) * 4;
  if (overlaps(packed, pb, x, xb) || overlaps(s_rms, gb, x, xb) || overlaps(s_abs, gb, x, xb) ||
      overlaps(packed, pb, s_rms, gb) || overlaps(packed, pb, s_abs, gb) ||
      overlaps(s_rms, gb, s_abs, gb))
    return FP4_EOVERLAP;
  if (blocks_for(n / 8, 1) > 0x7FFFFFFF) return FP4_ESHAPE;
  hipStream_t st = as_stream(stream);
  uint32_t* pk = reinterpret_cast<uint32_t*>(packed);
  if (dtype == FP4_DTYPE_BF16) launch_encode<true>(group, x, n, pk, s_rms, s_abs, st);
  else launch_encode<false>(group, x, n, pk, s_rms, s_abs, st);
  return launch_status();
}

extern "C" int fp4quant_decode(const uint8_t* packed, const float* s_rms, const float* s_abs,
                               int64_t rows, int64_t cols, int32_t group, void* y, int out_dtype,
                               void* stream) {
  int es = dtype_size(out_dtype);
  if (!es) return FP4_EDTYPE;
  if (!valid_group(group)) return FP4_EINVAL;
  int64_t n;
  if (!checked_count(rows, cols, &n)) return FP4_ESHAPE;
  if (cols % group) return FP4_ESHAPE;
  if (n == 0) return FP4_OK;
  if (!packed || !s_rms || !s_abs || !y) return FP4_EINVAL;
  if (!is_aligned(y, 16) || !is_aligned(packed, 4) || !is_aligned(s_rms, 4) || !is_aligned(s_abs, 4))
    return FP4_EALIGN;
  const int64_t yb = n * es, gb = (n / group) * 4;
  if (overlaps(y, yb, packed, n / 2) || overlaps(y, yb, s_rms, gb) || overlaps(y, yb, s_abs, gb))
    return FP4_EOVERLAP;
  if (blocks_for(n / 8, 1) > 0x7FFFFFFF) return FP4_ESHAPE;
  hipStream_t st = as_stream(stream);
  const uint32_t* pk = reinterpret_cast<const uint32_t*>(packed);
  if (out_dtype == FP4_DTYPE_BF16) launch_decode<true>(group, pk, s_rms, s_abs, n, y, st);
  else launch_decode<false>(group, pk, s_rms, s_abs, n, y, st);
  return launch_status();
}
