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

// Stochastic rounding of eight z / s2 values (|q| <= 6 up to rounding) with
// the draws of global octet oi of the stream keyed by (seed, step): the
// rounding rule of the NVFP4 path applied to the transformed elements.
template <bool WIDE>
__device__ __forceinline__ uint32_t sr8_octet(const float (&q)[8], int64_t oi, uint64_t seed,
                                              uint64_t step) {
  uint32_t u[8];
  sr_draws8<WIDE>(oi, seed, step, u);
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) w |= (e2m1_sr_mag(fabsf(q[j]), u[j], false) | sign_nibble(q[j])) << (4 * j);
  return w;
}

// Per-group encode of the EPL elements a lane holds (all lanes of the wave
// take part: the cross-lane stages and the ballot need every lane).  A group
// whose sum of squares leaves [2^-100, 2^126) (tiny, huge or zero groups) is
// first scaled by a power of two that brings its largest element to [1, 2):
// codes and s2 do not change under such scaling, s1 is scaled back exactly.
template <int EPL, int LPG, bool SR, bool WIDE>
__device__ __forceinline__ void encode_lane(float (&v)[EPL], int lane, float inv_g, float c_s2,
                                            uint32_t (&words)[EPL / 8], float* s1o, float* s2o,
                                            int64_t oct0, uint64_t seed, uint64_t step) {
  float ss = group_sum<LPG>(sumsq<EPL>(v));
  int e = 0;
  const bool odd = !(ss >= 0x1p-100f && ss < 0x1p+126f);
  if (__builtin_amdgcn_ballot_w64(odd)) {            // rare: some group of the wave
    float mxx = 0.0f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) mxx = fmaxf(mxx, fabsf(v[j]));
    mxx = group_max<LPG>(mxx);
    e = (odd && mxx > 0.0f) ? __builtin_amdgcn_frexp_expf(mxx) - 1 : 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) v[j] = __builtin_amdgcn_ldexpf(v[j], -e);
    ss = group_sum<LPG>(sumsq<EPL>(v));
  }
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
    if constexpr (SR) words[k] = zero ? 0u : sr8_octet<WIDE>(q, oct0 + k, seed, step);
    else words[k] = zero ? 0u : rtn8_unit(q);
  }
  *s1o = zero ? 0.0f : __builtin_amdgcn_ldexpf(s1, e);
  *s2o = zero ? 0.0f : (mx * c_s2) / s1;
}

// Thread t of workgroup b owns lane-items b*256*U + t + 256*k (k < U); each
// lane-item is EPL consecutive elements, LPG consecutive lane-items a group.
template <bool BF16, int EPL, int LPG, bool SR, bool WIDE>
__global__ __launch_bounds__(kThreads) void fp4quant_encode_kernel(
    const void* __restrict__ x, int64_t n_lane, float inv_g, float c_s2,
    uint32_t* __restrict__ packed, float* __restrict__ s_rms, float* __restrict__ s_abs,
    uint64_t seed, uint64_t step, int64_t blk0) {
  constexpr int U = (EPL == 8) ? 2 : 1;
  constexpr int OCT = EPL / 8;
  const int lane = threadIdx.x & 63;
  const int64_t base = ((int64_t)blockIdx.x + blk0) * (kThreads * U) + threadIdx.x;
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
    encode_lane<EPL, LPG, SR, WIDE>(v[k], lane, inv_g, c_s2, words, &s1, &s2, t * OCT, seed, step);
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

// The receiver's per-group factor s1 s2 / (2 sqrt(G)), formed as
// s1 * (s2 c_dec).  For the scales the encoder emits (s2 = max|z| / 6 with
// z of unit RMS, so 1/6 <= s2 <= sqrt(G) / 6) s2 c_dec lies in
// [1 / (12 sqrt(G)), 1/12] and the product never overflows.  For
// 0 < s1 < 2^-64 it would lose precision to gradual underflow, so it is
// returned scaled by 2^64 (*tiny set) and the outputs are scaled back, each
// rounded once more at the end.
constexpr int kTinyShift = 64;
__device__ __forceinline__ float group_factor(float s1, float s2, float c_dec, bool* tiny) {
  *tiny = s1 > 0.0f && s1 < 0x1p-64f;
  return (*tiny ? s1 * 0x1p+64f : s1) * (s2 * c_dec);
}

template <bool BF16OUT, int EPL, int LPG>
__global__ __launch_bounds__(kThreads) void fp4quant_decode_kernel(
    const uint32_t* __restrict__ packed, const float* __restrict__ s_rms,
    const float* __restrict__ s_abs, int64_t n_lane, float c_dec, void* __restrict__ y, int64_t blk0) {
  constexpr int U = (EPL == 8) ? 2 : 1;
  constexpr int OCT = EPL / 8;
  const int lane = threadIdx.x & 63;
  const int64_t base = ((int64_t)blockIdx.x + blk0) * (kThreads * U) + threadIdx.x;
  uint32_t w[U][OCT];
  float f[U];
  bool tiny[U];
  // 2 * e2m1 values are integers in [-12, 12]; every partial sum of the
  // transform is an integer below 2^14, so fp32 butterflies on them are exact.
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t t = base + (int64_t)k * kThreads;
    const bool ok = t < n_lane;
#pragma unroll
    for (int o = 0; o < OCT; ++o) w[k][o] = ok ? packed[t * OCT + o] : 0u;
    f[k] = ok ? group_factor(s_rms[t / LPG], s_abs[t / LPG], c_dec, &tiny[k]) : 0.0f;
    tiny[k] = ok && tiny[k];
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
    const bool any_tiny = __builtin_amdgcn_ballot_w64(tiny[k]) != 0;
    if (t >= n_lane) continue;
#pragma unroll
    for (int o = 0; o < OCT; ++o) {
      float out[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) out[j] = c[8 * o + j] * f[k];
      if (any_tiny) {
#pragma unroll
        for (int j = 0; j < 8; ++j) out[j] = __builtin_amdgcn_ldexpf(out[j], tiny[k] ? -kTinyShift : 0);
      }
      store8<BF16OUT>(y, t * OCT + o, out);
    }
  }
}

// ------------------------------------------- row layout (G <= 256)
// A wavefront converts a tile of 512 consecutive octets (4096 elements).
// Global memory sees only whole-tile streams: every load and store
// instruction moves 64 consecutive 16-byte chunks (1 KiB).  The tile passes
// through the wave's own LDS, where it is regrouped: the G / 8 octets of a
// group go to LPG lanes (1, 2 or 4) that lie D = 64 / LPG lanes apart (the
// same lane of different 32- or 16-lane rows), S = min(G / 8, 8) octets per
// lane, and a lane handles U groups in turn (512 octets = U * 64 * S).
// Every butterfly stage then runs inside a lane: stages over the element
// bits of an octet and over the octet bits a lane holds are register
// butterflies; the stage over a row bit of the octet index first exchanges
// that bit with a slot bit through the gfx950 row-swap instructions
// (v_permlane16_swap: rows 0<->1 and 2<->3 of 16 lanes; v_permlane32_swap:
// the two 32-lane halves), after which the two octets that differ in the row
// bit sit in one lane.  No select and no cross-lane shuffle through LDS.
//
// Octet index o within a group (bits: LPG row bits r, then slot bits s):
//   layout L0 (the encoder's input, the decoder's output): o = r + LPG s;
//   layout P  (the encoder's codes, the decoder's input): row bit k of o is
//     slot bit C_k of the register and slot bit C_k of o is row bit k of the
//     lane.  In P a lane holds runs of 4 (G = 16: 2) consecutive octets,
//     whose codes are one 16-byte (8-byte) LDS word.
// LDS chunks (16 bytes) are XOR-swizzled, chunk c at c ^ ((c >> sh) & 7),
// so that the 8 lanes served together by a 16-byte LDS access hit 8
// different bank quads both for the linear (global-side) and the grouped
// (compute-side) access.
template <int G> struct RowCfg;
template <> struct RowCfg<16> { static constexpr int LPG = 1, S = 2, C0 = 0, C1 = 0; };
template <> struct RowCfg<32> { static constexpr int LPG = 1, S = 4, C0 = 0, C1 = 0; };
template <> struct RowCfg<64> { static constexpr int LPG = 1, S = 8, C0 = 0, C1 = 0; };
template <> struct RowCfg<128> { static constexpr int LPG = 2, S = 8, C0 = 1, C1 = 0; };
template <> struct RowCfg<256> { static constexpr int LPG = 4, S = 8, C0 = 0, C1 = 1; };

constexpr int kTileOct = 512;                 // octets per wave tile
constexpr int kRowWaves = 4;                  // waves per workgroup

// Octet (within the group) of row r, slot s in layout P.
template <class C>
__host__ __device__ constexpr int oct_p(int r, int s) {
  int rr = 0, ss = s;
  if (C::LPG >= 2) {
    rr |= (s >> C::C0) & 1;
    ss = (ss & ~(1 << C::C0)) | ((r & 1) << C::C0);
  }
  if (C::LPG >= 4) {
    rr |= ((s >> C::C1) & 1) << 1;
    ss = (ss & ~(1 << C::C1)) | (((r >> 1) & 1) << C::C1);
  }
  return rr + C::LPG * ss;
}
template <class C> constexpr int kRun = C::S < 4 ? C::S : 4;     // octets per run in P
// The slot holding the octet whose row-0 index in layout P is o0.
template <class C>
__host__ __device__ constexpr int slot_of_p(int o0) {
  for (int s = 0; s < C::S; ++s)
    if (oct_p<C>(0, s) == o0) return s;
  return -1;
}
// The slot that starts the j-th run in layout P.
template <class C>
__host__ __device__ constexpr int run_start_slot(int j) {
  for (int s = 0; s < C::S; ++s)
    if (oct_p<C>(0, s) % kRun<C> == 0 && j-- == 0) return s;
  return -1;
}
constexpr int ilog2c(int v) { return v <= 1 ? 0 : 1 + ilog2c(v / 2); }
// Swizzled position of chunk c when a group spans `span` chunks.
template <int SPAN>
__device__ __forceinline__ int swz_chunk(int c) {
  constexpr int sh = ilog2c(SPAN) > 3 ? ilog2c(SPAN) : 3;
  return c ^ ((c >> sh) & 7);
}

__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(p[0]);
  b = __uint_as_float(p[1]);
}
__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(p[0]);
  b = __uint_as_float(p[1]);
}
// Exchange of row bit k with slot bit C_k for every slot pair, then the
// butterfly over the pair (now the stage over row bit k of the octet index).
template <class C, int K, int S>
__device__ __forceinline__ void row_stage(float (&v)[S][8]) {
  constexpr int h = 1 << (K == 0 ? C::C0 : C::C1);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (s & h) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = v[s][j], b = v[s | h][j];
      if constexpr (C::LPG == 4 && K == 0) swap16(a, b);
      else swap32(a, b);
      v[s][j] = a + b;
      v[s | h][j] = a - b;
    }
  }
}
// Register butterflies over the 8 elements of each octet and over the slot bits.
template <int S>
__device__ __forceinline__ void wht_in_lane(float (&v)[S][8]) {
#pragma unroll
  for (int s = 0; s < S; ++s) wht_local<8>(v[s]);
#pragma unroll
  for (int h = 1; h < S; h <<= 1) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (s & h) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = v[s][j], b = v[s | h][j];
        v[s][j] = a + b;
        v[s | h][j] = a - b;
      }
    }
  }
}
// Sum / max over the LPG lanes of a group (a row swap of a value with itself
// gives every lane its partner row's value in one of the two results).
template <int LPG>
__device__ __forceinline__ float rows_sum(float x) {
  if constexpr (LPG == 4) { float a = x, b = x; swap16(a, b); x = a + b; }
  if constexpr (LPG >= 2) { float a = x, b = x; swap32(a, b); x = a + b; }
  return x;
}
template <int LPG>
__device__ __forceinline__ float rows_max(float x) {
  if constexpr (LPG == 4) { float a = x, b = x; swap16(a, b); x = fmaxf(a, b); }
  if constexpr (LPG >= 2) { float a = x, b = x; swap32(a, b); x = fmaxf(a, b); }
  return x;
}
// Sum of squares of the lane's elements (short fma chains, then a tree).
template <int S>
__device__ __forceinline__ float lane_sumsq(const float (&v)[S][8]) {
  float t[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    float a = v[s][0] * v[s][0], b = v[s][4] * v[s][4];
#pragma unroll
    for (int j = 1; j < 4; ++j) {
      a = __builtin_fmaf(v[s][j], v[s][j], a);
      b = __builtin_fmaf(v[s][4 + j], v[s][4 + j], b);
    }
    t[s] = a + b;
  }
#pragma unroll
  for (int h = 1; h < S; h <<= 1)
#pragma unroll
    for (int s = 0; s < S; s += 2 * h) t[s] = t[s] + t[s + h];
  return t[0];
}
template <int S>
__device__ __forceinline__ float lane_absmax(const float (&v)[S][8]) {
  float m = 0.0f;
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int j = 0; j < 8; j += 2) m = fmaxf(m, fmaxf(fabsf(v[s][j]), fabsf(v[s][j + 1])));
  return m;
}

// Orders the wave's LDS accesses: writes by some lanes before reads of the
// same bytes by others.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Encoder arithmetic as above (codes 6 w / max|w|, s2 = max|w| / (6 sqrt(ss)),
// s1 = sqrt(ss / G)), with the approximate reciprocal and square-root
// instructions: this path is checked against the oracle within a tolerance,
// and their error (about 1 ulp each) stays far inside it.  A group whose sum
// of squares leaves [2^-100, 2^126) (tiny, huge or zero groups) is first
// scaled by a power of two that brings its largest element to [1, 2): the
// codes and s2 do not change under such scaling, s1 is scaled back exactly.
template <bool BF16, int G, bool SR, bool WIDE>
__global__ __launch_bounds__(64 * kRowWaves) void fq_encode_rows_kernel(
    const void* __restrict__ x, int64_t n_oct, uint32_t* __restrict__ packed,
    float* __restrict__ s_rms, float* __restrict__ s_abs, uint64_t seed, uint64_t step, int64_t blk0) {
  using C = RowCfg<G>;
  constexpr int LPG = C::LPG, S = C::S, D = 64 / LPG, NO = G / 8;
  constexpr int U = kTileOct / (D * NO);             // groups a lane handles in turn
  constexpr int NW = BF16 ? 1 : 2;                   // 16-byte chunks per octet
  constexpr int TCH = kTileOct * NW;                 // input chunks per tile
  __shared__ u32x4 tile_in[kRowWaves][TCH];
  __shared__ u32x4 tile_codes[kRowWaves][kTileOct / 4];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gw = lane % D, r = lane / D;
  const int64_t wave = ((int64_t)blockIdx.x + blk0) * kRowWaves + wv;
  const int64_t t0 = wave * kTileOct;                // first octet of the tile
  u32x4* lin = tile_in[wv];
  u32x4* lcodes = tile_codes[wv];

  // 1. the tile, linear 1 KiB streams -> LDS (chunks past the end read chunk 0)
  {
    const int64_t nch = n_oct * NW, c0 = t0 * NW;
    u32x4 a[TCH / 64];
#pragma unroll
    for (int k = 0; k < TCH / 64; ++k) {
      const int64_t c = c0 + 64 * k + lane;
      a[k] = ld_u32x4(static_cast<const uint8_t*>(x) + (c < nch ? c : 0) * 16);
    }
#pragma unroll
    for (int k = 0; k < TCH / 64; ++k) lin[swz_chunk<NO * NW>(64 * k + lane)] = a[k];
  }
  wave_lds_sync();

#pragma unroll 1
  for (int u = 0; u < U; ++u) {
    const int gl = u * D + gw;                       // group within the tile
    const int64_t g = t0 / NO + gl;
    // 2. the group's octets, layout L0
    float v[S][8];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int c = (gl * NO + r + LPG * s) * NW;
      const u32x4 p = lin[swz_chunk<NO * NW>(c)];
      if constexpr (BF16) {
        v[s][0] = bf16_lo(p.x); v[s][1] = bf16_hi(p.x); v[s][2] = bf16_lo(p.y); v[s][3] = bf16_hi(p.y);
        v[s][4] = bf16_lo(p.z); v[s][5] = bf16_hi(p.z); v[s][6] = bf16_lo(p.w); v[s][7] = bf16_hi(p.w);
      } else {
        const u32x4 q = lin[swz_chunk<NO * NW>(c + 1)];
        v[s][0] = __uint_as_float(p.x); v[s][1] = __uint_as_float(p.y);
        v[s][2] = __uint_as_float(p.z); v[s][3] = __uint_as_float(p.w);
        v[s][4] = __uint_as_float(q.x); v[s][5] = __uint_as_float(q.y);
        v[s][6] = __uint_as_float(q.z); v[s][7] = __uint_as_float(q.w);
      }
    }
    // 3. scales and codes
    float ss = rows_sum<LPG>(lane_sumsq<S>(v));
    int e = 0;
    const bool odd = !(ss >= 0x1p-100f && ss < 0x1p+126f);
    if (__builtin_amdgcn_ballot_w64(odd)) {          // rare: some group of the wave
      const float mxx = rows_max<LPG>(lane_absmax<S>(v));
      e = (odd && mxx > 0.0f) ? __builtin_amdgcn_frexp_expf(mxx) - 1 : 0;
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[s][j] = __builtin_amdgcn_ldexpf(v[s][j], -e);
      ss = rows_sum<LPG>(lane_sumsq<S>(v));
    }
    wht_in_lane<S>(v);
    if constexpr (LPG >= 2) row_stage<C, 0>(v);
    if constexpr (LPG >= 4) row_stage<C, 1>(v);
    const float mx = rows_max<LPG>(lane_absmax<S>(v));
    const bool zero = !(mx > 0.0f) || !(ss > 0.0f);
    const float rq = zero ? 0.0f : 6.0f * __builtin_amdgcn_rcpf(mx);
    const uint32_t keep = zero ? 0u : ~0u;             // a zero group's codes are 0
    uint32_t w[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      float q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = v[s][j] * rq;
      // slot s holds octet oct_p(r, s) of the group (layout P)
      if constexpr (SR) w[s] = sr8_octet<WIDE>(q, g * NO + oct_p<C>(r, s), seed, step) & keep;
      else w[s] = rtn8_unit(q) & keep;
    }
    // codes -> LDS in runs (layout P); word index = gl * NO + octet
#pragma unroll
    for (int jr = 0; jr < S / kRun<C>; ++jr) {
      constexpr int RL = kRun<C>;
      const int s0 = run_start_slot<C>(jr);
      const int o0 = oct_p<C>(0, s0);
      const int wi = gl * NO + oct_p<C>(r, s0);
      uint8_t* dst = reinterpret_cast<uint8_t*>(lcodes + swz_chunk<1>(wi >> 2)) + 4 * (wi & 3);
      if constexpr (RL == 4) {
        *reinterpret_cast<u32x4*>(dst) = u32x4{w[slot_of_p<C>(o0)], w[slot_of_p<C>(o0 + 1)],
                                               w[slot_of_p<C>(o0 + 2)], w[slot_of_p<C>(o0 + 3)]};
      } else {
        *reinterpret_cast<u32x2*>(dst) = u32x2{w[slot_of_p<C>(o0)], w[slot_of_p<C>(o0 + 1)]};
      }
    }
    if (r == 0 && g * NO < n_oct) {
      const float s1 = __builtin_amdgcn_sqrtf(ss * (1.0f / (float)G));
      const float s2 = (mx * __builtin_amdgcn_rsqf(ss)) * (1.0f / 6.0f);
      s_rms[g] = zero ? 0.0f : __builtin_amdgcn_ldexpf(s1, e);
      s_abs[g] = zero ? 0.0f : s2;
    }
  }
  wave_lds_sync();
  // 4. codes, linear 1 KiB streams (a chunk the end cuts in two: its 2 valid words)
#pragma unroll
  for (int k = 0; k < kTileOct / 4 / 64; ++k) {
    const int c = 64 * k + lane;
    const int64_t w0 = t0 + 4 * c;
    const u32x4 q = lcodes[swz_chunk<1>(c)];
    if (w0 + 4 <= n_oct) st_u32x4(packed + w0, q);
    else if (w0 < n_oct) __builtin_nontemporal_store(u32x2{q.x, q.y}, reinterpret_cast<u32x2*>(packed + w0));
  }
}

// Receiver: codes in layout P, output in layout L0.  2 e2m1 values are
// integers in [-12, 12] and every partial sum of the transform an integer
// below 2^13, so the fp32 butterflies are exact; one multiply by
// s1 s2 / (2 sqrt(G)) per element follows.
template <bool BF16OUT, int G>
__global__ __launch_bounds__(64 * kRowWaves) void fq_decode_rows_kernel(
    const uint32_t* __restrict__ packed, const float* __restrict__ s_rms,
    const float* __restrict__ s_abs, int64_t n_oct, float c_dec, void* __restrict__ y, int64_t blk0) {
  using C = RowCfg<G>;
  constexpr int LPG = C::LPG, S = C::S, D = 64 / LPG, NO = G / 8;
  constexpr int U = kTileOct / (D * NO);
  constexpr int NW = BF16OUT ? 1 : 2;                // 16-byte output chunks per octet
  constexpr int TCH = kTileOct * NW;
  __shared__ u32x4 tile_out[kRowWaves][TCH];
  __shared__ u32x4 tile_codes[kRowWaves][kTileOct / 4];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gw = lane % D, r = lane / D;
  const int64_t wave = ((int64_t)blockIdx.x + blk0) * kRowWaves + wv;
  const int64_t t0 = wave * kTileOct;
  u32x4* lout = tile_out[wv];
  u32x4* lcodes = tile_codes[wv];

  // 1. codes, linear 1 KiB streams -> LDS
  {
    u32x4 a[kTileOct / 4 / 64];
#pragma unroll
    for (int k = 0; k < kTileOct / 4 / 64; ++k) {
      const int64_t w0 = t0 + 4 * (64 * k + lane);
      if (w0 + 4 <= n_oct) {
        a[k] = *reinterpret_cast<const u32x4*>(packed + w0);
      } else {
        const u32x2 h = w0 < n_oct ? *reinterpret_cast<const u32x2*>(packed + w0) : u32x2{0u, 0u};
        a[k] = u32x4{h.x, h.y, 0u, 0u};
      }
    }
#pragma unroll
    for (int k = 0; k < kTileOct / 4 / 64; ++k) lcodes[swz_chunk<1>(64 * k + lane)] = a[k];
  }
  float f[U];
  bool tiny[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t g = t0 / NO + u * D + gw;
    const int64_t gc = g * NO < n_oct ? g : 0;       // past the end: group 0 (not stored)
    f[u] = group_factor(s_rms[gc], s_abs[gc], c_dec, &tiny[u]);
  }
  wave_lds_sync();

#pragma unroll 1
  for (int u = 0; u < U; ++u) {
    const int gl = u * D + gw;
    // 2. the group's codes, layout P
    uint32_t w[S];
#pragma unroll
    for (int jr = 0; jr < S / kRun<C>; ++jr) {
      constexpr int RL = kRun<C>;
      const int s0 = run_start_slot<C>(jr);
      const int o0 = oct_p<C>(0, s0);
      const int wi = gl * NO + oct_p<C>(r, s0);
      const uint8_t* src = reinterpret_cast<const uint8_t*>(lcodes + swz_chunk<1>(wi >> 2)) + 4 * (wi & 3);
      if constexpr (RL == 4) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(src);
        w[slot_of_p<C>(o0)] = q.x;
        w[slot_of_p<C>(o0 + 1)] = q.y;
        w[slot_of_p<C>(o0 + 2)] = q.z;
        w[slot_of_p<C>(o0 + 3)] = q.w;
      } else {
        const u32x2 q = *reinterpret_cast<const u32x2*>(src);
        w[slot_of_p<C>(o0)] = q.x;
        w[slot_of_p<C>(o0 + 1)] = q.y;
      }
    }
    // 3. transform and scale
    float c[S][8];
#pragma unroll
    for (int s = 0; s < S; ++s) e2m1x8_to_f32(w[s], 2.0f, c[s]);
    wht_in_lane<S>(c);
    if constexpr (LPG >= 2) row_stage<C, 0>(c);
    if constexpr (LPG >= 4) row_stage<C, 1>(c);
    // outputs -> LDS, layout L0
    const bool any_tiny = __builtin_amdgcn_ballot_w64(tiny[u]) != 0;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int ch = (gl * NO + r + LPG * s) * NW;
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = c[s][j] * f[u];
      if (any_tiny) {
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = __builtin_amdgcn_ldexpf(o[j], tiny[u] ? -kTinyShift : 0);
      }
      if constexpr (BF16OUT) {
        lout[swz_chunk<NO * NW>(ch)] = u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                             pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
      } else {
        lout[swz_chunk<NO * NW>(ch)] = u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]),
                                             __float_as_uint(o[2]), __float_as_uint(o[3])};
        lout[swz_chunk<NO * NW>(ch + 1)] = u32x4{__float_as_uint(o[4]), __float_as_uint(o[5]),
                                                 __float_as_uint(o[6]), __float_as_uint(o[7])};
      }
    }
  }
  wave_lds_sync();
  // 4. outputs, linear 1 KiB streams
  const int64_t nch = n_oct * NW, c0 = t0 * NW;
#pragma unroll
  for (int k = 0; k < TCH / 64; ++k) {
    const int c = 64 * k + lane;
    if (c0 + c < nch) st_u32x4(static_cast<uint8_t*>(y) + (c0 + c) * 16, lout[swz_chunk<NO * NW>(c)]);
  }
}

template <bool BF16, int G, bool SR, bool WIDE>
void launch_encode_rows(const void* x, int64_t n, uint32_t* pk, float* s1, float* s2,
                        uint64_t seed, uint64_t step, hipStream_t st) {
  const int64_t n_oct = n / 8;
  const int64_t waves = (n_oct + kTileOct - 1) / kTileOct;
  launch_1d(fq_encode_rows_kernel<BF16, G, SR, WIDE>, (waves + kRowWaves - 1) / kRowWaves,
            64 * kRowWaves, st, x, n_oct, pk, s1, s2, seed, step);
}
template <bool BF16OUT, int G>
void launch_decode_rows(const uint32_t* pk, const float* s1, const float* s2, int64_t n, void* y,
                        hipStream_t st) {
  const int64_t n_oct = n / 8;
  const int64_t waves = (n_oct + kTileOct - 1) / kTileOct;
  const float c_dec = (float)(0.5 / __builtin_sqrt((double)G));
  launch_1d(fq_decode_rows_kernel<BF16OUT, G>, (waves + kRowWaves - 1) / kRowWaves, 64 * kRowWaves,
            st, pk, s1, s2, n_oct, c_dec, y);
}

template <bool BF16, bool SR, bool WIDE>
void launch_encode_t(int G, const void* x, int64_t n, uint32_t* pk, float* s1, float* s2,
                     uint64_t seed, uint64_t step, hipStream_t st) {
  const float inv_g = 1.0f / (float)G;
  const float c_s2 = (float)(1.0 / (6.0 * __builtin_sqrt((double)G)));
#define FP4MI_ENC(EPL, LPG)                                                                   \
  {                                                                                           \
    int64_t nl = n / EPL;                                                                     \
    launch_1d(fp4quant_encode_kernel<BF16, EPL, LPG, SR, WIDE>, blocks_for(nl, EPL == 8 ? 2 : 1), \
              kThreads, st, x, nl, inv_g, c_s2, pk, s1, s2, seed, step);                      \
  }
  switch (G) {
    case 16: launch_encode_rows<BF16, 16, SR, WIDE>(x, n, pk, s1, s2, seed, step, st); break;
    case 32: launch_encode_rows<BF16, 32, SR, WIDE>(x, n, pk, s1, s2, seed, step, st); break;
    case 64: launch_encode_rows<BF16, 64, SR, WIDE>(x, n, pk, s1, s2, seed, step, st); break;
    case 128: launch_encode_rows<BF16, 128, SR, WIDE>(x, n, pk, s1, s2, seed, step, st); break;
    case 256: launch_encode_rows<BF16, 256, SR, WIDE>(x, n, pk, s1, s2, seed, step, st); break;
    case 512: FP4MI_ENC(8, 64); break;
    case 1024: FP4MI_ENC(16, 64); break;
  }
#undef FP4MI_ENC
}

// SR counters 2 i + 1 of octet i stay below 2^32 when 2 n_oct <= 2^32: their
// second word is then 0 (the narrow form of the draws).
template <bool BF16>
void launch_encode(int G, const void* x, int64_t n, uint32_t* pk, float* s1, float* s2, bool sr,
                   uint64_t seed, uint64_t step, hipStream_t st) {
  if (!sr) launch_encode_t<BF16, false, false>(G, x, n, pk, s1, s2, seed, step, st);
  else if (2 * (n / 8) <= (int64_t(1) << 32))
    launch_encode_t<BF16, true, false>(G, x, n, pk, s1, s2, seed, step, st);
  else launch_encode_t<BF16, true, true>(G, x, n, pk, s1, s2, seed, step, st);
}

template <bool BF16OUT>
void launch_decode(int G, const uint32_t* pk, const float* s1, const float* s2, int64_t n, void* y,
                   hipStream_t st) {
  const float c_dec = (float)(0.5 / __builtin_sqrt((double)G));
#define FP4MI_DEC(EPL, LPG)                                                                   \
  {                                                                                           \
    int64_t nl = n / EPL;                                                                     \
    launch_1d(fp4quant_decode_kernel<BF16OUT, EPL, LPG>, blocks_for(nl, EPL == 8 ? 2 : 1),     \
              kThreads, st, pk, s1, s2, nl, c_dec, y);                                        \
  }
  switch (G) {
    case 16: launch_decode_rows<BF16OUT, 16>(pk, s1, s2, n, y, st); break;
    case 32: launch_decode_rows<BF16OUT, 32>(pk, s1, s2, n, y, st); break;
    case 64: launch_decode_rows<BF16OUT, 64>(pk, s1, s2, n, y, st); break;
    case 128: launch_decode_rows<BF16OUT, 128>(pk, s1, s2, n, y, st); break;
    case 256: launch_decode_rows<BF16OUT, 256>(pk, s1, s2, n, y, st); break;
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
  return fp4quant_encode_ex(x, dtype, rows, cols, group, FP4_ROUND_RTN, 0, 0, packed, s_rms, s_abs,
                            stream);
}

extern "C" int fp4quant_encode_ex(const void* x, int dtype, int64_t rows, int64_t cols,
                                  int32_t group, int rounding, uint64_t seed, uint64_t step,
                                  uint8_t* packed, float* s_rms, float* s_abs, void* stream) {
  int es = dtype_size(dtype);
  if (!es) return FP4_EDTYPE;
  if (!valid_group(group)) return FP4_EINVAL;
  if (rounding != FP4_ROUND_RTN && rounding != FP4_ROUND_SR) return FP4_EINVAL;
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
  clear_stale_error();
  hipStream_t st = as_stream(stream);
  uint32_t* pk = reinterpret_cast<uint32_t*>(packed);
  const bool sr = rounding == FP4_ROUND_SR;
  if (dtype == FP4_DTYPE_BF16) launch_encode<true>(group, x, n, pk, s_rms, s_abs, sr, seed, step, st);
  else launch_encode<false>(group, x, n, pk, s_rms, s_abs, sr, seed, step, st);
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
  clear_stale_error();
  hipStream_t st = as_stream(stream);
  const uint32_t* pk = reinterpret_cast<const uint32_t*>(packed);
  if (out_dtype == FP4_DTYPE_BF16) launch_decode<true>(group, pk, s_rms, s_abs, n, y, st);
  else launch_decode<false>(group, pk, s_rms, s_abs, n, y, st);
  return launch_status();
}
