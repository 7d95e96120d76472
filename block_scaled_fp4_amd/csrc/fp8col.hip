// Fused MXFP4-row -> FP8-E4M3-column conversion over ragged expert shards
// (the MoE report "Practical FP4 Training for Large-Scale MoE Models on Hopper
// GPUs", section "核心技术贡献": item 1 the direct FP4->FP8 exponent remap with
// 4-to-1 scale alignment, item 2 the fused FP4RowToFP8Col kernel, item 3
// precomputed ragged shard offsets).
//
// Tiling.  A workgroup owns 64 consecutive tokens of the concatenated token
// axis, which may hold pieces ("segments") of several experts, and a run of
// 128-channel FP8 blocks.  Per FP8 block it
//   1. loads the 64 x 64 code bytes (a thread holds one 32-code MXFP4
//      sub-block of one token; a wave reads 16 tokens x 64 contiguous bytes)
//      and each token's four UE8M0 bytes as one dword;
//   2. takes S_tgt = max of the four bytes, d = S_tgt - S_sub, and remaps the
//      codes to E4M3 bytes through an 8-entry byte table per shift d
//      (v_perm_b32 does 4 lookups at once); the tables come from the
//      exponent-field mapping E8 = E4 - 1 + 7 - d, built once per workgroup;
//   3. transposes 4 x 4 byte blocks across the 4 lanes that hold 4
//      consecutive tokens (two DPP quad permutes + v_perm_b32), giving
//      dwords of 4 tokens of one channel;
//   4. stages them in LDS as [channel][token] rows of 16 dwords plus one pad
//      dword, the token-dword index XOR-swizzled by the sub-block so the
//      writes of a wave spread over the banks;
//   5. writes every output row with aligned dword stores: each output dword
//      is cut out of two LDS dwords with v_alignbyte_b32, so the per-row
//      misalignment of the ragged [H, n_e] matrices costs nothing; only the
//      partial dwords at segment edges fall back to byte stores;
//   6. writes the fp32 block scales 2^(S_tgt - 127).
// Segment bounds are checked against [0, T] per expert, so a malformed
// offsets array cannot cause out-of-bounds writes.
#include "device_common.hpp"
#include "host_common.hpp"

namespace fp4mi {
namespace {

constexpr int kTok = 64;         // tokens per tile
constexpr int kRowDw = 17;       // LDS dwords per channel row: 16 token dwords + 1 pad
constexpr int kMaxShift = 15;    // shifts >= 13 already map every value to 0
constexpr int kMaxSeg = 64;      // a 64-token tile holds at most 64 non-empty segments

// E4M3 magnitude byte of e2m1 magnitude m3 scaled by 2^-d, by exponent-field
// remapping.  Write the E2M1 magnitude as (2 + M) * 2^(E - 2) with E its
// exponent field and M its mantissa bit (0.5 is E = 1, M = 0 in this form:
// 2 * 2^-2).  The E4M3 exponent field is then ef = E - 1 + 7 - d and, when
// ef >= 1, the mantissa bit moves to the top of the 3-bit field.  When
// ef <= 0 the result is an E4M3 subnormal: in units of 2^-9 it is
// (2 + M) * 2^(ef + 1), rounded to nearest even when that is fractional.
__device__ uint32_t remap_e2m1_to_e4m3(uint32_t m3, int d) {
  if (m3 == 0) return 0;
  const int E = (m3 == 1) ? 1 : (int)(m3 >> 1);
  const int M = (m3 == 1) ? 0 : (int)(m3 & 1u);
  const int ef = (m3 == 1) ? (6 - d) : (E + 6 - d);
  if (ef >= 1) return ((uint32_t)ef << 3) | ((uint32_t)M << 2);
  const int num = 2 + M, p = ef + 1;
  if (p >= 0) return (uint32_t)(num << p);
  const int sh = -p;
  if (sh >= 8) return 0;
  int q = num >> sh, rem = num & ((1 << sh) - 1), half = 1 << (sh - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  return (uint32_t)q;
}

// 4 codes (low nibbles of the 4 bytes of `nib`) -> 4 E4M3 bytes.
__device__ __forceinline__ uint32_t lookup4(uint32_t nib, uint32_t tab_lo, uint32_t tab_hi) {
  const uint32_t mag = nib & 0x07070707u;
  const uint32_t sgn = (nib & 0x08080808u) << 4;
  return __builtin_amdgcn_perm(tab_hi, tab_lo, mag) | sgn;
}

__device__ __forceinline__ uint32_t dpp_xor1_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_xor2_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}

// Physical LDS dword of logical token-dword c (0..16) in channel row h.
__device__ __forceinline__ int lds_col(int h, int c) {
  return (c < 16) ? (c ^ (((h >> 5) & 3) << 2)) : c;
}

struct Segment {
  int64_t e_off;   // first token of the expert
  int64_t n;       // tokens of the expert
  int a, b;        // tile-local token range [a, b) of this segment
};

__global__ __launch_bounds__(kThreads) void fp8col_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ sb,
    const int64_t* __restrict__ off, int E, int64_t T, int64_t H, int blocks_per_wg,
    uint8_t* __restrict__ out, float* __restrict__ sc_out) {
  __shared__ uint32_t tile[128 * kRowDw];
  __shared__ uint32_t lut[(kMaxShift + 1) * 2];
  __shared__ Segment seg[kMaxSeg];
  __shared__ int32_t tgt[kTok];
  __shared__ int s_nseg;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int64_t t_end = (t0 + kTok < T) ? t0 + kTok : T;
  const int64_t HB = H / 128;

  // byte tables, one 8-byte table per shift d (bytes indexed by m3)
  if (tid < (kMaxShift + 1) * 2) {
    const int d = tid >> 1, half = tid & 1;
    uint32_t w = 0;
    for (int b = 0; b < 4; ++b) w |= remap_e2m1_to_e4m3((uint32_t)(4 * half + b), d) << (8 * b);
    lut[tid] = w;
  }

  // ---- segments of this tile (wave 0)
  if (tid < 64) {
    // expert of the first token: largest e < E with off[e] <= t0 (64-way search)
    int64_t lo = 0, hi = E;
    while (hi - lo > 1) {
      const int64_t step = (hi - lo + 63) / 64;
      const int64_t idx = lo + (int64_t)lane * step;
      const bool ok = idx < hi && off[idx] <= t0;
      const uint64_t m = __ballot(ok);
      const int top = 63 - __builtin_clzll(m | 1ull);
      lo = lo + (int64_t)top * step;
      hi = (lo + step < hi) ? lo + step : hi;
    }
    int nseg = 0;
    for (int64_t e0 = lo; e0 < E && nseg < kMaxSeg; e0 += 64) {
      const int64_t e = e0 + lane;
      const int64_t a_e = (e < E) ? off[e] : T;
      int64_t b_e = (e < E) ? off[e + 1] : T;
      if (b_e > T) b_e = T;
      const int64_t s0 = (a_e > t0) ? a_e : t0;
      const int64_t s1 = (b_e < t_end) ? b_e : t_end;
      const bool keep = e < E && a_e >= 0 && s0 < s1;
      const uint64_t m = __ballot(keep);
      const int pos = nseg + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (keep && pos < kMaxSeg) {
        Segment sg;
        sg.e_off = a_e;
        sg.n = b_e - a_e;
        sg.a = (int)(s0 - t0);
        sg.b = (int)(s1 - t0);
        seg[pos] = sg;
      }
      nseg += __builtin_popcountll(m);
      // stop once this window reaches the end of the tile
      const int64_t last_b = __shfl(b_e, 63);
      if (last_b >= t_end || e0 + 64 >= E) break;
    }
    if (lane == 0) s_nseg = nseg < kMaxSeg ? nseg : kMaxSeg;
  }

  // load-phase roles: token t = 4*(tid>>4) + (tid&3), sub-block (tid>>2)&3
  const int r = tid & 3, sub = (tid >> 2) & 3;
  const int tl = 4 * (tid >> 4) + r;
  const int64_t gl = t0 + tl;
  const bool lvalid = gl < T;
  const uint32_t sel1 = (r & 1) ? 0x03070105u : 0x06020400u;
  const uint32_t sel2 = (r & 2) ? 0x03020706u : 0x05040100u;
  const uint8_t* src_codes = packed + (lvalid ? gl : 0) * (H / 2) + sub * 16;
  const uint8_t* src_scales = sb + (lvalid ? gl : 0) * (H / 32);
  // this thread's LDS destinations: rows 32 sub + 4 g + r, swizzled token dword
  uint32_t* dst0 = tile + (32 * sub + r) * kRowDw + ((tid >> 4) ^ (sub << 2));
  // store-phase roles: 16 lanes per channel row, 16 rows per pass
  const int q = tid & 15, hr = tid >> 4;

  const int64_t b_begin = (int64_t)blockIdx.y * blocks_per_wg;
  const int64_t b_end = (b_begin + blocks_per_wg < HB) ? b_begin + blocks_per_wg : HB;

  // software pipeline: the codes and scales of block b are in registers
  // while block b-1 is being written out
  u32x4 w = {0u, 0u, 0u, 0u};
  uint32_t s4 = 0;
  if (lvalid && b_begin < b_end) {
    w = ld_u32x4(src_codes + b_begin * 64);
    s4 = *reinterpret_cast<const uint32_t*>(src_scales + b_begin * 4);
  }
  __syncthreads();            // LUT and segments ready (see above)
  const int nseg = s_nseg;

  for (int64_t b = b_begin; b < b_end; ++b) {
    // ---- 1-2: scale alignment and remap of block b
    const uint32_t s_tgt = max(max(s4 & 0xFFu, (s4 >> 8) & 0xFFu),
                               max((s4 >> 16) & 0xFFu, s4 >> 24));
    const uint32_t s_sub = (s4 >> (8 * sub)) & 0xFFu;
    const int d = min((int)(s_tgt - s_sub), kMaxShift);
    const uint32_t tlo = lut[2 * d], thi = lut[2 * d + 1];
    uint32_t D[8];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t ev = lookup4(ww[k], tlo, thi);          // channels 8k+0,2,4,6
      const uint32_t od = lookup4(ww[k] >> 4, tlo, thi);     // channels 8k+1,3,5,7
      D[2 * k] = __builtin_amdgcn_perm(od, ev, 0x05010400u);
      D[2 * k + 1] = __builtin_amdgcn_perm(od, ev, 0x07030602u);
    }
    // ---- 3-4: 4x4 byte transpose across the token quad, stage in LDS
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint32_t t1 = __builtin_amdgcn_perm(dpp_xor1_u(D[g]), D[g], sel1);
      const uint32_t t2 = __builtin_amdgcn_perm(dpp_xor2_u(t1), t1, sel2);
      dst0[4 * g * kRowDw] = t2;
    }
    if (sub == 0) tgt[tl] = (int32_t)s_tgt;
    __syncthreads();
    // prefetch block b+1 while block b is written out
    if (lvalid && b + 1 < b_end) {
      w = ld_u32x4(src_codes + (b + 1) * 64);
      s4 = *reinterpret_cast<const uint32_t*>(src_scales + (b + 1) * 4);
    }
    // ---- 5-6: aligned dword stores per segment and channel row
    for (int si = 0; si < nseg; ++si) {
      const Segment sg = seg[si];
      const int a = sg.a, bb = sg.b;
      // byte address of tile token 0 in channel row 128 b + hr of this expert
      int64_t rt = H * sg.e_off + (t0 - sg.e_off) + (128 * b + hr) * sg.n;
      const int64_t rstep = 16 * sg.n;
#pragma unroll
      for (int p = 0; p < 8; ++p, rt += rstep) {
        const int h = 16 * p + hr;
        const uint32_t* row = tile + h * kRowDw;
        const int colx = ((p >> 1) & 3) << 2;                 // swizzle of rows 32s..32s+31
        const int m = (int)(((uint32_t)rt + (uint32_t)a) & 3u);
        const int am = a - m;                                 // tile token of the first dword's byte 0
        const int base_c = am >> 2, sh = am & 3;              // floor / remainder (am >= -3)
        for (int item = q; item < 17; item += 16) {
          const int tt0 = am + 4 * item;
          if (tt0 >= bb) break;
          const int c = base_c + item;
          const int c0 = max(c, 0), c1 = c + 1;
          const uint32_t lo_dw = row[c0 < 16 ? (c0 ^ colx) : 16];
          const uint32_t hi_dw = row[c1 < 16 ? (c1 ^ colx) : 16];
          const uint32_t val = __builtin_amdgcn_alignbyte(hi_dw, lo_dw, (uint32_t)sh);
          const int blo = max(a - tt0, 0), bhi = min(bb - tt0, 4);
          uint8_t* A = out + rt + tt0;
          if (blo == 0 && bhi == 4) {
            *reinterpret_cast<uint32_t*>(A) = val;
          } else {
            for (int k = blo; k < bhi; ++k) A[k] = (uint8_t)(val >> (8 * k));
          }
        }
      }
      if (tid >= a && tid < bb)
        sc_out[HB * sg.e_off + b * sg.n + (t0 + tid - sg.e_off)] =
            __builtin_amdgcn_ldexpf(1.0f, tgt[tid] - 127);
    }
    __syncthreads();
  }
}

}  // namespace
}  // namespace fp4mi

using namespace fp4mi;

extern "C" int mxfp4_row_to_fp8_col(const uint8_t* packed, const uint8_t* scales_e8m0,
                                    const int64_t* token_offsets, int32_t num_experts,
                                    int64_t total_tokens, int64_t hidden, uint8_t* fp8_out,
                                    float* fp8_scales, void* stream) {
  if (num_experts < 1) return FP4_EINVAL;
  if (total_tokens < 0 || hidden <= 0 || hidden % 128) return FP4_ESHAPE;
  int64_t n;
  if (!checked_count(total_tokens, hidden, &n)) return FP4_ESHAPE;
  if (!token_offsets) return FP4_EINVAL;
  if (n == 0) return FP4_OK;
  if (!packed || !scales_e8m0 || !fp8_out || !fp8_scales) return FP4_EINVAL;
  if (!is_aligned(packed, 16) || !is_aligned(scales_e8m0, 4) || !is_aligned(token_offsets, 8) ||
      !is_aligned(fp8_out, 4) || !is_aligned(fp8_scales, 4))
    return FP4_EALIGN;
  const int64_t pb = n / 2, sbb = n / 32, ob = n, scb = (n / 128) * 4,
                offb = ((int64_t)num_experts + 1) * 8;
  const void* ins[3] = {packed, scales_e8m0, token_offsets};
  const int64_t inn[3] = {pb, sbb, offb};
  for (int k = 0; k < 3; ++k)
    if (overlaps(fp8_out, ob, ins[k], inn[k]) || overlaps(fp8_scales, scb, ins[k], inn[k]))
      return FP4_EOVERLAP;
  if (overlaps(fp8_out, ob, fp8_scales, scb)) return FP4_EOVERLAP;
  hipStream_t st = as_stream(stream);
  const int64_t tiles = (total_tokens + kTok - 1) / kTok;
  const int64_t HB = hidden / 128;
  const int bpw = (int)(HB < 8 ? HB : 8);
  const int64_t gy = (HB + bpw - 1) / bpw;
  if (tiles > 0x7FFFFFFF || gy > 65535) return FP4_ESHAPE;
  hipLaunchKernelGGL(fp8col_kernel, dim3((unsigned)tiles, (unsigned)gy), dim3(kThreads), 0, st,
                     packed, scales_e8m0, token_offsets, (int)num_experts, total_tokens, hidden,
                     bpw, fp8_out, fp8_scales);
  return launch_status();
}
