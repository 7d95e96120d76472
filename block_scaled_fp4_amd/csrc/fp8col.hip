// Fused MXFP4-row -> FP8-E4M3-column conversion over ragged expert shards
// (the MoE report "Practical FP4 Training for Large-Scale MoE Models on Hopper
// GPUs", section "核心技术贡献": item 1 the direct FP4->FP8 exponent remap with
// 4-to-1 scale alignment, item 2 the fused FP4RowToFP8Col kernel, item 3
// precomputed ragged shard offsets).
//
// Tiling.  A workgroup owns 64 consecutive tokens of the concatenated token
// axis (which may cover several small experts) and a run of 128-channel FP8
// blocks.  Per FP8 block it
//   1. reads 64 tokens x 64 bytes of codes (one 16-byte load per thread; a
//      thread holds one 32-element MXFP4 sub-block) and the 4 sub-scales;
//   2. takes S_tgt = max of the quad's 4 UE8M0 bytes (DPP) and remaps codes
//      to E4M3 bytes through an 8-entry byte table per shift d = S_tgt - S_sub
//      (v_perm_b32 as a 4-way table lookup), the table being built once per
//      workgroup from the exponent-field mapping E8 = E4 - 1 + 7 - d;
//   3. stages the [token][channel] tile in LDS with a row pitch of 132 bytes
//      (33 dwords, odd, so a column walk touches 64 distinct banks);
//   4. walks the tile by columns and writes each channel's token run into the
//      expert's [H, n_e] matrix, plus the fp32 block scale 2^(S_tgt-127).
// The expert of each token is found once per workgroup from the offsets.
// Tokens whose (offset, count) would address outside [0, T*H) are skipped, so
// a malformed offsets array cannot cause out-of-bounds writes.
#include "device_common.hpp"
#include "host_common.hpp"

namespace fp4mi {
namespace {

constexpr int kTok = 64;         // tokens per tile
constexpr int kPitch = 132;      // LDS bytes per token row of the tile
constexpr int kMaxShift = 15;    // shifts >= 13 already map every value to 0

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
  uint32_t mag = nib & 0x07070707u;
  uint32_t sgn = (nib & 0x08080808u) << 4;
  return __builtin_amdgcn_perm(tab_hi, tab_lo, mag) | sgn;
}

__global__ __launch_bounds__(kThreads) void fp8col_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ sb,
    const int64_t* __restrict__ off, int E, int64_t T, int64_t H, int blocks_per_wg,
    uint8_t* __restrict__ out, float* __restrict__ sc_out) {
  __shared__ uint32_t tile[kTok * kPitch / 4];
  __shared__ uint32_t lut[(kMaxShift + 1) * 2];
  __shared__ int64_t win[kTok];
  __shared__ int64_t tok_off[kTok];
  __shared__ int64_t tok_n[kTok];
  __shared__ int32_t tgt[kTok];
  __shared__ int64_t s_first[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int64_t HB = H / 128;

  // byte tables, one 8-byte table per shift d (bytes indexed by m3)
  if (tid < (kMaxShift + 1) * 2) {
    int d = tid >> 1, half = tid & 1;
    uint32_t w = 0;
    for (int b = 0; b < 4; ++b) w |= remap_e2m1_to_e4m3((uint32_t)(4 * half + b), d) << (8 * b);
    lut[tid] = w;
  }

  // expert of the tile's first token: largest e with off[e] <= t0 (64-way search)
  if (tid < 64) {
    int64_t lo = 0, hi = E;               // off[lo] <= t0 < off[E] = T
    while (hi - lo > 1) {
      int64_t step = (hi - lo + 63) / 64;
      int64_t idx = lo + (int64_t)lane * step;
      bool ok = idx < hi && off[idx] <= t0;
      uint64_t m = __ballot(ok);
      int top = 63 - __builtin_clzll(m | 1ull);
      lo = lo + (int64_t)top * step;
      hi = (lo + step < hi) ? lo + step : hi;
    }
    // window of the following offsets: win[k] = off[lo + 1 + k] (T beyond E)
    int64_t wi = lo + 1 + lane;
    win[lane] = (wi <= E) ? off[wi] : T;
    if (lane == 0) { s_first[0] = lo; s_first[1] = off[lo]; }
  }
  __syncthreads();

  // per-token expert: e = first + #(win entries <= g); beyond the window use
  // a binary search over the global offsets.
  if (tid < 64) {
    const int64_t g = t0 + lane;
    int64_t o = -1, n = 0;
    if (g < T) {
      int cnt = 0;
      for (int b = 64; b >= 1; b >>= 1)
        if (cnt + b <= 64 && win[cnt + b - 1] <= g) cnt += b;
      int64_t e = s_first[0] + cnt;
      if (cnt == 64) {                    // many (empty) experts inside the tile
        int64_t lo = e, hi = E;           // off[lo] <= g
        while (hi - lo > 1) {
          int64_t mid = (lo + hi) >> 1;
          if (off[mid] <= g) lo = mid; else hi = mid;
        }
        e = lo;
      }
      int64_t a = (cnt == 0) ? s_first[1] : off[e];
      int64_t b = (e + 1 <= E) ? off[e + 1] : T;
      if (b > T) b = T;
      if (a >= 0 && a <= g && g < b) { o = a; n = b - a; }
    }
    tok_off[lane] = o;
    tok_n[lane] = n;
  }
  __syncthreads();

  const int tl = tid >> 2, sub = tid & 3;        // load phase: token row, sub-block
  const int64_t gl = t0 + tl;
  const bool lvalid = gl < T;
  const int ot = tid & 63, og = tid >> 6;        // store phase: token, channel phase
  const int64_t o_off = tok_off[ot], o_n = tok_n[ot];
  const int64_t go = t0 + ot;
  const bool ovalid = o_off >= 0;

  const int64_t b_begin = (int64_t)blockIdx.y * blocks_per_wg;
  const int64_t b_end = (b_begin + blocks_per_wg < HB) ? b_begin + blocks_per_wg : HB;
  for (int64_t b = b_begin; b < b_end; ++b) {
    // ---- load + remap + stage
    int s_sub = 0;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (lvalid) {
      w = ld_u32x4(packed + gl * (H / 2) + b * 64 + sub * 16);
      s_sub = sb[gl * (H / 32) + b * 4 + sub];
    }
    int s_t = max(s_sub, lane_xor1_i(s_sub));
    s_t = max(s_t, lane_xor2_i(s_t));
    if (lvalid) {
      int d = min(s_t - s_sub, kMaxShift);
      uint32_t tlo = lut[2 * d], thi = lut[2 * d + 1];
      uint32_t* row = tile + (tl * kPitch + sub * 32) / 4;
      uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t ev = lookup4(ww[k], tlo, thi);          // elements 0,2,4,6
        uint32_t od = lookup4(ww[k] >> 4, tlo, thi);     // elements 1,3,5,7
        row[2 * k] = __builtin_amdgcn_perm(od, ev, 0x05010400u);
        row[2 * k + 1] = __builtin_amdgcn_perm(od, ev, 0x07030602u);
      }
      if (sub == 0) tgt[tl] = s_t;
    }
    __syncthreads();
    // ---- column walk: channel h of token ot -> out[H*off + (128b+h)*n + (g-off)]
    if (ovalid) {
      uint8_t* dst = out + H * o_off + (go - o_off);
      const uint8_t* src = reinterpret_cast<const uint8_t*>(tile) + ot * kPitch;
#pragma unroll 8
      for (int j = 0; j < 32; ++j) {
        int h = og + 4 * j;
        dst[(128 * b + h) * o_n] = src[h];
      }
      if (og == 0)
        sc_out[HB * o_off + b * o_n + (go - o_off)] =
            __builtin_amdgcn_ldexpf(1.0f, tgt[ot] - 127);
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
