// Fused MXFP4-row -> FP8-E4M3-column conversion over ragged expert shards
// (the MoE report "Practical FP4 Training for Large-Scale MoE Models on Hopper
// GPUs", section "核心技术贡献": item 1 the direct FP4->FP8 exponent remap with
// 4-to-1 scale alignment, item 2 the fused FP4RowToFP8Col kernel, item 3
// precomputed ragged shard offsets).
//
// Work decomposition.  The token space is cut into chunks of kChunk tokens;
// workgroup (chunk, b) converts FP8 block b (128 channels) of every expert
// piece in its chunk, and its four waves take the four 32-channel MXFP4
// sub-blocks.  Piece boundaries are snapped to multiples of 4 tokens of the
// expert, so neighbouring chunks agree on them.  A wave streams through its
// piece 252 new tokens at a time (lane L >= 1 holds 4 consecutive tokens;
// lane 0 re-reads the 4 before them) and writes its 32 output rows, which lie
// one after the other in memory, as a stream of aligned dwords:
//   1. per token: load the 16 code bytes and the four UE8M0 bytes (one
//      dword), S_tgt = max of the four, d = S_tgt - S_sub, remap the codes to
//      E4M3 bytes through an 8-entry byte table per shift d (v_perm_b32 does
//      4 lookups at once); the tables come from the exponent-field mapping
//      E8 = E4 - 1 + 7 - d, built once per workgroup;
//   2. transpose 4 x 4 byte blocks inside the lane (v_perm_b32), giving per
//      channel a dword of the lane's 4 tokens;
//   3. a row starting m = (address mod 4) bytes past a dword boundary is
//      written with aligned dwords cut (v_alignbyte_b32) from the lane's
//      dword and the one of the lane before it (a DPP wavefront shift); the
//      dword shared by the end of row h and the start of row h+1 is stitched
//      with row h+1's first 4 tokens by the piece that ends the expert.
// Loads go through buffer resources whose range check returns zero for
// tokens outside the piece, so no load sits in a branch, and the next tile's
// loads are issued before the current tile's stores.  Chunks are laid out so
// that neighbouring chunks (which share output lines at their seams) and the
// two blocks that share input lines run in one L2 domain.  Only experts of
// fewer than 4 tokens need byte stores.  Expert ranges are clamped to
// [0, T], so a malformed offsets array cannot cause out-of-bounds accesses.
#include "device_common.hpp"
#include "host_common.hpp"

namespace fp4mi {
namespace {

constexpr int kMaxShift = 15;    // shifts >= 13 already map every value to 0
// Buffer resource word 3 for raw (untyped, stride 0) buffer access on gfx9.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kTileNew = 252;    // new tokens per wave step (4 per lane, lanes 1..63)
constexpr int kChunk = 4 * kTileNew;   // positions of the padded token space per workgroup
// Each expert is followed by kPad positions of padding in the space that is
// cut into chunks: a piece costs about a tile of work beyond its tokens, so
// no chunk holds more than a few pieces.
constexpr int kPad = kTileNew;
constexpr int kXcds = 8;               // L2 domains the workgroups are spread over
// A load offset past every load window (windows stay below 2^30 bytes for
// H < 2^21): a token loaded at it reads as zero.
constexpr int kOutside = 0x7FFFFFF0;

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

struct TileIn {
  u32x4 w[4];        // code bytes of the lane's 4 tokens (one 32-channel sub-block)
  uint32_t s[4];     // their four UE8M0 block scales
};

// Loads the 4 tokens starting `first` tokens into the load window.
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                          int first, bool valid0, int cstride, int sstride,
                                          TileIn& x) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool ok = valid0 || (first + j >= 4);
    const int tok = first + j;
    x.w[j] = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? tok * cstride : kOutside, 0, 0);
    x.s[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? tok * sstride : kOutside, 0, 0);
  }
}

// Remaps the lane's 4 tokens of sub-block `sub` to E4M3 and transposes them:
// Y[c] holds channel c of the 4 tokens, token j in byte j.  tgt[j] is S_tgt.
__device__ __forceinline__ void convert_tile(const TileIn& x, int sub, const uint32_t* lut,
                                             uint32_t Y[32], uint32_t tgt[4]) {
  uint32_t X[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t s4 = x.s[j];
    const uint32_t s_tgt = max(max(s4 & 0xFFu, (s4 >> 8) & 0xFFu),
                               max((s4 >> 16) & 0xFFu, s4 >> 24));
    const uint32_t s_sub = (s4 >> (8 * sub)) & 0xFFu;
    const int d = min((int)(s_tgt - s_sub), kMaxShift);
    const uint32_t tlo = lut[2 * d], thi = lut[2 * d + 1];
    const uint32_t ww[4] = {x.w[j].x, x.w[j].y, x.w[j].z, x.w[j].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t ev = lookup4(ww[q], tlo, thi);         // channels 8q+0,2,4,6
      const uint32_t od = lookup4(ww[q] >> 4, tlo, thi);    // channels 8q+1,3,5,7
      X[j][2 * q] = __builtin_amdgcn_perm(od, ev, 0x05010400u);
      X[j][2 * q + 1] = __builtin_amdgcn_perm(od, ev, 0x07030602u);
    }
    tgt[j] = s_tgt;
  }
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const uint32_t a0 = X[0][g], a1 = X[1][g], a2 = X[2][g], a3 = X[3][g];
    const uint32_t l01 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);   // a0.b0 a1.b0 a0.b1 a1.b1
    const uint32_t h01 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);   // a0.b2 a1.b2 a0.b3 a1.b3
    const uint32_t l23 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
    const uint32_t h23 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
    Y[4 * g + 0] = __builtin_amdgcn_perm(l23, l01, 0x05040100u);
    Y[4 * g + 1] = __builtin_amdgcn_perm(l23, l01, 0x07060302u);
    Y[4 * g + 2] = __builtin_amdgcn_perm(h23, h01, 0x05040100u);
    Y[4 * g + 3] = __builtin_amdgcn_perm(h23, h01, 0x07060302u);
  }
}

__device__ __forceinline__ int64_t round_up4(int64_t v) { return (v + 3) & ~int64_t(3); }
__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

__global__ __launch_bounds__(kThreads) void fp8col_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ sb,
    const int64_t* __restrict__ off, int32_t E, int64_t T, int64_t H, int64_t nchunks,
    int64_t per_xcd, uint8_t* __restrict__ out, float* __restrict__ sc_out) {
  __shared__ uint32_t lut[(kMaxShift + 1) * 2];
  __shared__ int counts[2];
  const int tid = threadIdx.x;
  // the wave index is uniform across a wave; saying so keeps the buffer
  // resources built from it in scalar registers
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Workgroup -> (chunk, block).  Consecutive workgroups go to the L2 domains
  // in turn; domain x takes chunks [x per_xcd, (x + 1) per_xcd), block fastest.
  const int64_t HB = H / 128;
  const int64_t id = blockIdx.x;
  const int64_t slot = id / kXcds;
  const int64_t chunk = (id % kXcds) * per_xcd + slot / HB;
  const int64_t b = slot % HB;
  if (chunk >= nchunks) return;                         // uniform per workgroup
  const int64_t g0 = chunk * kChunk, g1 = g0 + kChunk;

  if (tid < (kMaxShift + 1) * 2) {
    const int d = tid >> 1, half = tid & 1;
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k) w |= remap_e2m1_to_e4m3((uint32_t)(4 * half + k), d) << (8 * k);
    lut[tid] = w;
  }
  if (tid < 2) counts[tid] = 0;
  __syncthreads();
  // Expert e starts at position off[e] + kPad e of the padded space.
  // Experts with a piece in this chunk: from the last one starting at or
  // before g0 up to the last one starting before g1 (offsets ascend).
  int c0 = 0, c1 = 0;
  for (int e = tid; e < E; e += kThreads) {
    const int64_t o = off[e] + (int64_t)kPad * e;
    c0 += o <= g0;
    c1 += o < g1;
  }
  if (c0) atomicAdd(&counts[0], c0);
  if (c1) atomicAdd(&counts[1], c1);
  __syncthreads();
  const int e_first = max(counts[0] - 1, 0), e_end = counts[1];

  const int h0 = 32 * wave;                             // first channel of the wave's run
  const int cs = (int)(H / 2), ss = (int)(H / 32);      // token strides of codes and scales
  for (int e = e_first; e < e_end; ++e) {               // uniform per workgroup
    const int64_t off_e = clamp64(off[e], 0, T);
    const int64_t end_e = clamp64(off[e + 1], off_e, T);
    const int n = (int)(end_e - off_e);                 // n < 2^26 (checked by the host)
    const int64_t pos = off_e + (int64_t)kPad * e;     // the expert's padded position
    const int a = (int)clamp64(round_up4(g0 - pos), 0, n);
    const int bb = (int)clamp64(round_up4(g1 - pos), 0, n);
    if (a >= bb) continue;
    const bool last = bb == n;
    const int len = bb - a;
    const int ntiles = (len + (last ? 3 : 0) + kTileNew - 1) / kTileNew;
    const int64_t R0 = H * off_e + (128 * b + h0) * (int64_t)n;   // the run of 32 rows
    float* const so = sc_out + HB * off_e + b * n;

    if (n < 4) {
      // Experts of 1..3 tokens: one piece; rows shorter than a dword, so each
      // output byte is computed and stored on its own.
      for (int i = lane; i < 32 * n; i += 64) {
        const int r = i / n, t = i - r * n;
        const int ch = 32 * wave + r;                   // channel within the block
        const int64_t tok = off_e + t;
        const uint32_t s4 = *reinterpret_cast<const uint32_t*>(sb + tok * ss + 4 * b);
        const uint32_t s_tgt = max(max(s4 & 0xFFu, (s4 >> 8) & 0xFFu),
                                   max((s4 >> 16) & 0xFFu, s4 >> 24));
        const uint32_t s_sub = (s4 >> (8 * wave)) & 0xFFu;
        const int d = min((int)(s_tgt - s_sub), kMaxShift);
        const uint32_t code = (packed[tok * cs + 64 * b + ch / 2] >> (4 * (ch & 1))) & 0xFu;
        const uint32_t v = lookup4(code, lut[2 * d], lut[2 * d + 1]) & 0xFFu;
        out[R0 + (int64_t)r * n + t] = (uint8_t)v;
        if (wave == 0 && r == 0) so[t] = __builtin_amdgcn_ldexpf(1.0f, (int)s_tgt - 127);
      }
      continue;
    }

    // Stores go through the run's window, which begins 8 bytes before the run
    // (R0 is a multiple of 32, so every dword offset is positive) and ends
    // with it; the buffer range check drops stores at kOutside.
    const __amdgpu_buffer_rsrc_t win = __builtin_amdgcn_make_buffer_rsrc(
        out + R0 - 8, (short)0, 32 * n + 8, kBufferWord3);
    const __amdgpu_buffer_rsrc_t wsc = __builtin_amdgcn_make_buffer_rsrc(
        so, (short)0, 4 * n, kBufferWord3);
    // Load windows: tokens a - 4 .. bb - 1 of the expert.
    const int64_t wtok = off_e + a - 4;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(packed) + wtok * cs + 64 * b + 16 * wave, (short)0, (len + 4) * cs,
        kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(sb) + wtok * ss + 4 * b, (short)0, (len + 4) * ss, kBufferWord3);
    const bool valid0 = a > 0;                          // the 4 tokens before the piece exist

    // Row heads (tokens 0..3 of row c in lane c) for the stitched row ends of
    // a piece that ends the expert: from tile 0 when the piece also starts
    // it, else loaded here.
    uint32_t hv = 0;
    if (last && a > 0) {
      TileIn hx;
      const uint8_t* c0p = packed + off_e * cs + 64 * b + 16 * wave;
      const uint8_t* s0p = sb + off_e * ss + 4 * b;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hx.w[j] = *reinterpret_cast<const u32x4*>(c0p + j * cs);
        hx.s[j] = *reinterpret_cast<const uint32_t*>(s0p + j * ss);
      }
      uint32_t Yh[32], th[4];
      convert_tile(hx, wave, lut, Yh, th);
#pragma unroll
      for (int c = 0; c < 32; ++c) hv = lane == c ? Yh[c] : hv;
    }

    // Tiles alternate between two load buffers.  Every tile issues the same
    // memory operations (the next tile's 8 loads, then 33 stores), so the
    // loads of tile k + 1 stay in flight while tile k is converted and
    // stored, and the wait for them leaves tile k's stores outstanding.
    auto process = [&](const TileIn& x, int k) {
      uint32_t Y[32], tgt[4];
      convert_tile(x, wave, lut, Y, tgt);
      const int tl = a - 4 + kTileNew * k + 4 * lane;   // the lane's first token
      if (last && a == 0 && k == 0) {
#pragma unroll
        for (int c = 0; c < 32; ++c)                    // lane 1 holds tokens 0..3
          hv = lane == c ? (uint32_t)__builtin_amdgcn_readlane(Y[c], 1) : hv;
      }

      // wave w stores the FP8 block scale of the lane's token w
      const uint32_t tg = wave == 0 ? tgt[0] : wave == 1 ? tgt[1] : wave == 2 ? tgt[2] : tgt[3];
      const bool sc_ok = lane > 0 && tl + wave < bb;
      __builtin_amdgcn_raw_buffer_store_b32(
          __float_as_uint(__builtin_amdgcn_ldexpf(1.0f, (int)tg - 127)), wsc,
          sc_ok ? 4 * (tl + wave) : kOutside, 0, 0);

      // Aligned dword stores along each row.  Lane L >= 1 writes the dword
      // starting at row token tf = tl - m; the piece owns tf in [0, bb - m),
      // or [0, n) when it ends the expert (tf < 0 is a row head, written
      // with the end of the row before).  A row end dword (tf + 4 > n) takes
      // the next row's first tokens; a run ends dword aligned, so row 31
      // never has one.
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        const int rowoff = c * n;                       // row c starts at run byte c n
        const int m = rowoff & 3;
        const uint32_t own = Y[c];
        // lane L - 1's dword (wavefront shift right by one lane)
        const uint32_t prev =
            (uint32_t)__builtin_amdgcn_update_dpp(0, (int)own, 0x138, 0xf, 0xf, false);
        const int tf = tl - m;
        uint32_t val = (m == 0) ? own : __builtin_amdgcn_alignbyte(own, prev, (uint32_t)(4 - m));
        const bool owned = lane > 0 && tf >= 0 && tf < (last ? n : bb - m);
        if (c < 31 && tf + 4 > n && owned) {
          const int hi = n - tf;                        // 1..3 bytes of this row
          const uint32_t mask = (1u << (8 * hi)) - 1u;
          val = (val & mask) | ((uint32_t)__builtin_amdgcn_readlane(hv, c + 1) << (8 * hi));
        }
        __builtin_amdgcn_raw_buffer_store_b32(val, win, owned ? 8 + rowoff + tf : kOutside, 0, 0);
      }
    };
    TileIn A, B;
    load_tile(rc, rs, 4 * lane, valid0, cs, ss, A);
    __builtin_amdgcn_s_waitcnt(0);                      // A is in: every entry to the loop alike
    for (int k = 0;; k += 2) {
      load_tile(rc, rs, kTileNew * (k + 1) + 4 * lane, valid0, cs, ss, B);
      process(A, k);
      if (k + 1 >= ntiles) break;
      load_tile(rc, rs, kTileNew * (k + 2) + 4 * lane, valid0, cs, ss, A);
      process(B, k + 1);
      if (k + 2 >= ntiles) break;
    }
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
  // 32-bit offsets in the load and store windows
  if (total_tokens >= (int64_t(1) << 26) || hidden >= (int64_t(1) << 21)) return FP4_ESHAPE;
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
  const int64_t HB = hidden / 128;
  const int64_t nchunks = (total_tokens + (int64_t)kPad * num_experts + kChunk - 1) / kChunk;
  const int64_t per_xcd = (nchunks + kXcds - 1) / kXcds;
  const int64_t grid = kXcds * per_xcd * HB;
  if (grid > 0x7FFFFFFF) return FP4_ESHAPE;
  hipLaunchKernelGGL(fp8col_kernel, dim3((unsigned)grid), dim3(kThreads), 0, st, packed,
                     scales_e8m0, token_offsets, num_experts, total_tokens, hidden, nchunks,
                     per_xcd, fp8_out, fp8_scales);
  return launch_status();
}
