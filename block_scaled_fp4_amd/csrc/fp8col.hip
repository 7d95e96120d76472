// MXFP4 rows -> FP8 E4M3 over ragged expert shards (the MoE report
// "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs", section
// "核心技术贡献": item 1 the direct FP4->FP8 exponent remap with 4-to-1 scale
// alignment, item 2 the fused FP4RowToFP8Col kernel, item 3 precomputed
// ragged shard offsets), and the same conversion without the transpose.
//
// FP8 columns.  Expert e occupies positions poff(e) = 16 (ceil(off_e / 16) +
// e) .. poff(e) + n_e - 1 of a padded position space: every expert starts on
// a multiple of 16 and owns at least 16 positions, so each 16-position chunk
// lies in one expert and a 512-position tile meets at most 33 experts.  poff
// is a closed form of off_e and e (no prefix sum over the experts).
//
// A work item is (tile of 512 positions, pair of 128-channel blocks), taken
// by a workgroup of 16 waves (one per CU: its LDS tile is 128 KB):
//   1. lane l of wave w loads, for sub-block s8 = l mod 8 of the pair, the 16
//      code bytes and the block's four UE8M0 bytes of the 4 positions 4 g ..
//      4 g + 3, g = 8 w + l / 8: eight neighbouring lanes read one token's
//      whole 128-byte line.  S_tgt is the max of the four UE8M0 bytes, d =
//      S_tgt - S_sub, and the codes become E4M3 bytes through an 8-entry byte
//      table per shift d (v_perm_b32 does 4 lookups at once; the tables come
//      from the exponent-field mapping E8 = E4 - 1 + 7 - d).  4 x 4 byte
//      blocks are transposed inside the lane, and each channel's dword of 4
//      positions goes to LDS, [256 rows][128 dwords], with the columns of each
//      sub-block XOR-swizzled so that every write is bank-conflict-free;
//   2. after a barrier, wave w reads rows 16 w .. 16 w + 15, one 16-byte chunk
//      per lane, and writes it with one unaligned 16-byte store at
//      H off_e + h n_e + u.  Stores are byte-masked, so chunks of neighbouring
//      tiles and experts meet without stitching; the last chunk of an expert
//      row takes 8/4/2/1-byte stores.
// Output rows start at any byte, so the 64-byte sectors at tile seams are
// written in two parts by two tiles.  HBM takes a partial sector at about
// half the rate of a whole one unless the two parts meet in an L2 first, so
// tiles are long (512 bytes of each row) and the workgroups of one L2 domain
// convert neighbouring tiles together (see fp8col_tiles_kernel).  Offsets are clamped to [0, T]; with malformed
// (non-ascending) offsets every access still stays inside the buffers.
#include "device_common.hpp"
#include "host_common.hpp"

namespace fp4mi {
namespace {

constexpr int kMaxShift = 15;    // shifts >= 13 already map every value to 0
constexpr int kXcds = 8;         // L2 domains the workgroups are spread over

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

// A 4 x 4 byte transpose: byte j of b[r] = byte r of a[j].
__device__ __forceinline__ void transpose4x4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                             uint32_t& b0, uint32_t& b1, uint32_t& b2,
                                             uint32_t& b3) {
  const uint32_t l01 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);   // a0.0 a1.0 a0.1 a1.1
  const uint32_t h01 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);   // a0.2 a1.2 a0.3 a1.3
  const uint32_t l23 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
  const uint32_t h23 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
  b0 = __builtin_amdgcn_perm(l23, l01, 0x05040100u);
  b1 = __builtin_amdgcn_perm(l23, l01, 0x07060302u);
  b2 = __builtin_amdgcn_perm(h23, h01, 0x05040100u);
  b3 = __builtin_amdgcn_perm(h23, h01, 0x07060302u);
}

// Orders the workgroup's LDS accesses (only those: global stores in flight
// stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int kCTile = 512;                 // positions per tile
constexpr int kCThreads = 1024;             // 16 waves
constexpr int kCRowDw = kCTile / 4;         // dwords per LDS row

typedef uint32_t u32x4_ua __attribute__((ext_vector_type(4), aligned(1)));
typedef uint32_t u32x2_ua __attribute__((ext_vector_type(2), aligned(1)));
typedef uint32_t u32_ua __attribute__((aligned(1)));
typedef uint16_t u16_ua __attribute__((aligned(1)));

// Column swizzle of the LDS rows of sub-block s8 (0..7 over the block pair):
// XOR with 8 s8 + 4 (s8 / 4) dwords (the row pitch is a multiple of 64
// dwords).  A ds_write_b32 of a wave covers 8 rows (one per s8) x 8
// consecutive columns; the XOR gives the 8 rows distinct
// 8-dword groups mod 64 and, for each half wave, distinct 4-dword groups
// mod 32, so it is conflict-free with 64 or 32 banks.  Multiples of 4 keep
// every 16-byte chunk contiguous.
__device__ __forceinline__ int col_swz(int s8) { return 8 * s8 + 4 * (s8 >> 2); }

__device__ __forceinline__ int clampT(int64_t v, int T) {
  return (int)(v < 0 ? 0 : (v > T ? T : v));
}

struct ColPlan {
  int bp;              // block pair of the item
  int off1, n1, u1;    // loader: expert of the lane's 4 positions, first local index
  int e1;              // loader: that expert's index
  int off2, n2, u2;    // storer: expert of the lane's chunk, its first local index
};

struct ColRegs {
  u32x4 w[4];          // code bytes of the lane's 4 positions (one sub-block)
  uint32_t s[4];       // the block's four UE8M0 bytes for each
};

// Lane (s8, g): the 16 code bytes of sub-block s8 of the block pair (byte
// 128 bp + 16 s8 of the token row) and the UE8M0 dword of its block, for
// positions 4 g .. 4 g + 3.  Eight neighbouring lanes read one token's whole
// 128-byte line.
__device__ __forceinline__ void load_item(const uint8_t* packed, const uint8_t* sb,
                                          const ColPlan& p, int64_t HB, int64_t H, int s8,
                                          ColRegs& r) {
  const int64_t b = 2 * (int64_t)p.bp + (s8 >> 2);
  const bool blk_ok = b < HB;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int u = p.u1 + k;
    const bool ok = blk_ok && u >= 0 && u < p.n1;
    const int64_t t = (int64_t)p.off1 + u;
    // a plain load: measured ~5% faster here than the streaming (nontemporal) hint
    r.w[k] = ok ? *reinterpret_cast<const u32x4*>(packed + t * (H / 2) + 128 * (int64_t)p.bp +
                                                  16 * s8)
                : u32x4{0u, 0u, 0u, 0u};
    r.s[k] = ok ? *reinterpret_cast<const uint32_t*>(sb + t * (H / 32) + 4 * b) : 0u;
  }
}

// Stores the first L (1..15) bytes of v at p.
__device__ __forceinline__ void store_partial(uint8_t* p, u32x4 v, int L) {
  if (L & 8) *reinterpret_cast<u32x2_ua*>(p) = u32x2{v.x, v.y};
  const int o8 = L & 8;
  const uint32_t a = o8 ? v.z : v.x, a2 = o8 ? v.w : v.y;
  if (L & 4) *reinterpret_cast<u32_ua*>(p + o8) = a;
  const uint32_t c = (L & 4) ? a2 : a;                 // the dword at L & 12
  if (L & 2) *reinterpret_cast<u16_ua*>(p + (L & 12)) = (uint16_t)c;
  if (L & 1) p[L & 14] = (uint8_t)((L & 2) ? (c >> 16) : c);
}

// Clamped offsets of experts 0 .. E in LDS when E + 1 <= kOffLds (the
// expert lookups then use LDS only, so they never wait behind the global
// stores of the previous item); larger E searches global memory.
constexpr int kOffLds = 2048;

template <bool LDS_TABLE>
__device__ __forceinline__ int off_at(const int64_t* off, const int* offs, int T, int e) {
  if constexpr (LDS_TABLE) return offs[e];
  else return clampT(off[e], T);
}

// Padded start of expert e whose first token is o: PAD (ceil(o / PAD) + e).
template <int PAD>
__device__ __forceinline__ int padded_start(int o, int e) { return PAD * ((o + PAD - 1) / PAD + e); }

// Expert whose padded range holds position P, by 64-way search (uniform).
template <bool LDS_TABLE, int PAD>
__device__ int find_expert_t(const int64_t* off, const int* offs, int E, int T, int P, int lane) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int e = lo + lane * step;
    const bool le = e < hi && padded_start<PAD>(off_at<LDS_TABLE>(off, offs, T, e), e) <= P;
    const uint64_t m = __ballot(le);
    const int last = m ? 63 - __builtin_clzll(m) : 0;
    lo += last * step;
    hi = min(lo + step, hi);
  }
  return lo;
}

// Dense 128-position layout of the token-block kernel: expert e starts at
// position 128 pst[e], pst being the exclusive prefix sum of ceil(n_e / 128)
// (in LDS).  Experts with no tokens take no slot, so several can share a
// start; the search returns the last expert starting at or before P.
__device__ int find_expert_dense(const int* pst, int E, int P, int lane) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int e = lo + lane * step;
    const bool le = e < hi && 128 * pst[e] <= P;
    const uint64_t m = __ballot(le);
    const int last = m ? 63 - __builtin_clzll(m) : 0;
    lo += last * step;
    hi = min(lo + step, hi);
  }
  return lo;
}

// Plan of item (tile, bp) in the dense layout: every 128-position slot lies
// in one expert (or past the last one), so the four slots' experts are found
// first (lane k holds slot k's) and each lane takes the one of its slot.
__device__ __forceinline__ ColPlan plan_item_dense(const int* offs, const int* pst, int E, int tile,
                                                   int bp, int lane, int g, int q2) {
  const int P0 = tile * kCTile;
  int se = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int ek = find_expert_dense(pst, E, P0 + 128 * k, lane);
    se = (lane == k) ? ek : se;
  }
  const int s_off = offs[se], s_n = max(offs[se + 1] - s_off, 0), s_poff = 128 * pst[se];
  const int k1 = g >> 5, k2 = q2 >> 3;          // slots of the loader positions and of the chunk
  ColPlan p;
  p.bp = bp;
  p.off1 = __shfl(s_off, k1);
  p.n1 = __shfl(s_n, k1);
  p.u1 = P0 + 4 * g - __shfl(s_poff, k1);
  p.e1 = __shfl(se, k1);
  p.off2 = __shfl(s_off, k2);
  p.n2 = __shfl(s_n, k2);
  p.u2 = P0 + 16 * q2 - __shfl(s_poff, k2);
  return p;
}

// Plan of item (tile, bp): candidate experts e_base + lane (e_base starts at
// or before the tile), then per chunk the last candidate starting at or
// before it.
template <bool LDS_TABLE, int PAD>
__device__ __forceinline__ ColPlan plan_item(const int64_t* off, const int* offs, int E, int T,
                                             int tile, int bp, int lane, int q1, int g, int q2) {
  const int P0 = tile * kCTile;
  const int eb = find_expert_t<LDS_TABLE, PAD>(off, offs, E, T, P0, lane);
  const int e = eb + lane;
  int c_off = T, c_n = 0, c_poff = 0x7FFFFFFF;
  if (e < E) {
    c_off = off_at<LDS_TABLE>(off, offs, T, e);
    c_n = max(off_at<LDS_TABLE>(off, offs, T, e + 1) - c_off, 0);
    c_poff = padded_start<PAD>(c_off, e);
  }
  // per lane, the last candidate starting at or before each of its two chunks:
  // a binary search over the candidates' starts (ascending for ascending
  // offsets; any other order still yields a candidate index in 0..63)
  const int t1 = P0 + 16 * q1, t2 = P0 + 16 * q2;
  int i1 = 0, i2 = 0;
#pragma unroll
  for (int st = 32; st >= 1; st >>= 1) {
    const int a1 = __shfl(c_poff, i1 + st), a2 = __shfl(c_poff, i2 + st);
    i1 = (a1 <= t1) ? i1 + st : i1;
    i2 = (a2 <= t2) ? i2 + st : i2;
  }
  ColPlan p;
  p.bp = bp;
  p.off1 = __shfl(c_off, i1);
  p.n1 = __shfl(c_n, i1);
  p.u1 = P0 + 16 * q1 - __shfl(c_poff, i1) + 4 * (g & 3);
  p.e1 = eb + i1;
  p.off2 = __shfl(c_off, i2);
  p.n2 = __shfl(c_n, i2);
  p.u2 = P0 + 16 * q2 - __shfl(c_poff, i2);
  return p;
}

// Items are numbered tile fastest.  Workgroups are dispatched to the L2
// domains round-robin, so domain x holds workgroups x, x + 8, ...; it takes
// items [x ipx, (x + 1) ipx), and at step k its workgroup in slot s takes
// item x ipx + k S + s (S slots per domain).  The S workgroups of a domain
// thus convert S consecutive tiles at about the same time, and the two parts
// of an output sector that straddles neighbouring tiles mostly meet in that
// L2 before write-back instead of reaching HBM as two partial writes.  (The
// dispatch order is a performance assumption only.)
template <bool LDS_TABLE>
__global__ __launch_bounds__(kCThreads) void fp8col_tiles_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ sb,
    const int64_t* __restrict__ off, int E, int T, int64_t H, int ntiles, int64_t nitems,
    int64_t ipx, int slots, uint8_t* __restrict__ out, float* __restrict__ sc_out) {
  __shared__ uint32_t tile[2 * 128 * kCRowDw];
  __shared__ uint32_t lut[(kMaxShift + 1) * 2];
  __shared__ int offs[LDS_TABLE ? kOffLds : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // loader role: sub-block s8 of the pair, positions 4 g .. 4 g + 3 of the tile;
  // storer role: LDS rows 16 wave .. 16 wave + 15 (sub-block s8 = wave / 2)
  const int s8 = lane & 7, g = 8 * wave + (lane >> 3), q1 = g >> 2, q2 = lane & 31;
  const int64_t HB = H / 128;
  const int xcd = (int)(blockIdx.x % kXcds), slot = (int)(blockIdx.x / kXcds);
  const int64_t i0 = xcd * ipx, i1 = min(i0 + ipx, nitems);
  int64_t j = i0 + slot;
  if (j >= i1) return;                                  // uniform per workgroup
  if (tid < (kMaxShift + 1) * 2) {
    const int d = tid >> 1, hf = tid & 1;
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k) w |= remap_e2m1_to_e4m3((uint32_t)(4 * hf + k), d) << (8 * k);
    lut[tid] = w;
  }
  if constexpr (LDS_TABLE)
    for (int e = tid; e <= E; e += kCThreads) offs[e] = clampT(off[e], T);
  __syncthreads();

  ColPlan cur = plan_item<LDS_TABLE, 16>(off, offs, E, T, (int)(j % ntiles), (int)(j / ntiles), lane,
                                     q1, g, q2);
  ColRegs rc;
  load_item(packed, sb, cur, HB, H, s8, rc);

#pragma unroll 1
  for (;;) {
    // plan and loads of the next item
    const int64_t jn = j + slots;
    const bool more = jn < i1;
    ColPlan nxt = cur;
    ColRegs rn = rc;
    if (more) {
      nxt = plan_item<LDS_TABLE, 16>(off, offs, E, T, (int)(jn % ntiles), (int)(jn / ntiles), lane,
                                 q1, g, q2);
      load_item(packed, sb, nxt, HB, H, s8, rn);
    }

    // item j: remap, transpose, LDS
    uint32_t tgt_s = 0;
    {
      uint32_t ev[4][4], od[4][4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t s4 = rc.s[k];
        const uint32_t s_tgt = max(max(s4 & 0xFFu, (s4 >> 8) & 0xFFu),
                                   max((s4 >> 16) & 0xFFu, s4 >> 24));
        const uint32_t s_sub = (s4 >> (8 * (s8 & 3))) & 0xFFu;
        const int d = min((int)(s_tgt - s_sub), kMaxShift);
        const uint32_t tlo = lut[2 * d], thi = lut[2 * d + 1];
        const uint32_t ww[4] = {rc.w[k].x, rc.w[k].y, rc.w[k].z, rc.w[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = ww[i];
          ev[k][i] = __builtin_amdgcn_perm(thi, tlo, w & 0x07070707u) | ((w << 4) & 0x80808080u);
          od[k][i] = __builtin_amdgcn_perm(thi, tlo, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
        }
        tgt_s = (k == (s8 & 3)) ? s_tgt : tgt_s;
      }
      uint32_t* row0 = tile + 32 * s8 * kCRowDw + (g ^ col_swz(s8));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t y[8];
        transpose4x4(ev[0][i], ev[1][i], ev[2][i], ev[3][i], y[0], y[2], y[4], y[6]);
        transpose4x4(od[0][i], od[1][i], od[2][i], od[3][i], y[1], y[3], y[5], y[7]);
#pragma unroll
        for (int c = 0; c < 8; ++c) row0[(8 * i + c) * kCRowDw] = y[c];
      }
    }
    // fp32 scale of block 2 bp + s8 / 4 at position 4 g + s8 mod 4
    {
      const int64_t b = 2 * (int64_t)cur.bp + (s8 >> 2);
      const int u = cur.u1 + (s8 & 3);
      if (b < HB && u >= 0 && u < cur.n1)
        sc_out[HB * cur.off1 + b * cur.n1 + u] = __builtin_amdgcn_ldexpf(1.0f, (int)tgt_s - 127);
    }
    lds_barrier();
    // rows 16 wave .. 16 wave + 15, one 16-byte chunk per lane
    {
      const bool blk_ok = 2 * (int64_t)cur.bp + (wave >> 3) < HB;
      const int L = (blk_ok && cur.u2 >= 0) ? min(max(cur.n2 - cur.u2, 0), 16) : 0;
      const int64_t rowbase = H * (int64_t)cur.off2 + cur.u2;
      const uint32_t* src = tile + (16 * wave + (lane >> 5)) * kCRowDw +
                            ((4 * q2) ^ col_swz(wave >> 1));
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + 2 * k * kCRowDw);
        const int64_t h = 256 * (int64_t)cur.bp + 16 * wave + 2 * k + (lane >> 5);
        uint8_t* dst = out + rowbase + h * cur.n2;
        if (L == 16) *reinterpret_cast<u32x4_ua*>(dst) = v;
        else if (L > 0) store_partial(dst, v, L);
      }
    }
    if (!more) break;
    lds_barrier();
    j = jn;
    cur = nxt;
    rc = rn;
  }
}

// Items and workgroups of the tiled FP8-column kernel.
int launch_fp8col_tiles(const uint8_t* packed, const uint8_t* sb, const int64_t* off, int E,
                        int64_t T, int64_t H, uint8_t* out, float* sc_out, hipStream_t st) {
  const int64_t ptot = 16 * ((T + 15) / 16 + (int64_t)E);
  const int64_t ntiles = (ptot + kCTile - 1) / kCTile;
  const int64_t npairs = (H / 128 + 1) / 2;
  const int64_t nitems = ntiles * npairs;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  // one resident workgroup per CU (its LDS tile is 128 KB), spread over the
  // L2 domains
  const int64_t ipx = (nitems + kXcds - 1) / kXcds;
  int64_t slots = max((int64_t)(max(cus, 1) / kXcds), (int64_t)1);
  if (slots > ipx) slots = ipx;
  const unsigned grid = (unsigned)(kXcds * slots);
  if (E + 1 <= kOffLds)
    hipLaunchKernelGGL((fp8col_tiles_kernel<true>), dim3(grid), dim3(kCThreads), 0, st, packed,
                       sb, off, E, (int)T, H, (int)ntiles, nitems, ipx, (int)slots, out, sc_out);
  else
    hipLaunchKernelGGL((fp8col_tiles_kernel<false>), dim3(grid), dim3(kCThreads), 0, st, packed,
                       sb, off, E, (int)T, H, (int)ntiles, nitems, ipx, (int)slots, out, sc_out);
  return launch_status();
}

// ------------------------------------------- FP8 columns, blocks of 128 tokens
// The same conversion with FP8 blocks along the tokens (the FP8 copy that
// the backward pass contracts over the tokens): after the per-expert
// transpose, block j of channel h is tokens 128 j .. 128 j + 127 of the
// expert, and its target scale is the largest UE8M0 byte of those tokens for
// the channel's 32-channel group (a partial last block uses the tokens it
// has).  The tiles of fp8col_tiles_kernel are reused with every expert
// starting on a multiple of 128 positions, so every 128-position slot of a
// 512-position tile is one token block of one expert or padding.  With
// E + 1 <= kOffLds each workgroup first builds the dense layout in LDS
// (expert e at slot pst[e], the exclusive prefix sum of ceil(n_e / 128), and
// the item count from its total); otherwise, or when malformed offsets make
// that layout longer, expert e starts at slot ceil(off_e / 128) + e, a closed
// form that needs no prefix sum but pads every expert by up to a slot more
// (on 65,536 tokens over 256 Zipf(1.1) experts, 768 slots against 652).
// Per item:
//   1. each loader lane takes the largest sub-block byte of its 4 tokens; a
//      wave reduces its 8 lanes of each sub-block with shuffles and LDS
//      max-atomics combine the 4 waves of a slot: S_tgt[slot][sub-block];
//   2. after a barrier the values are remapped with d = S_tgt - S_sub and
//      transposed into the LDS tile as before, and thread (slot, channel)
//      writes the fp32 scale 2^(S_tgt - 127) of its channel and block;
//   3. after a second barrier the rows are stored as before.
// Expert e's scales form an [H, ceil(n_e / 128)] matrix at element
// H (ceil(off_e / 128) + e) in either layout: a closed form of the offsets.
template <bool LDS_TABLE>
__global__ __launch_bounds__(kCThreads) void fp8col_tokblk_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ sb,
    const int64_t* __restrict__ off, int E, int T, int64_t H, int ntiles, int64_t nitems,
    int64_t ipx, int slots, uint8_t* __restrict__ out, float* __restrict__ sc_out) {
  __shared__ uint32_t tile[2 * 128 * kCRowDw];
  __shared__ uint32_t lut[(kMaxShift + 1) * 2];
  __shared__ int offs[LDS_TABLE ? kOffLds : 1];
  __shared__ uint32_t tmax[4][8];       // S_tgt per (128-position slot, sub-block of the pair)
  __shared__ int slot_u[4], slot_n[4];  // local index of the slot's first position, expert size
  __shared__ int slot_b[4];             // the expert's first scale block: ceil(off / 128) + e
  __shared__ int pst[LDS_TABLE ? kOffLds : 1];   // dense layout: first slot of each expert
  __shared__ int wsum[kCThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s8 = lane & 7, g = 8 * wave + (lane >> 3), q1 = g >> 2, q2 = lane & 31;
  const int slot = wave >> 2;           // the loader lane's slot: positions 128 slot ..
  const int64_t HB = H / 128;
  const int xcd = (int)(blockIdx.x % kXcds), sl = (int)(blockIdx.x / kXcds);
  int64_t i0 = xcd * ipx, i1 = min(i0 + ipx, nitems);
  int64_t j = i0 + sl;
  if (!LDS_TABLE && j >= i1) return;                    // uniform per workgroup
  if (tid < (kMaxShift + 1) * 2) {
    const int d = tid >> 1, hf = tid & 1;
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k) w |= remap_e2m1_to_e4m3((uint32_t)(4 * hf + k), d) << (8 * k);
    lut[tid] = w;
  }
  if (tid < 32) tmax[tid >> 3][tid & 7] = 0u;
  if constexpr (LDS_TABLE)
    for (int e = tid; e <= E; e += kCThreads) offs[e] = clampT(off[e], T);
  __syncthreads();
  // the dense layout: thread t scans experts 2t and 2t + 1 (E + 1 <= 2 kCThreads)
  bool dense = false;
  if constexpr (LDS_TABLE) {
    const int e0 = 2 * tid, e1 = e0 + 1;
    const int a0 = e0 < E ? (max(offs[e0 + 1] - offs[e0], 0) + 127) / 128 : 0;
    const int a1 = e1 < E ? (max(offs[e1 + 1] - offs[e1], 0) + 127) / 128 : 0;
    int v = a0 + a1;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(v, d);
      v += lane >= d ? t : 0;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    const int excl = base + v - (a0 + a1);
    if (e0 <= E) pst[e0] = excl;
    if (e1 <= E) pst[e1] = excl + a0;
    __syncthreads();
    const int stot = pst[E];
    // never longer than the closed form for ordered offsets; malformed ones
    // that would make it longer keep the closed form (and its launch sizes)
    dense = stot <= (T + 127) / 128 + E;
    if (dense) {
      ntiles = (stot + 3) / 4;
      nitems = (int64_t)ntiles * ((HB + 1) / 2);
      const int64_t ipd = (nitems + kXcds - 1) / kXcds;
      i0 = xcd * ipd;
      i1 = min(i0 + ipd, nitems);
      j = i0 + sl;
    }
    if (j >= i1) return;                                // uniform per workgroup
  }

  ColPlan cur = dense ? plan_item_dense(offs, pst, E, (int)(j % ntiles), (int)(j / ntiles), lane, g, q2)
                     : plan_item<LDS_TABLE, 128>(off, offs, E, T, (int)(j % ntiles), (int)(j / ntiles),
                                                 lane, q1, g, q2);
  ColRegs rc;
  load_item(packed, sb, cur, HB, H, s8, rc);

#pragma unroll 1
  for (;;) {
    const int64_t jn = j + slots;
    const bool more = jn < i1;
    ColPlan nxt = cur;
    ColRegs rn = rc;
    if (more) {
      nxt = dense ? plan_item_dense(offs, pst, E, (int)(jn % ntiles), (int)(jn / ntiles), lane, g, q2)
                  : plan_item<LDS_TABLE, 128>(off, offs, E, T, (int)(jn % ntiles), (int)(jn / ntiles),
                                              lane, q1, g, q2);
      load_item(packed, sb, nxt, HB, H, s8, rn);
    }
    // 1. block targets (tokens outside the experts load byte 0, which never raises a max)
    {
      uint32_t m = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) m = max(m, (rc.s[k] >> (8 * (s8 & 3))) & 0xFFu);
      m = max(m, (uint32_t)__shfl_xor((int)m, 8));
      m = max(m, (uint32_t)__shfl_xor((int)m, 16));
      m = max(m, (uint32_t)__shfl_xor((int)m, 32));
      if ((lane >> 3) == 0) atomicMax(&tmax[slot][s8], m);
      if (lane == 0 && (wave & 3) == 0) {
        slot_u[slot] = cur.u1;
        slot_n[slot] = cur.n1;
        slot_b[slot] = (cur.off1 + 127) / 128 + cur.e1;
      }
    }
    lds_barrier();
    // 2. remap, transpose, LDS; scales
    {
      const uint32_t s_tgt = tmax[slot][s8];
      uint32_t ev[4][4], od[4][4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t s_sub = (rc.s[k] >> (8 * (s8 & 3))) & 0xFFu;
        const int d = min((int)(s_tgt - s_sub), kMaxShift);
        const uint32_t tlo = lut[2 * d], thi = lut[2 * d + 1];
        const uint32_t ww[4] = {rc.w[k].x, rc.w[k].y, rc.w[k].z, rc.w[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = ww[i];
          ev[k][i] = __builtin_amdgcn_perm(thi, tlo, w & 0x07070707u) | ((w << 4) & 0x80808080u);
          od[k][i] = __builtin_amdgcn_perm(thi, tlo, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
        }
      }
      uint32_t* row0 = tile + 32 * s8 * kCRowDw + (g ^ col_swz(s8));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t y[8];
        transpose4x4(ev[0][i], ev[1][i], ev[2][i], ev[3][i], y[0], y[2], y[4], y[6]);
        transpose4x4(od[0][i], od[1][i], od[2][i], od[3][i], y[1], y[3], y[5], y[7]);
#pragma unroll
        for (int c = 0; c < 8; ++c) row0[(8 * i + c) * kCRowDw] = y[c];
      }
      // thread (slot ts, channel c of the pair): fp32 scale of channel 256 bp + c, block u / 128
      const int ts = tid >> 8, c = tid & 255;
      const int u = slot_u[ts], n = slot_n[ts];
      const int64_t h = 256 * (int64_t)cur.bp + c;
      if (h < H && u >= 0 && u < n) {
        const int64_t nb = (n + 127) / 128;
        sc_out[H * (int64_t)slot_b[ts] + h * nb + u / 128] =
            __builtin_amdgcn_ldexpf(1.0f, (int)tmax[ts][c >> 5] - 127);
      }
    }
    lds_barrier();
    // 3. rows 16 wave .. 16 wave + 15, one 16-byte chunk per lane
    {
      if (tid < 32) tmax[tid >> 3][tid & 7] = 0u;       // for the next item (read before the barrier)
      const bool blk_ok = 2 * (int64_t)cur.bp + (wave >> 3) < HB;
      const int L = (blk_ok && cur.u2 >= 0) ? min(max(cur.n2 - cur.u2, 0), 16) : 0;
      const int64_t rowbase = H * (int64_t)cur.off2 + cur.u2;
      const uint32_t* src = tile + (16 * wave + (lane >> 5)) * kCRowDw +
                            ((4 * q2) ^ col_swz(wave >> 1));
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + 2 * k * kCRowDw);
        const int64_t h = 256 * (int64_t)cur.bp + 16 * wave + 2 * k + (lane >> 5);
        uint8_t* dst = out + rowbase + h * cur.n2;
        if (L == 16) *reinterpret_cast<u32x4_ua*>(dst) = v;
        else if (L > 0) store_partial(dst, v, L);
      }
    }
    if (!more) break;
    lds_barrier();
    j = jn;
    cur = nxt;
    rc = rn;
  }
}

// Items and workgroups of the token-block kernel: the tiles kernel's, over
// 128 (ceil(T / 128) + E) padded positions.
int launch_fp8col_tokblk(const uint8_t* packed, const uint8_t* sb, const int64_t* off, int E,
                         int64_t T, int64_t H, uint8_t* out, float* sc_out, hipStream_t st) {
  const int64_t ptot = 128 * ((T + 127) / 128 + (int64_t)E);
  const int64_t ntiles = (ptot + kCTile - 1) / kCTile;
  const int64_t npairs = (H / 128 + 1) / 2;
  const int64_t nitems = ntiles * npairs;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t ipx = (nitems + kXcds - 1) / kXcds;
  int64_t slots = max((int64_t)(max(cus, 1) / kXcds), (int64_t)1);
  if (slots > ipx) slots = ipx;
  const unsigned grid = (unsigned)(kXcds * slots);
  if (E + 1 <= kOffLds)
    hipLaunchKernelGGL((fp8col_tokblk_kernel<true>), dim3(grid), dim3(kCThreads), 0, st, packed,
                       sb, off, E, (int)T, H, (int)ntiles, nitems, ipx, (int)slots, out, sc_out);
  else
    hipLaunchKernelGGL((fp8col_tokblk_kernel<false>), dim3(grid), dim3(kCThreads), 0, st, packed,
                       sb, off, E, (int)T, H, (int)ntiles, nitems, ipx, (int)slots, out, sc_out);
  return launch_status();
}

// ------------------------------------------------------------ FP8 rows
// FP4RowToFP8Row: the same remap and 4-to-1 scale alignment with no
// transpose.  Thread-item s is one 32-channel sub-block of one token: its 16
// code bytes sit at 16 s, its block's four UE8M0 bytes are scale dword s / 4
// (H / 32 is a multiple of 4), its 32 FP8 bytes go to 32 s and its block's
// fp32 scale to element s / 4 -- every access a plain stream.
constexpr int kRowChunks = 2;                         // 16-channel chunks per thread

// Rows: thread t of workgroup b converts 16-channel chunks c = b 256 K + t +
// 256 k (k < K) of the flattened [T, H] codes: chunk c is half of the
// 32-channel sub-block c / 2, its 8 code bytes at 8 c, its 16 FP8 bytes at
// 16 c.  Every load and store instruction of a wave covers one contiguous
// range (512 code bytes in, 1 KiB FP8 out).
__global__ __launch_bounds__(kThreads) void fp8row_kernel(const uint8_t* __restrict__ packed,
                                                         const uint32_t* __restrict__ sb4,
                                                         int64_t n_chunk, uint8_t* __restrict__ out,
                                                         float* __restrict__ sc_out, int64_t blk0) {
  __shared__ uint32_t lut[(kMaxShift + 1) * 2];
  if (threadIdx.x < (kMaxShift + 1) * 2) {
    const int d = threadIdx.x >> 1, half = threadIdx.x & 1;
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k) w |= remap_e2m1_to_e4m3((uint32_t)(4 * half + k), d) << (8 * k);
    lut[threadIdx.x] = w;
  }
  const int64_t base = ((int64_t)blockIdx.x + blk0) * (kThreads * kRowChunks) + threadIdx.x;
  u32x2 cw[kRowChunks];
  uint32_t s4[kRowChunks];
#pragma unroll
  for (int k = 0; k < kRowChunks; ++k) {
    const int64_t c = base + (int64_t)k * kThreads;
    const bool ok = c < n_chunk;
    cw[k] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(packed + 8 * c))
               : u32x2{0u, 0u};
    s4[k] = ok ? sb4[c >> 3] : 0u;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kRowChunks; ++k) {
    const int64_t c = base + (int64_t)k * kThreads;
    if (c >= n_chunk) continue;
    const uint32_t v4 = s4[k];
    const uint32_t s_tgt = max(max(v4 & 0xFFu, (v4 >> 8) & 0xFFu), max((v4 >> 16) & 0xFFu, v4 >> 24));
    const uint32_t s_sub = (v4 >> (8 * ((c >> 1) & 3))) & 0xFFu;
    const int d = min((int)(s_tgt - s_sub), kMaxShift);
    const uint32_t tlo = lut[2 * d], thi = lut[2 * d + 1];
    const uint32_t ww[2] = {cw[k].x, cw[k].y};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      // byte i of ww[q]: channel 8q+2i (low nibble) and 8q+2i+1 (high)
      const uint32_t w = ww[q];
      const uint32_t me = __builtin_amdgcn_perm(thi, tlo, w & 0x07070707u) | ((w << 4) & 0x80808080u);
      const uint32_t mo = __builtin_amdgcn_perm(thi, tlo, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
      o[2 * q] = __builtin_amdgcn_perm(mo, me, 0x05010400u);       // channels 8q .. 8q+3
      o[2 * q + 1] = __builtin_amdgcn_perm(mo, me, 0x07030602u);   // channels 8q+4 .. 8q+7
    }
    st_u32x4(out + 16 * c, u32x4{o[0], o[1], o[2], o[3]});
    if ((c & 7) == 0) sc_out[c >> 3] = __builtin_amdgcn_ldexpf(1.0f, (int)s_tgt - 127);
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
  // token indices and padded positions (< 16 (T / 16 + E + 1)) stay in int32
  if (total_tokens >= (int64_t(1) << 26) || hidden >= (int64_t(1) << 21) ||
      num_experts >= (1 << 26))
    return FP4_ESHAPE;
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
  clear_stale_error();
  return launch_fp8col_tiles(packed, scales_e8m0, token_offsets, num_experts, total_tokens,
                             hidden, fp8_out, fp8_scales, as_stream(stream));
}

extern "C" int mxfp4_row_to_fp8_col_tokblk(const uint8_t* packed, const uint8_t* scales_e8m0,
                                           const int64_t* token_offsets, int32_t num_experts,
                                           int64_t total_tokens, int64_t hidden, uint8_t* fp8_out,
                                           float* fp8_scales, void* stream) {
  if (num_experts < 1) return FP4_EINVAL;
  if (total_tokens < 0 || hidden <= 0 || hidden % 128) return FP4_ESHAPE;
  // padded positions (< 128 (T / 128 + E + 2)) stay in int32
  if (total_tokens >= (int64_t(1) << 26) || hidden >= (int64_t(1) << 21) ||
      num_experts >= (1 << 23))
    return FP4_ESHAPE;
  int64_t n;
  if (!checked_count(total_tokens, hidden, &n)) return FP4_ESHAPE;
  if (!token_offsets) return FP4_EINVAL;
  if (n == 0) return FP4_OK;
  if (!packed || !scales_e8m0 || !fp8_out || !fp8_scales) return FP4_EINVAL;
  if (!is_aligned(packed, 16) || !is_aligned(scales_e8m0, 4) || !is_aligned(token_offsets, 8) ||
      !is_aligned(fp8_out, 4) || !is_aligned(fp8_scales, 4))
    return FP4_EALIGN;
  const int64_t pb = n / 2, sbb = n / 32, ob = n,
                scb = hidden * ((total_tokens + 127) / 128 + num_experts) * 4,
                offb = ((int64_t)num_experts + 1) * 8;
  const void* ins[3] = {packed, scales_e8m0, token_offsets};
  const int64_t inn[3] = {pb, sbb, offb};
  for (int k = 0; k < 3; ++k)
    if (overlaps(fp8_out, ob, ins[k], inn[k]) || overlaps(fp8_scales, scb, ins[k], inn[k]))
      return FP4_EOVERLAP;
  if (overlaps(fp8_out, ob, fp8_scales, scb)) return FP4_EOVERLAP;
  clear_stale_error();
  return launch_fp8col_tokblk(packed, scales_e8m0, token_offsets, num_experts, total_tokens,
                              hidden, fp8_out, fp8_scales, as_stream(stream));
}

extern "C" int mxfp4_row_to_fp8_row(const uint8_t* packed, const uint8_t* scales_e8m0,
                                    int64_t total_tokens, int64_t hidden, uint8_t* fp8_out,
                                    float* fp8_scales, void* stream) {
  if (total_tokens < 0 || hidden <= 0 || hidden % 128) return FP4_ESHAPE;
  int64_t n;
  if (!checked_count(total_tokens, hidden, &n)) return FP4_ESHAPE;
  if (n == 0) return FP4_OK;
  if (!packed || !scales_e8m0 || !fp8_out || !fp8_scales) return FP4_EINVAL;
  if (!is_aligned(packed, 16) || !is_aligned(scales_e8m0, 4) || !is_aligned(fp8_out, 16) ||
      !is_aligned(fp8_scales, 4))
    return FP4_EALIGN;
  const int64_t pb = n / 2, sbb = n / 32, ob = n, scb = (n / 128) * 4;
  if (overlaps(fp8_out, ob, packed, pb) || overlaps(fp8_out, ob, scales_e8m0, sbb) ||
      overlaps(fp8_scales, scb, packed, pb) || overlaps(fp8_scales, scb, scales_e8m0, sbb) ||
      overlaps(fp8_out, ob, fp8_scales, scb))
    return FP4_EOVERLAP;
  const int64_t n_sub = n / 32;
  const int64_t n_chunk = 2 * n_sub;
  const int64_t grid = (n_chunk + kThreads * kRowChunks - 1) / (kThreads * kRowChunks);
  clear_stale_error();
  launch_1d(fp8row_kernel, grid, kThreads, as_stream(stream), packed,
            reinterpret_cast<const uint32_t*>(scales_e8m0), n_chunk, fp8_out, fp8_scales);
  return launch_status();
}
