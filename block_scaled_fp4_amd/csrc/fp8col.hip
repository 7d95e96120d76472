// Fused MXFP4-row -> FP8-E4M3-column conversion over ragged expert shards
// (the MoE report "Practical FP4 Training for Large-Scale MoE Models on Hopper
// GPUs", section "核心技术贡献": item 1 the direct FP4->FP8 exponent remap with
// 4-to-1 scale alignment, item 2 the fused FP4RowToFP8Col kernel, item 3
// precomputed ragged shard offsets).
//
// Work decomposition.  Expert e occupies positions off[e] + kPad e ..
// off[e+1] + kPad e - 1 of a padded token space (kPad positions of padding
// after each expert stand for the fixed cost of a piece), which is cut into
// chunks of kChunk positions.  Workgroup (chunk, b) converts FP8 block b
// (128 channels) of every expert piece in its chunk; its four waves take the
// four 32-channel MXFP4 sub-blocks.  Piece boundaries are snapped to
// multiples of 4 tokens of the expert, so neighbouring chunks agree on them.
// A wave streams through the tiles of its pieces, 252 new tokens per tile
// (lane L >= 1 holds 4 consecutive tokens; lane 0 re-reads the 4 before
// them), and writes its 32 output rows, which lie one after the other in
// memory, as a stream of aligned dwords:
//   1. per token: load the 16 code bytes and the four UE8M0 bytes (one
//      dword), S_tgt = max of the four, d = S_tgt - S_sub, remap the codes to
//      E4M3 bytes through an 8-entry byte table per shift d (v_perm_b32 does
//      4 lookups at once); the tables come from the exponent-field mapping
//      E8 = E4 - 1 + 7 - d, built once per workgroup;
//   2. transpose 4 x 4 byte blocks inside the lane (v_perm_b32), giving per
//      channel a dword of the lane's 4 tokens;
//   3. a row starting m = (address mod 4) bytes past a dword boundary is
//      written with aligned dwords cut (v_alignbyte_b32) from the lane's
//      dword and the one of the lane before it (a DPP wavefront shift).  m of
//      row c is c n mod 4, so the store code is specialised on n mod 4; the
//      dword shared by the end of row h and the start of row h+1 is stitched
//      with row h+1's first 4 tokens by the piece that ends the expert.
// Loads go through buffer resources whose range check returns zero for
// tokens outside the piece, and stores not owned by the piece go to an
// offset the range check drops, so every tile issues the same memory
// operations: the loads of the next tile (of this piece or the next one)
// stay in flight while the current tile is converted and stored.  Chunks are
// laid out so that neighbouring chunks (which share output lines at their
// seams) and the two blocks that share input lines run in one L2 domain.
// Experts of fewer than 4 tokens take a per-byte path.  Expert ranges are
// clamped to [0, T], so a malformed offsets array cannot cause
// out-of-bounds accesses.
#include "device_common.hpp"
#include "host_common.hpp"

namespace fp4mi {
namespace {

constexpr int kMaxShift = 15;    // shifts >= 13 already map every value to 0
// Buffer resource word 3 for raw (untyped, stride 0) buffer access on gfx9.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kTileNew = 252;    // new tokens per wave step (4 per lane, lanes 1..63)
constexpr int kChunk = 4 * kTileNew;   // positions of the padded token space per workgroup
constexpr int kPad = kTileNew;         // padding positions after each expert
constexpr int kXcds = 8;               // L2 domains the workgroups are spread over
constexpr int kListMax = 64;           // experts listed per pass
// A buffer offset past every load and store window (windows stay below 2^31
// bytes): a load from it reads zero, a store to it is dropped.
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

// Hides a lane value from the optimiser.  Buffer offsets pass through it so
// that `valid ? offset : kOutside` stays one select feeding one memory
// operation, instead of being split into branches around two of them (which
// would leave the number of outstanding memory operations unknown and force
// waits for the previous tile's stores).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
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

struct TileIn {
  u32x4 w[4];        // code bytes of the lane's 4 tokens (one 32-channel sub-block)
  uint32_t s[4];     // their four UE8M0 block scales
};

// One expert piece: tokens [a, bb) of expert e (n tokens from off_e).
struct Piece {
  int64_t off_e;
  int e, n, a, bb, ntiles;
  int last;          // the piece ends the expert (an int: no padding to copy)
};

__device__ __forceinline__ int64_t round_up4(int64_t v) { return (v + 3) & ~int64_t(3); }
__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// Piece of expert e in chunk [g0, g1) of the padded space.
__device__ __forceinline__ Piece piece_of(const int64_t* off, int e, int64_t T, int64_t g0,
                                          int64_t g1) {
  Piece p;
  p.e = e;
  p.off_e = clamp64(off[e], 0, T);
  const int64_t end_e = clamp64(off[e + 1], p.off_e, T);
  p.n = (int)(end_e - p.off_e);                         // n < 2^26 (checked by the host)
  const int64_t pos = p.off_e + (int64_t)kPad * e;      // the expert's padded position
  p.a = (int)clamp64(round_up4(g0 - pos), 0, p.n);
  p.bb = (int)clamp64(round_up4(g1 - pos), 0, p.n);
  p.last = p.bb == p.n ? 1 : 0;
  p.ntiles = (p.bb - p.a + (p.last ? 3 : 0) + kTileNew - 1) / kTileNew;
  return p;
}

// A tile as loaded by the workgroup: thread t holds the 64 code bytes of
// block b of window tokens 64 j + t / 4 (j = 0..3), quarter t mod 4 of each
// (so four neighbouring threads read one token's 64 bytes), and the four
// UE8M0 scales of window token t.
struct TileLoad {
  u32x4 w[4];
  uint32_t s;
};

// Loads tile k of piece p (window tokens a - 4 + kTileNew k + 0..255), or,
// when !live, issues the same loads at kOutside.
__device__ __forceinline__ void load_tile(const uint8_t* packed, const uint8_t* sb, const Piece& p,
                                          int k, bool live, int64_t b, int tid, int cs, int ss,
                                          TileLoad& x) {
  // load windows: tokens a - 4 .. bb - 1 of the expert
  const int64_t wtok = p.off_e + p.a - 4;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(packed) + wtok * cs + 64 * b, (short)0, (p.bb - p.a + 4) * cs,
      kBufferWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(sb) + wtok * ss + 4 * b, (short)0, (p.bb - p.a + 4) * ss,
      kBufferWord3);
  const int first = kTileNew * k;                       // window token of the tile's first
  // window tokens 0..3 are real when the piece does not start the expert
  const bool from0 = p.a > 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = first + 64 * j + (tid >> 2);
    const bool ok = live && (from0 || tok >= 4);
    x.w[j] = __builtin_amdgcn_raw_buffer_load_b128(
        rc, opaque(ok ? tok * cs + 16 * (tid & 3) : kOutside), 0, 0);
  }
  const int tok = first + tid;
  const bool ok = live && (from0 || tok >= 4);
  x.s = __builtin_amdgcn_raw_buffer_load_b32(rs, opaque(ok ? tok * ss : kOutside), 0, 0);
}

// The tile in LDS, laid out for the reader: wave s lane L takes window tokens
// 4L..4L+3 of sub-block s, the 16 bytes of token 4L + i at position
// i ^ ((L >> 1) & 3) ^ s of its 64 bytes (the XOR spreads the 16-byte reads of
// eight neighbouring lanes over all banks).
struct TileLds {
  u32x4 codes[4][64][4];
  uint32_t scales[256];
};

__device__ __forceinline__ int swz(int i, int L, int s) { return i ^ ((L >> 1) & 3) ^ s; }

__device__ __forceinline__ void tile_to_lds(const TileLoad& x, int tid, TileLds& t) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = 64 * j + (tid >> 2), s = tid & 3, L = tok >> 2;
    t.codes[s][L][swz(tok & 3, L, s)] = x.w[j];
  }
  t.scales[tid] = x.s;
}

__device__ __forceinline__ void tile_from_lds(const TileLds& t, int wave, int lane, TileIn& x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x.w[i] = t.codes[wave][lane][swz(i, lane, wave)];
  const u32x4 sc = *reinterpret_cast<const u32x4*>(&t.scales[4 * lane]);
  x.s[0] = sc.x;
  x.s[1] = sc.y;
  x.s[2] = sc.z;
  x.s[3] = sc.w;
}

// Orders the workgroup's LDS accesses (only those: global stores in flight
// stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Remaps the lane's 4 tokens of sub-block `sub` to E4M3 and transposes them:
// Y[c] holds channel c of the 4 tokens, token j in byte j.  tgt[j] is S_tgt.
__device__ __forceinline__ void convert_tile(const TileIn& x, int sub, const uint32_t* lut,
                                             uint32_t Y[32], uint32_t tgt[4]) {
  uint32_t ev[4][4], od[4][4];   // [token][q]: channels 8q+0,2,4,6 / 8q+1,3,5,7
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
      // byte i of ww[q] holds channel 8q+2i (low nibble) and 8q+2i+1 (high);
      // the table gives the magnitude, the code's sign bit moves to bit 7
      const uint32_t w = ww[q];
      const uint32_t me = __builtin_amdgcn_perm(thi, tlo, w & 0x07070707u);
      const uint32_t mo = __builtin_amdgcn_perm(thi, tlo, (w >> 4) & 0x07070707u);
      ev[j][q] = me | ((w << 4) & 0x80808080u);
      od[j][q] = mo | (w & 0x80808080u);
    }
    tgt[j] = s_tgt;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    transpose4x4(ev[0][q], ev[1][q], ev[2][q], ev[3][q], Y[8 * q + 0], Y[8 * q + 2],
                 Y[8 * q + 4], Y[8 * q + 6]);
    transpose4x4(od[0][q], od[1][q], od[2][q], od[3][q], Y[8 * q + 1], Y[8 * q + 3],
                 Y[8 * q + 5], Y[8 * q + 7]);
  }
}

// Aligned dword stores of the 32 rows of a run for one tile.  Row c starts
// c n bytes into the run (the run itself starts dword aligned), so m =
// (c n) mod 4 = (c NM4) mod 4 is a constant per row here.  Lane L >= 1 writes
// the dword starting at row token tf = tl - m when the piece owns it: tf in
// [0, bb - m), or, when the piece ends the expert, the dwords that lie
// wholly in the row (tf <= n - 4).  The dword a row head shares with the end
// of the row before is written by stitch_row_ends.
template <int NM4>
__device__ __forceinline__ void store_rows(const uint32_t Y[32], const Piece& p, int tl, int lane,
                                           __amdgpu_buffer_rsrc_t win) {
  const int n = p.n;
  int vo[4];           // per m: window offset (8 + tf) of the lane's dword, or kOutside
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (((NM4 * 0) & 3) != m && ((NM4 * 1) & 3) != m && ((NM4 * 2) & 3) != m &&
        ((NM4 * 3) & 3) != m)
      continue;        // no row of this misalignment
    const int tf = tl - m;
    const bool owned = lane > 0 && tf >= 0 && tf < (p.last ? n - 3 : p.bb - m);
    vo[m] = opaque(owned ? 8 + tf : kOutside);
  }
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const int m = (c * NM4) & 3;
    const uint32_t own = Y[c];
    uint32_t val = own;
    if (m != 0) {
      // lane L - 1's dword (wavefront shift right by one lane; lane 0 gets 0)
      const uint32_t prev = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0x138, 0xf, 0xf, true);
      val = __builtin_amdgcn_alignbyte(own, prev, (uint32_t)(4 - m));
    }
    __builtin_amdgcn_raw_buffer_store_b32(val, win, vo[m] + c * n, 0, 0);   // row c: run byte c n
  }
}

// E4M3 byte of channel ch (0..127 within block b) of token tok.
__device__ __forceinline__ uint32_t fp8_byte(const uint8_t* __restrict__ packed,
                                             const uint8_t* __restrict__ sb, const uint32_t* lut,
                                             int64_t tok, int ch, int64_t b, int cs, int ss) {
  const uint32_t s4 = *reinterpret_cast<const uint32_t*>(sb + tok * ss + 4 * b);
  const uint32_t s_tgt = max(max(s4 & 0xFFu, (s4 >> 8) & 0xFFu), max((s4 >> 16) & 0xFFu, s4 >> 24));
  const uint32_t s_sub = (s4 >> (8 * (ch >> 5))) & 0xFFu;
  const int d = min((int)(s_tgt - s_sub), kMaxShift);
  const uint32_t code = (packed[tok * cs + 64 * b + ch / 2] >> (4 * (ch & 1))) & 0xFu;
  const uint32_t mag = __builtin_amdgcn_perm(lut[2 * d + 1], lut[2 * d], code & 7u) & 0xFFu;
  return mag | ((code & 8u) << 4);
}

// The dwords shared by the end of row c and the start of row c + 1 (c < 31)
// of the run of sub-block `wave`, for an expert of n >= 4 tokens: lane c
// assembles the last m' = ((c + 1) n) mod 4 bytes of row c and the first
// 4 - m' of row c + 1 (none when m' = 0: that row end is dword aligned).
__device__ __forceinline__ void stitch_row_ends(const uint8_t* __restrict__ packed,
                                                const uint8_t* __restrict__ sb,
                                                const uint32_t* lut, const Piece& p, int64_t H,
                                                int64_t b, int wave, int lane,
                                                uint8_t* __restrict__ out) {
  const int n = p.n, cs = (int)(H / 2), ss = (int)(H / 32);
  const int c = lane < 31 ? lane : 30;
  const int mp = ((c + 1) * n) & 3;
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool rowc = j < mp;
    const int t = rowc ? n - mp + j : j - mp;             // in [n - 3, n) or [0, 3]
    const int ch = 32 * wave + c + (rowc ? 0 : 1);
    v |= fp8_byte(packed, sb, lut, p.off_e + t, ch, b, cs, ss) << (8 * j);
  }
  const int64_t R0 = H * p.off_e + (128 * b + 32 * wave) * (int64_t)n;
  const __amdgpu_buffer_rsrc_t win = __builtin_amdgcn_make_buffer_rsrc(
      out + R0, (short)0, 32 * n, kBufferWord3);
  const bool act = lane < 31 && mp != 0;
  __builtin_amdgcn_raw_buffer_store_b32(v, win, opaque(act ? (c + 1) * n - mp : kOutside), 0, 0);
}

// Converts the listed pieces (experts lst[0..np), all with n = NM4 mod 4) of
// chunk [g0, g1), block b, as one stream of tiles; wave w converts sub-block w.
template <int NM4>
__device__ __forceinline__ void stream_pieces(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ sb,
    const int64_t* __restrict__ off, int64_t T, int64_t H, int64_t g0, int64_t g1, int64_t b,
    int tid, int wave, int lane, const uint32_t* lut, const int* lst, int np, TileLds* tiles,
    uint8_t* __restrict__ out, float* __restrict__ sc_out) {
  const int64_t HB = H / 128;
  const int cs = (int)(H / 2), ss = (int)(H / 32);      // token strides of codes and scales
  const int h0 = 128 * (int)b + 32 * wave;              // first channel of the wave's run
  auto get = [&](int i) -> Piece {
    return piece_of(off, __builtin_amdgcn_readfirstlane(lst[i]), T, g0, g1);
  };

  Piece P = get(0), Q;  // P: the piece of the tile in hand; Q: of the tile being loaded
  int iP = 0, kP = 0, iQ = 0, kQ = 0;

  // Converts and stores tile kP of P.
  auto process = [&](const TileIn& x) {
    uint32_t Y[32], tgt[4];
    convert_tile(x, wave, lut, Y, tgt);
    const int tl = P.a - 4 + kTileNew * kP + 4 * lane;  // the lane's first token
    const int64_t R0 = H * P.off_e + (int64_t)h0 * P.n; // the run of 32 rows
    float* const so = sc_out + HB * P.off_e + b * P.n;
    // stores go through the run's window, which begins 8 bytes before the
    // run (R0 is a multiple of 32, so every owned offset is positive)
    const __amdgpu_buffer_rsrc_t win = __builtin_amdgcn_make_buffer_rsrc(
        out + R0 - 8, (short)0, 32 * P.n + 8, kBufferWord3);
    const __amdgpu_buffer_rsrc_t wsc = __builtin_amdgcn_make_buffer_rsrc(
        so, (short)0, 4 * P.n, kBufferWord3);
    // wave w stores the FP8 block scale of the lane's token w
    const uint32_t tg = wave == 0 ? tgt[0] : wave == 1 ? tgt[1] : wave == 2 ? tgt[2] : tgt[3];
    const bool sc_ok = lane > 0 && tl + wave < P.bb;
    __builtin_amdgcn_raw_buffer_store_b32(
        __float_as_uint(__builtin_amdgcn_ldexpf(1.0f, (int)tg - 127)), wsc,
        opaque(sc_ok ? 4 * (tl + wave) : kOutside), 0, 0);
    store_rows<NM4>(Y, P, tl, lane, win);
  };
  // The tile after (Q, kQ)... set Q, kQ to the tile after (P, kP): the next
  // of P, else the first of the next piece.
  auto advance = [&]() -> bool {
    if (kP + 1 < P.ntiles) {
      Q = P;
      iQ = iP;
      kQ = kP + 1;
      return true;
    }
    if (iP + 1 >= np) return false;
    iQ = iP + 1;
    kQ = 0;
    Q = get(iQ);
    return true;
  };
  auto take = [&]() {
    P = Q;
    iP = iQ;
    kP = kQ;
  };

  // Tiles pass through two LDS buffers.  Every step issues the same global
  // memory operations (the next tile's 5 loads, then 33 stores), so the
  // loads of the next tile stay in flight while this one is converted and
  // stored, and the wait for them leaves this tile's stores outstanding.
  TileLoad G;
  TileIn x;
  load_tile(packed, sb, P, 0, true, b, tid, cs, ss, G);
  __builtin_amdgcn_s_waitcnt(0);                        // every entry to the loop alike
  tile_to_lds(G, tid, tiles[0]);
  lds_barrier();
  bool more = advance();
  for (int buf = 0;; buf ^= 1) {
    load_tile(packed, sb, more ? Q : P, kQ, more, b, tid, cs, ss, G);
    tile_from_lds(tiles[buf], wave, lane, x);
    process(x);
    if (!more) break;
    take();
    more = advance();
    tile_to_lds(G, tid, tiles[buf ^ 1]);
    lds_barrier();
  }
  lds_barrier();                                        // the buffers are free again
}

__global__ __launch_bounds__(kThreads) void fp8col_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ sb,
    const int64_t* __restrict__ off, int32_t E, int64_t T, int64_t H, int64_t nchunks,
    int64_t per_xcd, uint8_t* __restrict__ out, float* __restrict__ sc_out) {
  __shared__ uint32_t lut[(kMaxShift + 1) * 2];
  __shared__ int counts[6];                             // expert range; pieces per class
  __shared__ int lists[4][kListMax];                    // pieces of >= 4 tokens, by n mod 4
  __shared__ TileLds tiles[2];                          // the tile stream's two buffers
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
  // (uniform values; saying so keeps the piece state in scalar registers)
  const int e_first = __builtin_amdgcn_readfirstlane(max(counts[0] - 1, 0));
  const int e_end = __builtin_amdgcn_readfirstlane(counts[1]);

  const int cs = (int)(H / 2), ss = (int)(H / 32);      // token strides of codes and scales
  const int h0 = 128 * (int)b + 32 * wave;              // first channel of the wave's run

  // Experts are taken kListMax at a time (one pass: a chunk meets at most
  // kChunk / kPad + 1 experts when the offsets ascend): their pieces of 4 or
  // more tokens are listed in LDS by n mod 4, the others (1..3 tokens) are
  // converted byte by byte.
  for (int eb = e_first; eb < e_end; eb += kListMax) {
    __syncthreads();                                    // the lists are free again
    if (tid < 4) counts[2 + tid] = 0;
    __syncthreads();
    const int e = eb + tid;
    if (tid < kListMax && e < e_end) {
      const Piece p = piece_of(off, e, T, g0, g1);
      if (p.a < p.bb && p.n >= 4) lists[p.n & 3][atomicAdd(&counts[2 + (p.n & 3)], 1)] = e;
    }
    // Experts of 1..3 tokens: one piece each; rows shorter than a dword, so
    // each output byte is computed and stored on its own.  Experts of 4 or
    // more whose last piece is here: the dwords at their row junctions.
    for (int et = eb; et < min(eb + kListMax, e_end); ++et) {
      const Piece p = piece_of(off, et, T, g0, g1);
      if (p.a >= p.bb) continue;
      if (p.n >= 4) {
        if (p.last) stitch_row_ends(packed, sb, lut, p, H, b, wave, lane, out);
        continue;
      }
      const int n = p.n;
      const int64_t R0 = H * p.off_e + (int64_t)h0 * n;
      for (int i = lane; i < 32 * n; i += 64) {
        const int r = i / n, t = i - r * n;
        out[R0 + (int64_t)r * n + t] =
            (uint8_t)fp8_byte(packed, sb, lut, p.off_e + t, 32 * wave + r, b, cs, ss);
      }
      if (wave == 0 && lane < n) {
        const uint32_t s4 = *reinterpret_cast<const uint32_t*>(sb + (p.off_e + lane) * ss + 4 * b);
        const uint32_t s_tgt = max(max(s4 & 0xFFu, (s4 >> 8) & 0xFFu),
                                   max((s4 >> 16) & 0xFFu, s4 >> 24));
        sc_out[HB * p.off_e + b * n + lane] = __builtin_amdgcn_ldexpf(1.0f, (int)s_tgt - 127);
      }
    }
    __syncthreads();
#pragma unroll 1
    for (int cls = 0; cls < 4; ++cls) {
      const int np = __builtin_amdgcn_readfirstlane(counts[2 + cls]);
      if (np == 0) continue;
      const int* lst = lists[cls];
      switch (cls) {
        case 0: stream_pieces<0>(packed, sb, off, T, H, g0, g1, b, tid, wave, lane, lut, lst, np, tiles, out, sc_out); break;
        case 1: stream_pieces<1>(packed, sb, off, T, H, g0, g1, b, tid, wave, lane, lut, lst, np, tiles, out, sc_out); break;
        case 2: stream_pieces<2>(packed, sb, off, T, H, g0, g1, b, tid, wave, lane, lut, lst, np, tiles, out, sc_out); break;
        default: stream_pieces<3>(packed, sb, off, T, H, g0, g1, b, tid, wave, lane, lut, lst, np, tiles, out, sc_out); break;
      }
    }
  }
}

// ------------------------------------------------------------ FP8 rows
// FP4RowToFP8Row: the same remap and 4-to-1 scale alignment with no
// transpose.  Thread-item s is one 32-channel sub-block of one token: its 16
// code bytes sit at 16 s, its block's four UE8M0 bytes are scale dword s / 4
// (H / 32 is a multiple of 4), its 32 FP8 bytes go to 32 s and its block's
// fp32 scale to element s / 4 -- every access a plain stream.
constexpr int kRowItems = 1;                          // sub-blocks per thread (1 measured best)

__global__ __launch_bounds__(kThreads) void fp8row_kernel(const uint8_t* __restrict__ packed,
                                                         const uint32_t* __restrict__ sb4,
                                                         int64_t n_sub, uint8_t* __restrict__ out,
                                                         float* __restrict__ sc_out) {
  __shared__ uint32_t lut[(kMaxShift + 1) * 2];
  if (threadIdx.x < (kMaxShift + 1) * 2) {
    const int d = threadIdx.x >> 1, half = threadIdx.x & 1;
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k) w |= remap_e2m1_to_e4m3((uint32_t)(4 * half + k), d) << (8 * k);
    lut[threadIdx.x] = w;
  }
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kRowItems) + threadIdx.x;
  u32x4 cw[kRowItems];
  uint32_t s4[kRowItems];
#pragma unroll
  for (int k = 0; k < kRowItems; ++k) {
    const int64_t s = base + (int64_t)k * kThreads;
    const bool ok = s < n_sub;
    cw[k] = ok ? ld_u32x4(packed + 16 * s) : u32x4{0u, 0u, 0u, 0u};
    s4[k] = ok ? sb4[s >> 2] : 0u;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kRowItems; ++k) {
    const int64_t s = base + (int64_t)k * kThreads;
    if (s >= n_sub) continue;
    const uint32_t v4 = s4[k];
    const uint32_t s_tgt = max(max(v4 & 0xFFu, (v4 >> 8) & 0xFFu), max((v4 >> 16) & 0xFFu, v4 >> 24));
    const uint32_t s_sub = (v4 >> (8 * (s & 3))) & 0xFFu;
    const int d = min((int)(s_tgt - s_sub), kMaxShift);
    const uint32_t tlo = lut[2 * d], thi = lut[2 * d + 1];
    const uint32_t ww[4] = {cw[k].x, cw[k].y, cw[k].z, cw[k].w};
    uint32_t o[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // byte i of ww[q]: channel 8q+2i (low nibble) and 8q+2i+1 (high)
      const uint32_t w = ww[q];
      const uint32_t me = __builtin_amdgcn_perm(thi, tlo, w & 0x07070707u) | ((w << 4) & 0x80808080u);
      const uint32_t mo = __builtin_amdgcn_perm(thi, tlo, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
      o[2 * q] = __builtin_amdgcn_perm(mo, me, 0x05010400u);       // channels 8q .. 8q+3
      o[2 * q + 1] = __builtin_amdgcn_perm(mo, me, 0x07030602u);   // channels 8q+4 .. 8q+7
    }
    st_u32x4(out + 32 * s, u32x4{o[0], o[1], o[2], o[3]});
    st_u32x4(out + 32 * s + 16, u32x4{o[4], o[5], o[6], o[7]});
    if ((s & 3) == 0) sc_out[s >> 2] = __builtin_amdgcn_ldexpf(1.0f, (int)s_tgt - 127);
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
  const int64_t grid = (n_sub + kThreads * kRowItems - 1) / (kThreads * kRowItems);
  if (grid > 0x7FFFFFFF) return FP4_ESHAPE;
  hipLaunchKernelGGL(fp8row_kernel, dim3((unsigned)grid), dim3(kThreads), 0, as_stream(stream),
                     packed, reinterpret_cast<const uint32_t*>(scales_e8m0), n_sub, fp8_out,
                     fp8_scales);
  return launch_status();
}
