// MFMA tile kernels of Fibonacci-spaced sparse attention (bf16 inputs, gfx950).
//
// Method: Depth-Staggered Fibonacci Spacing for Sparse Attention (gist.science
// technical summary), Methodology > Architecture and attention. A query at i
// attends the window keys i-W+1..i and, for every Fibonacci distance f_k with
// d_k = alpha*f_k >= W, the interpolated row (1-t_k) X[i-c_k] + t_k X[i-c_k+1]
// of both K and V (c_k = ceil(d_k), t_k = c_k - d_k); one softmax covers them.
//
// Work decomposition. One wavefront owns a tile of kTileQ = 15 consecutive
// queries of one (b, h). Every attended row of the tile lies in a "key block"
// of 16 consecutive rows:
//   window blocks  rows i0-16b .. i0-16b+15, b = 0..nwb-1;
//   tap blocks     rows i0-c_k .. i0-c_k+15: query i0+n needs rows n and n+1 of
//                  the block, which is why a tile holds 15 queries, not 16.
// Scores of a block come from one 16x16 MFMA product S^T = K_block Q_tile^T
// (v_mfma_f32_16x16x32_bf16, K rows as the A operand read from the block
// staged in LDS, Q rows as the B operand held in registers). For a tap block
// only the diagonal (weight 1-t) and the super-diagonal (weight t) of S^T are
// used.
//
// MFMA lane layout (16x16x32 bf16): lane l holds A[m=l%16][k=8(l/16)+e],
// B[k=8(l/16)+e][n=l%16] and C[m=4(l/16)+j][n=l%16]. With n = l%16 the query of
// the tile and g = l/16, lane (g, n) therefore holds the scores of query n
// against block rows 4g..4g+3.
//
// Blocks are taken in pairs (window pairs, then tap pairs): K and V of a pair
// are staged in the wavefront's LDS by coalesced direct-to-LDS loads, then
// consumed. Softmax is online in log2 units (running max and sum per query).
//
// P.V is the product O^T = V_blk^T P^T over the pair (32 MFMA k-slots: slots
// 8g..8g+3 are rows 4g..4g+3 of block X, slots 8g+4..8g+7 rows 4g..4g+3 of
// block Y), so the P values come straight from the score layout; V^T comes
// from transposing LDS reads (ds_read_b64_tr_b16) of the staged block. P is
// split into bf16 hi + lo parts (two MFMAs) so it keeps about 2^-16 relative.
// The backward kernels below reuse the geometry (dq) or swap the roles of
// queries and keys (dk/dv).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>

#include "fsa.h"
#include "fsa_internal.h"

namespace fsa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kTileQ = 15;          // queries per wavefront tile
constexpr int kTileK = 14;          // key rows per dk/dv tile

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Map the 1-D workgroup id to (head, tile). Workgroups are dispatched
// round-robin over the 8 XCDs; when the head count allows, all tiles of one
// head go to one XCD, consecutively, so the rows its taps re-read stay in
// that XCD's L2. Tiles run from the end of the sequence backwards: for the
// key-side kernel the query rows a tile's taps read lie ahead of it and have
// then already been fetched by the tiles dispatched before it (measured:
// dk/dv 71 -> 62 us at T=4096).
__device__ __forceinline__ void map_tile(int bid, int BH, int n_tiles, int* bh,
                                         int* tile) {
  if ((BH & 7) == 0) {
    const int xcd = bid & 7;
    const int slot = bid >> 3;
    *bh = (slot / n_tiles) * 8 + xcd;
    *tile = n_tiles - 1 - slot % n_tiles;
  } else {
    *bh = bid / n_tiles;
    *tile = n_tiles - 1 - bid % n_tiles;
  }
}

// Forward order: the tiles of `hg` heads of one XCD interleaved (tile
// positions from the end, the group's heads in turn), groups one after the
// other; hg = 1 is map_tile's order. The host picks hg so that the group's K
// and V rows fit in half of the XCD's L2: the longest tiles of all the
// group's heads then start first, and when every tile of a launch is
// resident at once they no longer end last (forward 15.9 -> 14.9 us at
// B8 H8 T1024, hg = 8; unchanged at B4 H8 T4096, hg = 2). dq takes the same
// groups (20.0 -> 19.5 us at T1024 against pairs of heads, unchanged at
// T4096); the key-side kernel keeps map_tile's order, which measured
// fastest for it.
__device__ __forceinline__ void map_tile_grouped(int bid, int BH, int n_tiles, int hg,
                                                 int* bh, int* tile) {
  if ((BH & 7) == 0 && hg > 1) {
    const int xcd = bid & 7;
    const int slot = bid >> 3;
    const int hpx = BH >> 3;
    const int gi = slot / (hg * n_tiles);
    const int h0 = gi * hg;
    const int hge = min(hg, hpx - h0);
    const int s = slot - gi * hg * n_tiles;
    *bh = (h0 + s % hge) * 8 + xcd;
    *tile = n_tiles - 1 - s / hge;
  } else {
    map_tile(bid, BH, n_tiles, bh, tile);
  }
}

// ---------------------------------------------------------------- buffer access
// Every (b, h) slab is read through a buffer resource that covers exactly the
// slab (T*D bf16). Offsets outside it -- rows before 0 or at or past T -- read
// as zero by the hardware range check, so no row index needs clamping.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           bytes, 0x00020000);
}

// A slab as a plain (base, byte length) pair; the buffer resource is formed
// where a load is issued.
struct Slab {
  const uint16_t* p;
  uint32_t bytes;
};

// A 16-byte load with the default cache policy. The tile's own rows (q and
// dout of a query tile, k and v of a key tile) are read once per launch, but
// marking these loads non-temporal made every kernel slower (measured at
// B8 H8 T1024 / B4 H8 T4096: forward 14.6 -> 14.2 / 29.6 -> 29.2 us, dq
// 20.5 -> 19.6 / 38.1 -> 37.1, dk/dv 21.0 -> 18.8 / 42.7 -> 35.2 once
// dropped).
__device__ __forceinline__ u32x4 bld16(rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Keep a byte offset whole in the VGPR operand: a constant part folded into
// the instruction's immediate field would be checked together with a negative
// VGPR part, so a row >= 0 reached from a negative block start is loaded with
// its full offset instead.
__device__ __forceinline__ int whole(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Within each 16-lane row: lane i takes lane i+1's value (row_shl:1) or lane
// i-1's value (row_shr:1); lanes whose source lies outside the row get 0.
__device__ __forceinline__ float row_next(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x101, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_prev(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
}

__device__ __forceinline__ uint2 bld8(rsrc_t r, int off) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, whole(off), 0, 0);
  return make_uint2(x[0], x[1]);
}

// Cross-row (g) sum and max of the 4 lanes l, l^16, l^32, l^48 with the
// gfx950 row-swap permutes: after permlane16_swap(x, x) the two results hold
// x[l] and x[l^16] in some order, likewise x[l^32] for permlane32_swap.
__device__ __forceinline__ float rsum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float rmax4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Hardware exp2 / log2 (v_exp_f32, v_log_f32). Arguments below -126 give
// denormal results that flush to zero; here they are softmax weights below
// 2^-126 of the largest, which do not change a sum in fp32.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// bf16 hi/lo split: hi = p truncated to bf16, lo = bf16(p - hi). The pair
// carries p to about 2^-16 relative.
__device__ __forceinline__ void split8(const float* p, u32x4* hi, u32x4* lo) {
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    r[e] = p[e] - __uint_as_float(__float_as_uint(p[e]) & 0xffff0000u);
  u32x4 h;
  bf16x8 l;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    h[e] = __builtin_amdgcn_perm(__float_as_uint(p[2 * e + 1]), __float_as_uint(p[2 * e]), 0x07060302u);
#pragma unroll
  for (int e = 0; e < 8; ++e) l[e] = static_cast<__bf16>(r[e]);
  *hi = h;
  *lo = __builtin_bit_cast(u32x4, l);
}

// A/B operand rows of a 16-row block starting at row0: lane (g, n) reads row
// row0 + n, bytes 16g.. of each 64-byte k-step. `lane_a` = n*2D + 16g.
template <int D>
__device__ __forceinline__ void bload_rows(rsrc_t r, int lane_a, int row0, u32x4* a) {
  const int off = lane_a + row0 * (2 * D);
#pragma unroll
  for (int s = 0; s < D / 32; ++s) a[s] = bld16(r, off + 64 * s);
}

template <int D>
__device__ __forceinline__ f32x4 mfma_rows(const u32x4* a, const u32x4* b) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < D / 32; ++s) acc = mfma(a[s], b[s], acc);
  return acc;
}

// Register j of a C fragment, j = 2*b1 + b0 given as lane-constant selects.
__device__ __forceinline__ float pick4(const f32x4& x, bool b0, bool b1) {
  const float lo = b0 ? x[1] : x[0];
  const float hi = b0 ? x[3] : x[2];
  return b1 ? hi : lo;
}

// Per-lane selects of the 16x16 C layout: lane (g, n) holds rows 4g..4g+3 of
// column n. For a tap block, query column n takes row n with weight 1-t and
// row n+1 with weight t; the selects pick which of the lane's 4 rows those
// are (lane-constant booleans live in scalar mask registers, not VGPRs).
struct LaneSel {
  bool on_lo, lo0, lo1;    // register n - 4g, if it is one of this lane's
  bool on_hi, hi0, hi1;    // register n + 1 - 4g, likewise
};

__device__ __forceinline__ LaneSel lane_sel(int n, int g) {
  const int jl = n - 4 * g, jh = n + 1 - 4 * g;
  return LaneSel{jl >= 0 && jl < 4, (jl & 1) != 0, (jl & 2) != 0,
                 jh >= 0 && jh < 4, (jh & 1) != 0, (jh & 2) != 0};
}

// The lower-row (row n) and upper-row (row n + 1) terms of a tap block's
// scores held by lane (g, n), zero where the lane holds neither; the
// cross-row sum over g completes them.
__device__ __forceinline__ float pick_lo(const f32x4& s, const LaneSel& ls) {
  return ls.on_lo ? pick4(s, ls.lo0, ls.lo1) : 0.f;
}
__device__ __forceinline__ float pick_hi(const f32x4& s, const LaneSel& ls) {
  return ls.on_hi ? pick4(s, ls.hi0, ls.hi1) : 0.f;
}

// ---------------------------------------------------------------- LDS tiles
// A 16-row block of a row tensor (q, k, v or dout of one slab) is staged in
// LDS row-major, 2D bytes per row, by fully coalesced 16-byte direct-to-LDS
// buffer loads (lane l of a load writes bytes 16l.. of the load's 1 KB).
//
// LDS of gfx950 (measured with the bank-conflict counter): 64 banks of 4
// bytes, i.e. one 256-byte bank line; ds_read_b64 and ds_read_b64_tr_b16
// serve 32 consecutive lanes per cycle; ds_read_b128 serves 16 lanes per
// cycle, in each half-wave the quads (lane >> 2) whose index has an even
// number of set bits ({0-3, 12-15, 20-23, 24-27} + 32h), then the others.
// Within row r the 16-byte chunk c sits at position c ^ swz(r), with
//   swz(r) = 2 * ((r / rows per bank line) mod (chunks per row / 2)),
// i.e. r & 6 for 128-byte rows and 2 (r & 7) for 256-byte rows, which keeps
// both read patterns free of bank conflicts:
//   natural operand  ds_read_b128, lane (g, n): row n, chunk g + 4s;
//   transposed       ds_read_b64_tr_b16, lanes 0-31: rows 0..7 (4g + n/4),
//                    one chunk pair {2mb, 2mb + 1} each -- the pair moves as a
//                    whole (the XOR is even), so 8 rows x 2 chunks fill all
//                    64 banks.
// ds_read_b64_tr_b16: within a 16-lane group, lane i receives element
// i % 4 of the 8 bytes that lane 4e + i/4 points at, for e = 0..3. With lane j
// pointing at row k0 + j/4, columns 16mb + 4(j%4)..+3, lane i receives
// X[k0 + e][16mb + i], e = 0..3: four consecutive rows of one column -- the
// A operand of a product over rows.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 64 ? (r & 6) : 2 * (r & 7);
}

template <int D>
struct Tile {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = D / 8;               // 16-byte chunks per row
  static constexpr int kBlockBytes = 16 * kRowBytes;   // 16 rows
  static constexpr int kLoads = kBlockBytes / 1024;    // 1 KB per wave load
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;
};

// Per-lane byte offsets, fixed for the whole kernel. The swizzle XORs chunk
// bits only, so the offsets of a family differ from their first member in bit
// fields that the row part never touches:
//   natural read, k-step s:   nat0 ^ 64 s
//   transposed read, d-block: tr0 ^ 32 mb
//   load ii of a block:       src0 + 1024 ii           (128-byte rows)
//                             (src0 ^ 128 (ii & 1)) + 1024 ii (256-byte rows)
// and three registers hold them all.
template <int D>
struct TileLane {
  int src0, nat0, tr0;
  __device__ __forceinline__ int src(int ii) const {
    return (D == 64 ? src0 : (src0 ^ (128 * (ii & 1)))) + 1024 * ii;
  }
  __device__ __forceinline__ int nat(int s) const { return nat0 ^ (64 * s); }
  __device__ __forceinline__ int tr(int mb) const { return tr0 ^ (32 * mb); }
};

// The same offsets, marked as changed so that the offsets derived from them
// are formed where they are used, not hoisted out of a loop into registers.
template <int D>
__device__ __forceinline__ TileLane<D> refresh(TileLane<D> t) {
  asm volatile("" : "+v"(t.nat0), "+v"(t.tr0));
  return t;
}

template <int D>
__device__ __forceinline__ TileLane<D> tile_lane(int lane) {
  using Tl = Tile<D>;
  TileLane<D> t;
  const int n = lane & 15, g = lane >> 4;
  const int r = 16 * lane / Tl::kRowBytes;             // row of load 0
  const int pos = (16 * lane % Tl::kRowBytes) / 16;
  t.src0 = r * Tl::kRowBytes + 16 * (pos ^ swz<D>(r));
  t.nat0 = n * Tl::kRowBytes + 16 * (g ^ swz<D>(n));
  const int row = 4 * g + (n >> 2);
  t.tr0 = row * Tl::kRowBytes + 16 * (((n & 3) >> 1) ^ swz<D>(row)) + 8 * (n & 1);
  return t;
}

// Issue the loads of rows row0..row0+15 into the LDS block at `dst`. Rows
// outside the slab are not read (buffer range check).
template <int D>
__device__ __forceinline__ void stage_block(Slab sl, const TileLane<D>& tl,
                                            int row0, lds_char* dst) {
  using Tl = Tile<D>;
  const rsrc_t r = make_rsrc(sl.p, sl.bytes);
#pragma unroll
  for (int ii = 0; ii < Tl::kLoads; ++ii)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, dst + ii * 1024, 16, whole(row0 * Tl::kRowBytes + tl.src(ii)), 0, 0, 0);
}

// Stage rows r0.. and r1.. (INT_MIN: absent) of tensors A and B into the four
// blocks A_x A_y B_x B_y of an LDS stage.
template <int D>
__device__ __forceinline__ void stage_two(Slab ra, Slab rb, const TileLane<D>& tl, int r0,
                                          int r1, lds_char* st) {
  constexpr int kB = Tile<D>::kBlockBytes;
  if (r0 != INT_MIN) {
    stage_block<D>(ra, tl, r0, st);
    stage_block<D>(rb, tl, r0, st + 2 * kB);
  }
  if (r1 != INT_MIN) {
    stage_block<D>(ra, tl, r1, st + kB);
    stage_block<D>(rb, tl, r1, st + 3 * kB);
  }
}

template <int D>
__device__ __forceinline__ void nat_operand(const lds_char* blk, const TileLane<D>& tl,
                                            u32x4* a) {
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    a[s] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(blk + tl.nat(s));
}

// A operand X^T for d-block mb over a pair of blocks (x rows 4g..4g+3 then y).
template <int D>
__device__ __forceinline__ u32x4 tr_operand(const lds_char* x, const lds_char* y,
                                            const TileLane<D>& tl, int mb) {
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(x + tl.tr(mb)));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(y + tl.tr(mb)));
  const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  u32x4 r;
  r[0] = ua.x; r[1] = ua.y; r[2] = ub.x; r[3] = ub.y;
  return r;
}

// Zero an LDS region (so that rows never loaded read as 0, not as stale
// bit patterns).
__device__ __forceinline__ void zero_lds(lds_char* p, int bytes, int lane) {
  for (int off = 16 * lane; off < bytes; off += 1024)
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(p + off) = u32x4{0u, 0u, 0u, 0u};
}

// Wait until at most n vector-memory loads of this wavefront are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}


// ---------------------------------------------------------------- tap helpers
// Tap constants live in lanes: lane t (< kNumTaps) holds tap t's values, and a
// loop over taps reads them into scalar registers with v_readlane (no memory
// access inside the loop). Lanes >= kNumTaps hold tap 0's values.
struct TapLane {
  int c;
  float wl, wh, nf;
};

// Lane L of x takes the scalar v (v_writelane_b32 with an inline-constant
// lane index).
template <int L>
__device__ __forceinline__ void write_lane(int* x, int v) {
  asm("v_writelane_b32 %0, %1, %2" : "+v"(*x) : "s"(v), "n"(L));
}

template <int L>
__device__ __forceinline__ void fill_tap_lanes(CTaps& taps, int* c, int* wl, int* wh, int* nf) {
  if constexpr (L < kNumTaps) {
    write_lane<L>(c, taps.c[L]);
    write_lane<L>(wl, __float_as_int(taps.w_lo[L]));
    write_lane<L>(wh, __float_as_int(taps.w_hi[L]));
    write_lane<L>(nf, __float_as_int(taps.neg_f[L]));
    fill_tap_lanes<L + 1>(taps, c, wl, wh, nf);
  }
}

// Built with v_writelane (one per tap and field), so that the compiler does
// not turn a per-lane select into an indexed copy of the argument block.
__device__ __forceinline__ TapLane tap_lane(CTaps& taps) {
  int c = taps.c[0], wl = __float_as_int(taps.w_lo[0]);
  int wh = __float_as_int(taps.w_hi[0]), nf = __float_as_int(taps.neg_f[0]);
  fill_tap_lanes<1>(taps, &c, &wl, &wh, &nf);
  return TapLane{c, __int_as_float(wl), __int_as_float(wh), __int_as_float(nf)};
}

__device__ __forceinline__ int rl_i(int x, int t) { return __builtin_amdgcn_readlane(x, t); }
__device__ __forceinline__ float rl_f(float x, int t) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), t));
}

// Number of taps whose lower row lies at or before `last` (the taps are sorted
// by distance, so they form a prefix).
__device__ __forceinline__ int taps_upto(const TapLane& tv, int ntaps, int lane, int last) {
  return __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < ntaps && tv.c <= last));
}

// Two cross-row (g) sums at once, each left in every lane. permlane16_swap
// exchanges the odd rows of its first operand with the even rows of its
// second; permlane32_swap exchanges rows 2-3 of the first with rows 0-1 of the
// second:
//   swap16(x, y) -> [x0 y0 x2 y2], [x1 y1 x3 y3]; sum = [x01 y01 x23 y23]
//   swap32(s, s) -> [s0 s1 s0 s1], [s2 s3 s2 s3]; sum = [X Y X Y]
//   swap16(t, t) -> [X X X X], [Y Y Y Y].
__device__ __forceinline__ void rsum4x2(float* x, float* y) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(*x), __float_as_uint(*y), false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  const float t = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  *x = __uint_as_float(c[0]);
  *y = __uint_as_float(c[1]);
}

// P operand of a tap pair. In lane (g, n), k-slot j of a block is row 4g + j;
// query n takes weight a on row n and b on row n + 1 of the block, so each
// slot holds a, b or 0. One v_perm per dword picks the upper half (the bf16
// truncation) of a or b, or zero, per 16-bit slot:
//   selector bytes 2,3 -> src1 (a), 6,7 -> src0 (b), 0x0c -> 0x00.
struct TapSel {
  uint32_t s01, s23;   // dwords with slots (0, 1) and (2, 3)
};

__device__ __forceinline__ TapSel tap_sel(int n, int g) {
  uint32_t code[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    code[j] = (4 * g + j == n) ? 0x0302u : ((4 * g + j == n + 1) ? 0x0706u : 0x0c0cu);
  return TapSel{code[0] | (code[1] << 16), code[2] | (code[3] << 16)};
}

// B operands (hi and lo bf16 parts) of a tap pair with weights (ax, bx) for
// block X and (ay, by) for block Y: hi is the truncation, lo the truncation of
// the remainder, so hi + lo carries each weight to about 2^-16 relative.
__device__ __forceinline__ void tap_operands(float ax, float bx, float ay, float by,
                                             const TapSel& ts, u32x4* hi, u32x4* lo) {
  const uint32_t uax = __float_as_uint(ax), ubx = __float_as_uint(bx);
  const uint32_t uay = __float_as_uint(ay), uby = __float_as_uint(by);
  const uint32_t rax = __float_as_uint(ax - __uint_as_float(uax & 0xffff0000u));
  const uint32_t rbx = __float_as_uint(bx - __uint_as_float(ubx & 0xffff0000u));
  const uint32_t ray = __float_as_uint(ay - __uint_as_float(uay & 0xffff0000u));
  const uint32_t rby = __float_as_uint(by - __uint_as_float(uby & 0xffff0000u));
  (*hi)[0] = __builtin_amdgcn_perm(ubx, uax, ts.s01);
  (*hi)[1] = __builtin_amdgcn_perm(ubx, uax, ts.s23);
  (*hi)[2] = __builtin_amdgcn_perm(uby, uay, ts.s01);
  (*hi)[3] = __builtin_amdgcn_perm(uby, uay, ts.s23);
  (*lo)[0] = __builtin_amdgcn_perm(rbx, rax, ts.s01);
  (*lo)[1] = __builtin_amdgcn_perm(rbx, rax, ts.s23);
  (*lo)[2] = __builtin_amdgcn_perm(rby, ray, ts.s01);
  (*lo)[3] = __builtin_amdgcn_perm(rby, ray, ts.s23);
}

// Weighted tap score part of lane (g, n): (1-t) x lower-row term + t x
// upper-row term.
__device__ __forceinline__ float tap_part(const f32x4& s, const LaneSel& ls, float wl, float wh) {
  return wl * pick_lo(s, ls) + wh * pick_hi(s, ls);
}


// Store a 16-row result tile held in the C layout of the products over rows
// (lane (g, n): row n, columns 16mb + 4g .. +3) through LDS, so that each
// non-temporal store instruction writes whole rows (1 KB: 4 rows of fp32 at
// D = 64, 2 at D = 128; bf16 rows take half). Stored piecewise from the C
// layout, the non-temporal writes cover half cache lines and are not merged
// (measured HBM writes 1.3-1.4x the bytes). Row r of the tile goes to
// dst + r*D when row_ok(r); `buf` needs 16 * (4D + 16) bytes and must no
// longer be read by this wavefront.
template <int D>
__device__ __forceinline__ void tile_to_lds(lds_char* buf, const f32x4* acc, int lane) {
  constexpr int kPitch = 4 * D + 16;                   // padded row (bank spread)
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb)
    *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(buf + n * kPitch + (16 * mb + 4 * g) * 4) = acc[mb];
  __builtin_amdgcn_s_waitcnt(0xc07f);                  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

template <int D, typename RowOk>
__device__ __forceinline__ void store_tile(lds_char* buf, const f32x4* acc, float* dst, int lane,
                                           RowOk row_ok) {
  constexpr int kPitch = 4 * D + 16;
  constexpr int kLanesPerRow = D / 4;                  // float4 per row
  constexpr int kRowsPerStore = 64 / kLanesPerRow;
  tile_to_lds<D>(buf, acc, lane);
  const int c = lane % kLanesPerRow;
#pragma unroll
  for (int it = 0; it < 16 / kRowsPerStore; ++it) {
    const int r = kRowsPerStore * it + lane / kLanesPerRow;
    const f32x4 x = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(buf + r * kPitch + 16 * c);
    if (row_ok(r)) __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(dst + static_cast<size_t>(r) * D + 4 * c));
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats as packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// The same tile rounded to bf16 (dst holds bf16 bits): 8 elements per lane.
template <int D, typename RowOk>
__device__ __forceinline__ void store_tile(lds_char* buf, const f32x4* acc, uint16_t* dst, int lane,
                                           RowOk row_ok) {
  constexpr int kPitch = 4 * D + 16;
  constexpr int kLanesPerRow = D / 8;                  // 16 bytes of bf16 per lane
  constexpr int kRowsPerStore = 64 / kLanesPerRow;
  tile_to_lds<D>(buf, acc, lane);
  const int c = lane % kLanesPerRow;
#pragma unroll
  for (int it = 0; it < 16 / kRowsPerStore; ++it) {
    const int r = kRowsPerStore * it + lane / kLanesPerRow;
    const auto* src = reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(buf + r * kPitch + 32 * c);
    const f32x4 x0 = src[0], x1 = src[1];
    const u32x4 y{pack_bf16(x0[0], x0[1]), pack_bf16(x0[2], x0[3]),
                  pack_bf16(x1[0], x1[1]), pack_bf16(x1[2], x1[3])};
    if (row_ok(r)) __builtin_nontemporal_store(y, reinterpret_cast<u32x4*>(dst + static_cast<size_t>(r) * D + 8 * c));
  }
}

// ---------------------------------------------------------------- fused RoPE
// The rotation before the gather (Depth-Staggered Fibonacci Spacing for Sparse
// Attention, Methodology > Architecture and attention > Implementation) done
// on rows the kernels hold in registers: the forward's query tile, and dq and
// dk turned back at store time. Pairs (m, m + D/2), frequency base^(-2m/D),
// row t of batch entry b at position pos0[b] + t.
constexpr double kInv2Pi = 0.15915494309189533577;   // 1 / (2 pi)

// Position of row 0 of slab bh.
__device__ __forceinline__ long long rope_row0(const RopeArg& rope, int bh, int H) {
  return rope.pos0 ? static_cast<long long>(rope.pos0[bh / H]) : 0LL;
}

// The angles of four consecutive frequencies m0..m0+3 (m0 a multiple of 4)
// at position p, formed as the RoPE pass forms them so that both give the
// same bits: theta_m0 = 2^(-(2 m0 / D) log2(base)), then times base^(-2/D)
// for each next m, in fp64; the turn count p theta / (2 pi) reduced to
// [-1/2, 1/2] in fp64; sine and cosine in fp32 of the reduced angle.
template <int D>
__device__ __forceinline__ void rope_angles4(int m0, double pd, const RopeArg& rope,
                                             float* sn, float* cs) {
  double theta = exp2(-(2.0 * m0 / D) * rope.log2_base);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    double rev = pd * theta * kInv2Pi;
    rev -= rint(rev);
    sincospif(static_cast<float>(2.0 * rev), &sn[j], &cs[j]);
    theta *= rope.ratio;
  }
}

// Turn the query tile held as B operands (lane (g, n): row n, elements
// 32s + 8g + e of k-step s, e = 0..7) to position p: the pair (m, m + D/2) is
// element e of steps s and s + D/64, m = 32s + 8g + e. Results are rounded
// to bf16, nearest even.
template <int D>
__device__ __forceinline__ void rope_qtile(u32x4* qb, int g, long long p, const RopeArg& rope) {
  constexpr int kHalf = D / 64;                        // k-steps per half row
  const double pd = static_cast<double>(p);
#pragma unroll
  for (int s = 0; s < kHalf; ++s) {
    float a[8], b[8], sn[8], cs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wa = qb[s][e >> 1], wb = qb[s + kHalf][e >> 1];
      a[e] = __uint_as_float((e & 1) ? (wa & 0xffff0000u) : (wa << 16));
      b[e] = __uint_as_float((e & 1) ? (wb & 0xffff0000u) : (wb << 16));
    }
    rope_angles4<D>(32 * s + 8 * g, pd, rope, sn, cs);
    rope_angles4<D>(32 * s + 8 * g + 4, pd, rope, sn + 4, cs + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = a[e], y = b[e];
      a[e] = fmaf(x, cs[e], -(y * sn[e]));             // the RoPE pass's rounding order
      b[e] = fmaf(x, sn[e], y * cs[e]);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      qb[s][w] = pack_bf16(a[2 * w], a[2 * w + 1]);
      qb[s + kHalf][w] = pack_bf16(b[2 * w], b[2 * w + 1]);
    }
  }
}

// Turn a result tile in the C layout of the products over rows (lane (g, n):
// row n, columns 16mb + 4g + j of acc[mb]) by the angle sgn * p * theta_m; the
// pair (m, m + D/2) is register j of acc[mb] and acc[mb + D/32],
// m = 16mb + 4g + j. sgn = -1 is the transpose: it maps a gradient with
// respect to rotated rows to the gradient with respect to the rows before
// rotation.
template <int D>
__device__ __forceinline__ void rope_tile(f32x4* acc, int g, long long p, const RopeArg& rope,
                                          float sgn) {
  constexpr int kHalf = D / 32;
  const double pd = static_cast<double>(p);
#pragma unroll
  for (int mb = 0; mb < kHalf; ++mb) {
    float sn[4], cs[4];
    rope_angles4<D>(16 * mb + 4 * g, pd, rope, sn, cs);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float s = sn[j] * sgn;
      const float x = acc[mb][j], y = acc[mb + kHalf][j];
      acc[mb][j] = fmaf(x, cs[j], -(y * s));           // the RoPE pass's rounding order
      acc[mb + kHalf][j] = fmaf(x, s, y * cs[j]);
    }
  }
}

// ---------------------------------------------------------------- forward
// One wavefront per 15-query tile. Key blocks are taken in pairs: the window
// pairs first, then the tap pairs; K and V of a pair are staged in the
// wavefront's LDS region (8 KB at D = 64), then consumed. One stage per
// wavefront keeps the LDS footprint small, so that many wavefronts per CU hide
// the load latency (a two-stage ring with the next pair in flight measured
// slower: it halves the resident wavefronts).
//
// Softmax is online, in log2 units: running max m and sum l per query. The
// window pairs update m exactly. In the tap pairs every lane of column n holds
// query n's score, and m is raised only when a score passes it by more than
// 2^kLazy (weights up to 2^kLazy are summed as they are): the rescale of the
// accumulators is then rare, and l, the output and lse stay exact.
template <int D, typename OutT, bool kRope>
__global__ __launch_bounds__(64) void fwd_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, Problem pr, TapsArg taps_arg, int n_tiles, int hg,
    OutT* __restrict__ out, float* __restrict__ lse, RopeArg rope) {
  CTaps& taps = taps_of(taps_arg);
  using Tl = Tile<D>;
  constexpr int kStage = 4 * Tl::kBlockBytes;         // K_x K_y V_x V_y
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kLazy = 8.f;
  __shared__ __attribute__((aligned(16))) char smem[kStage];
  lds_char* lds = (lds_char*)(smem);
  const int lane = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;
  const int T = pr.T, W = pr.W;
  int bh, tile;
  map_tile_grouped(blockIdx.x, pr.B * pr.H, n_tiles, hg, &bh, &tile);
  const int i0 = tile * kTileQ;
  const size_t base = static_cast<size_t>(bh) * T * D;
  const uint32_t slab = static_cast<uint32_t>(T) * D * 2;
  const rsrc_t rq = make_rsrc(q + base, slab);
  const Slab sk{k + base, slab}, sv{v + base, slab};
  const TileLane<D> tl = tile_lane<D>(lane);
  const TapLane tv = tap_lane(taps);
  const int i = i0 + n;
  const bool qvalid = n < kTileQ && i < T;
  const float c2 = pr.scale * kLog2e;                 // scores in log2 units
  const LaneSel ls = lane_sel(n, g);
  // window blocks i0 - 16b: enough for the window (a window of T or more
  // is the causal one), none wholly before row 0
  const int nwb = min((min(W, T) + kTileQ - 1) / 16 + 1, (i0 + 15) / 16 + 1);
  const int nwp = (nwb + 1) / 2;
  const int ntap = taps_upto(tv, taps.n, lane, min(i0 + kTileQ - 1, T - 1));

  zero_lds(lds, kStage, lane);
  __builtin_amdgcn_s_waitcnt(0xc07f);                  // lgkmcnt(0)

  u32x4 qb[D / 32];
  bload_rows<D>(rq, 16 * g + n * 2 * D, i0, qb);
  stage_two<D>(sk, sv, tl, i0, nwb > 1 ? i0 - 16 : INT_MIN, lds);

  f32x4 acc[D / 16];
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  // ---- window pairs: blocks i0 - 16b, b = 2p, 2p + 1
  for (int p = 0; p < nwp; ++p) {
    if (p > 0)
      stage_two<D>(sk, sv, tl, i0 - 32 * p, 2 * p + 1 < nwb ? i0 - 32 * p - 16 : INT_MIN, lds);
    wait_vm<0>();
    __builtin_amdgcn_wave_barrier();
    if (kRope && p == 0) {
      // the tile's rows have arrived: turn them, and hand the turned rows on
      rope_qtile<D>(qb, g, rope_row0(rope, bh, pr.H) + i, rope);
      if (rope.q_out != nullptr && qvalid) {
        uint16_t* dst = rope.q_out + base + static_cast<size_t>(i) * D + 8 * g;
#pragma unroll
        for (int st = 0; st < D / 32; ++st)
          __builtin_nontemporal_store(qb[st], reinterpret_cast<u32x4*>(dst + 32 * st));
      }
    }
    float sc[2][4];
    float lmax = -INFINITY;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int b = 2 * p + hf;
      u32x4 ka[D / 32];
      nat_operand<D>(lds + hf * Tl::kBlockBytes, tl, ka);
      const f32x4 s = mfma_rows<D>(ka, qb);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rel = 4 * g + j - 16 * b;            // key - i0
        const bool ok = b < nwb && qvalid && rel <= n && rel > n - W && i0 + rel >= 0;
        sc[hf][j] = ok ? s[j] * c2 : -INFINITY;
        lmax = fmaxf(lmax, sc[hf][j]);
      }
    }
    lmax = rmax4(lmax);
    const float mn = fmaxf(m, lmax);
    const float ms = mn == -INFINITY ? 0.f : mn;
    const float corr = ex2(m - ms);                    // 0 when m = -inf
    float pv[8];
    float ladd = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[e] = ex2(sc[e >> 2][e & 3] - ms);
      ladd += pv[e];
    }
    l = l * corr + rsum4(ladd);
    m = mn;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[mb][j] *= corr;
    u32x4 bhi, blo;
    split8(pv, &bhi, &blo);
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      const u32x4 a = tr_operand<D>(lds + 2 * Tl::kBlockBytes, lds + 3 * Tl::kBlockBytes, tl, mb);
      acc[mb] = mfma(a, bhi, acc[mb]);
      acc[mb] = mfma(a, blo, acc[mb]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);                // reads of stage done
    __builtin_amdgcn_wave_barrier();
  }
  // a query with no entry (outside the sequence) keeps finite exponents
  if (m == -INFINITY) m = 0.f;

  // ---- tap pairs: blocks i0 - c_t, t = 2tp, 2tp + 1
  const TapSel ts = tap_sel(n, g);
  for (int tp = 0; 2 * tp < ntap; ++tp) {
    const int t0 = 2 * tp, t1 = t0 + 1;
    const bool has1 = t1 < ntap;
    const int c0 = rl_i(tv.c, t0), c1 = rl_i(tv.c, t1);
    const float wl0 = rl_f(tv.wl, t0), wh0 = rl_f(tv.wh, t0);
    const float wl1 = rl_f(tv.wl, t1), wh1 = rl_f(tv.wh, t1);
    stage_two<D>(sk, sv, tl, i0 - c0, has1 ? i0 - c1 : INT_MIN, lds);
    wait_vm<0>();
    __builtin_amdgcn_wave_barrier();
    u32x4 ka[D / 32];
    nat_operand<D>(lds, tl, ka);
    const f32x4 s0 = mfma_rows<D>(ka, qb);
    nat_operand<D>(lds + Tl::kBlockBytes, tl, ka);
    const f32x4 s1 = mfma_rows<D>(ka, qb);
    float x0 = tap_part(s0, ls, wl0, wh0), x1 = tap_part(s1, ls, wl1, wh1);
    rsum4x2(&x0, &x1);
    const float sc0 = (qvalid && i >= c0) ? x0 * c2 : -INFINITY;
    const float sc1 = (qvalid && has1 && i >= c1) ? x1 * c2 : -INFINITY;
    const float mx = fmaxf(sc0, sc1);
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazy)) {
      const float mn = fmaxf(m, mx);
      const float corr = ex2(m - mn);
      l *= corr;
      m = mn;
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mb][j] *= corr;
    }
    const float p0 = ex2(sc0 - m), p1 = ex2(sc1 - m);
    l += p0 + p1;
    u32x4 bhi, blo;
    tap_operands(p0 * wl0, p0 * wh0, p1 * wl1, p1 * wh1, ts, &bhi, &blo);
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      const u32x4 a = tr_operand<D>(lds + 2 * Tl::kBlockBytes, lds + 3 * Tl::kBlockBytes, tl, mb);
      acc[mb] = mfma(a, bhi, acc[mb]);
      acc[mb] = mfma(a, blo, acc[mb]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }

  const float inv = qvalid ? 1.f / l : 0.f;
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[mb][j] *= inv;
  store_tile<D>(lds, acc, out + base + static_cast<size_t>(i0) * D, lane,
                [&](int r) { return r < kTileQ && i0 + r < T; });
  if (qvalid && g == 0)
    __builtin_nontemporal_store((m + lg2(l)) * 0.6931471805599453f, lse + static_cast<size_t>(bh) * T + i);
}

// ---------------------------------------------------------------- backward
// Query side: one wavefront per 15-query tile, the forward's key blocks and
// pair loop (K and V of a pair staged in LDS). For each attended entry
// e of query i, with p = exp(s - lse_i) and dP_e = dout_i . value_e:
//   Delta_i = sum_e p_e dP_e,  dS_e = p_e (dP_e - Delta_i),
//   dq_i = scale * sum_e dS_e key_e
//        = scale * (sum_e p_e dP_e key_e - Delta_i sum_e p_e key_e),
// so one pass accumulates the two products K^T (P o dP) and K^T P (MFMA, K^T
// read transposed from the same LDS tile) and applies Delta_i at the end.
// Likewise the alpha gradient of a tap entry, moving the sample point
// i - alpha*f (Depth-Staggered Fibonacci Spacing, Methodology > Architecture
// and attention > Implementation),
//   -f * [dS * scale * q.(K[a+1]-K[a]) + p * dout.(V[a+1]-V[a])]
// = A - Delta_i * B with A and B accumulated per lane. The wavefront writes
// Delta_i, dq, and one dalpha partial.
// Register budget: five wavefronts per SIMD at D = 64 (96 VGPRs).
template <int D, bool kRope>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(D == 64 ? 5 : 1))) void bwd_dq_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, Problem pr, TapsArg taps_arg, int n_tiles, int hg,
    float* __restrict__ dq, float* __restrict__ delta,
    float* __restrict__ partials, RopeArg rope) {
  CTaps& taps = taps_of(taps_arg);
  using Tl = Tile<D>;
  constexpr int kStage = 4 * Tl::kBlockBytes;          // K_x K_y V_x V_y
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ __attribute__((aligned(16))) char smem[kStage];
  lds_char* lds = (lds_char*)(smem);
  const int lane = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;
  const int T = pr.T, W = pr.W;
  int bh, tile;
  map_tile_grouped(blockIdx.x, pr.B * pr.H, n_tiles, hg, &bh, &tile);
  const int i0 = tile * kTileQ;
  const size_t base = static_cast<size_t>(bh) * T * D;
  const uint32_t slab = static_cast<uint32_t>(T) * D * 2;
  const rsrc_t rq = make_rsrc(q + base, slab);
  const rsrc_t rg = make_rsrc(dout + base, slab);
  const Slab sk{k + base, slab}, sv{v + base, slab};
  const TileLane<D> tl = tile_lane<D>(lane);
  const int i = i0 + n;
  const bool qvalid = n < kTileQ && i < T;
  const float scale = pr.scale;
  const float c2 = scale * kLog2e;
  const float L2 = qvalid ? lse[static_cast<size_t>(bh) * T + i] * kLog2e : 0.f;
  const LaneSel ls = lane_sel(n, g);
  // window blocks i0 - 16b: enough for the window (a window of T or more
  // is the causal one), none wholly before row 0
  const int nwb = min((min(W, T) + kTileQ - 1) / 16 + 1, (i0 + 15) / 16 + 1);
  const int nwp = (nwb + 1) / 2;
  int ntap = 0;                                         // taps some query reaches
  while (ntap < taps.n && taps.c[ntap] <= min(i0 + kTileQ - 1, T - 1)) ++ntap;

  zero_lds(lds, kStage, lane);
  __builtin_amdgcn_s_waitcnt(0xc07f);

  u32x4 qb[D / 32], gb[D / 32];
  bload_rows<D>(rq, 16 * g + n * 2 * D, i0, qb);
  bload_rows<D>(rg, 16 * g + n * 2 * D, i0, gb);
  stage_two<D>(sk, sv, tl, i0, nwb > 1 ? i0 - 16 : INT_MIN, lds);

  f32x4 a1[D / 16], a2[D / 16];
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) {
    a1[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    a2[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float dwin = 0.f, dtap = 0.f, al_a = 0.f, al_b = 0.f;

  // ---- window pairs: blocks i0 - 16b, b = 2p, 2p + 1
  for (int p = 0; p < nwp; ++p) {
    if (p > 0)
      stage_two<D>(sk, sv, tl, i0 - 32 * p, 2 * p + 1 < nwb ? i0 - 32 * p - 16 : INT_MIN, lds);
    wait_vm<0>();
    __builtin_amdgcn_wave_barrier();
    float w1[8], w2[8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int b = 2 * p + hf;
      u32x4 ka[D / 32], va[D / 32];
      nat_operand<D>(lds + hf * Tl::kBlockBytes, tl, ka);
      nat_operand<D>(lds + (2 + hf) * Tl::kBlockBytes, tl, va);
      const f32x4 s = mfma_rows<D>(ka, qb);
      const f32x4 d = mfma_rows<D>(va, gb);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rel = 4 * g + j - 16 * b;
        const bool ok = b < nwb && qvalid && rel <= n && rel > n - W && i0 + rel >= 0;
        const float pe = ok ? ex2(s[j] * c2 - L2) : 0.f;
        w1[4 * hf + j] = pe * d[j];
        w2[4 * hf + j] = pe;
        dwin += pe * d[j];
      }
    }
    // K^T (P o dP) first, then K^T P: one pair of hi/lo operands live at a time
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      u32x4 hi, lo;
      split8(part ? w2 : w1, &hi, &lo);
      f32x4* acc = part ? a2 : a1;
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb) {
        const u32x4 a = tr_operand<D>(lds, lds + Tl::kBlockBytes, tl, mb);
        acc[mb] = mfma(a, hi, acc[mb]);
        acc[mb] = mfma(a, lo, acc[mb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }

  // ---- tap pairs: blocks i0 - c_t, t = 2tp, 2tp + 1. The alpha-gradient
  // terms are kept as per-lane parts (the masked lower/upper row terms of
  // lane (g, n)); they are linear in those parts, so the final sum over all
  // lanes completes them without a cross-row sum per entry.
  const TapSel ts = tap_sel(n, g);
  for (int tp = 0; 2 * tp < ntap; ++tp) {
    const int t0 = 2 * tp, t1 = t0 + 1;
    const bool has1 = t1 < ntap;
    // tap constants by scalar loads from the table (no lanes held for them)
    const int t1c = min(t1, kNumTaps - 1);
    const int c0 = taps.c[t0], c1 = taps.c[t1c];
    const float wl0 = taps.w_lo[t0], wh0 = taps.w_hi[t0];
    const float wl1 = taps.w_lo[t1c], wh1 = taps.w_hi[t1c];
    const float nf0 = taps.neg_f[t0], nf1 = taps.neg_f[t1c];
    stage_two<D>(sk, sv, tl, i0 - c0, has1 ? i0 - c1 : INT_MIN, lds);
    wait_vm<0>();
    __builtin_amdgcn_wave_barrier();
    // one block at a time: its score fragments reduce to the lane's two
    // picks before the next block's are formed
    float sl[2], sh[2], dl[2], dh[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      u32x4 ka[D / 32];
      nat_operand<D>(lds + hf * Tl::kBlockBytes, tl, ka);
      const f32x4 sx = mfma_rows<D>(ka, qb);
      nat_operand<D>(lds + (2 + hf) * Tl::kBlockBytes, tl, ka);
      const f32x4 dx = mfma_rows<D>(ka, gb);
      sl[hf] = pick_lo(sx, ls);
      sh[hf] = pick_hi(sx, ls);
      dl[hf] = pick_lo(dx, ls);
      dh[hf] = pick_hi(dx, ls);
    }
    const float sl0 = sl[0], sh0 = sh[0], sl1 = sl[1], sh1 = sh[1];
    const float dl0 = dl[0], dh0 = dh[0], dl1 = dl[1], dh1 = dh[1];
    float ps0 = wl0 * sl0 + wh0 * sh0, ps1 = wl1 * sl1 + wh1 * sh1;
    float pd0 = wl0 * dl0 + wh0 * dh0, pd1 = wl1 * dl1 + wh1 * dh1;
    const float sdf0 = sh0 - sl0, sdf1 = sh1 - sl1;     // per-lane parts of q.(K[a+1]-K[a])
    const float gdf0 = dh0 - dl0, gdf1 = dh1 - dl1;     // and of dout.(V[a+1]-V[a])
    rsum4x2(&ps0, &ps1);
    rsum4x2(&pd0, &pd1);
    const float pe0 = (qvalid && i >= c0) ? ex2(ps0 * c2 - L2) : 0.f;
    const float pe1 = (qvalid && has1 && i >= c1) ? ex2(ps1 * c2 - L2) : 0.f;
    dtap += pe0 * pd0 + pe1 * pd1;
    al_a += nf0 * pe0 * (pd0 * scale * sdf0 + gdf0) + nf1 * pe1 * (pd1 * scale * sdf1 + gdf1);
    al_b += nf0 * pe0 * sdf0 + nf1 * pe1 * sdf1;
    // K^T (P o dP) first, then K^T P: one pair of hi/lo operands live at a time
    u32x4 ohi, olo;
    const float q0 = pe0 * pd0, q1 = pe1 * pd1;
    tap_operands(q0 * wl0, q0 * wh0, q1 * wl1, q1 * wh1, ts, &ohi, &olo);
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      const u32x4 a = tr_operand<D>(lds, lds + Tl::kBlockBytes, tl, mb);
      a1[mb] = mfma(a, ohi, a1[mb]);
      a1[mb] = mfma(a, olo, a1[mb]);
    }
    tap_operands(pe0 * wl0, pe0 * wh0, pe1 * wl1, pe1 * wh1, ts, &ohi, &olo);
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      const u32x4 a = tr_operand<D>(lds, lds + Tl::kBlockBytes, tl, mb);
      a2[mb] = mfma(a, ohi, a2[mb]);
      a2[mb] = mfma(a, olo, a2[mb]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }

  const float Dl = rsum4(dwin) + dtap;
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) a1[mb][j] = scale * (a1[mb][j] - Dl * a2[mb][j]);
  if (kRope)                          // the gradient of the rows before rotation
    rope_tile<D>(a1, g, rope_row0(rope, bh, pr.H) + i, rope, -1.f);
  store_tile<D>(lds, a1, dq + base + static_cast<size_t>(i0) * D, lane,
                [&](int r) { return r < kTileQ && i0 + r < T; });
  if (qvalid && g == 0)
    reinterpret_cast<float2*>(delta)[static_cast<size_t>(bh) * T + i] = make_float2(L2, Dl);
  float dal = al_a - Dl * (scale * al_b);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) dal += __shfl_xor(dal, off);
  if (lane == 0) partials[blockIdx.x] = dal;
}

// Key side: one wavefront per tile of kTileK = 14 key rows j0..j0+13, handled
// as the 16-row block rowb = j0-1 .. j0+14 (the two end rows are halos whose
// sums are discarded). Row r of the block collects
//   window: dk_r += scale dS_ir q_i, dv_r += p_ir dout_i for i = r..r+W-1;
//   tap:    the same with weight 1-t from query r + c and weight t from query
//           r + c - 1 (r is then the upper interpolation row).
// The query rows involved come in 16-row query blocks: window blocks
// rowb + 16b, and for a tap the 15 queries ib = j0+c-1 .. ib+14, which use
// block rows n' and n'+1 (the forward's geometry with the roles swapped). A
// 15-key tile would need query ib+15, whose upper row is the next tile's
// first key: its score is not in this block's product.
// Query and dout blocks of a pair are staged in LDS;
// scores are recomputed as S = Q_blk K^T (query rows natural from LDS as A,
// the tile's key rows as B in registers), so lane (g, m) holds query 4g+j
// against key m. For a tap block, query n' = 4g + jj (jj = m - 4g) lives in
// lane (g, m = n') register jj: its lower-row score is that register, its
// upper-row score register jj of lane m + 1 (one row shift).
// dk^T += Q_blk^T (W o dS) and dv^T += dout_blk^T (W o P) read Q^T and dout^T
// transposed from the same LDS tiles.

// P operand selectors of a key-side tap block: lane (g, m) places its own
// query's weight a at slot jj = m - 4g and the previous lane's weight b (query
// m - 1, for which row m is the upper row) at slot jj - 1.
__device__ __forceinline__ TapSel key_tap_sel(int n, int g) {
  const int jj = n - 4 * g;
  uint32_t code[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) code[j] = (j == jj) ? 0x0302u : ((j == jj - 1) ? 0x0706u : 0x0c0cu);
  return TapSel{code[0] | (code[1] << 16), code[2] | (code[3] << 16)};
}

// Register budget: five wavefronts per SIMD at D = 64 (96 VGPRs), three at
// D = 128 (164 VGPRs; two, at 171, took 5-8% longer at T = 65536).
template <int D, bool kRope>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(D == 64 ? 5 : 3))) void bwd_dkdv_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ partials, int n_partials, Problem pr, TapsArg taps_arg,
    int n_tiles, float* __restrict__ dk, float* __restrict__ dv,
    float* __restrict__ dalpha, RopeArg rope) {
  CTaps& taps = taps_of(taps_arg);
  using Tl = Tile<D>;
  constexpr int kStage = 4 * Tl::kBlockBytes;          // Q_x Q_y G_x G_y
  __shared__ __attribute__((aligned(16))) char smem[kStage];
  lds_char* lds = (lds_char*)(smem);
  const int lane = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;              // n: key row m of the block
  const int T = pr.T, W = pr.W;
  int bh, tile;
  map_tile(blockIdx.x, pr.B * pr.H, n_tiles, &bh, &tile);
  const int j0 = tile * kTileK;
  const int rowb = j0 - 1;
  const size_t base = static_cast<size_t>(bh) * T * D;
  const size_t rbase = static_cast<size_t>(bh) * T;
  const uint32_t slab = static_cast<uint32_t>(T) * D * 2;
  const rsrc_t rk = make_rsrc(k + base, slab);
  const rsrc_t rv = make_rsrc(v + base, slab);
  const Slab sq{q + base, slab}, sg{dout + base, slab};
  const TileLane<D> tl_ = tile_lane<D>(lane);
  const TileLane<D>& tl = tl_;
  const float scale = pr.scale;
  const float c2 = scale * 1.4426950408889634f;
  // per query {lse * log2(e), Delta}, written by the dq stage
  const rsrc_t rd = make_rsrc(delta + 2 * rbase, static_cast<uint32_t>(T) * 8u);
  // The dq stage has finished (same stream): workgroup 0, dispatched first,
  // also sums the per-tile dalpha partials, in fp64 and a fixed order: lane l
  // takes the 4-float chunks l, l + 64, ... (eight chunks in flight per
  // round), then the tail, then a butterfly over the lanes. One load and its
  // wait per partial chained n_partials / 64 L2 round trips onto this
  // workgroup, whose tile is also one of the longest, and set the end of the
  // launch (dk/dv 60 -> 48 us at T = 4096 once the loads are batched).
  if (blockIdx.x == 0) {
    double acc = 0.0;
    const int nchunk = n_partials / 4;                 // partials is 256-byte aligned
    const float4* p4 = reinterpret_cast<const float4*>(partials);
    for (int c0 = 0; c0 < nchunk; c0 += 8 * 64) {
      float4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + 64 * u + lane;
        x[u] = c < nchunk ? p4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc += static_cast<double>(x[u].x);
        acc += static_cast<double>(x[u].y);
        acc += static_cast<double>(x[u].z);
        acc += static_cast<double>(x[u].w);
      }
    }
    const int tail = 4 * nchunk + lane;
    if (tail < n_partials) acc += static_cast<double>(partials[tail]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) dalpha[0] = static_cast<float>(acc);
  }
  // window query blocks rowb + 16b: enough for the window, none wholly past
  // the last row
  const int nqb = min((min(W, T) + kTileK + 15) / 16, (T - rowb + 15) / 16);
  const int nwp = (nqb + 1) / 2;
  int ntap = 0;                                         // taps with a query < T
  while (ntap < taps.n && taps.c[ntap] <= T - j0) ++ntap;

  zero_lds(lds, kStage, lane);
  __builtin_amdgcn_s_waitcnt(0xc07f);

  u32x4 kb[D / 32], vb[D / 32];
  bload_rows<D>(rk, 16 * g + n * 2 * D, rowb, kb);
  bload_rows<D>(rv, 16 * g + n * 2 * D, rowb, vb);
  stage_two<D>(sq, sg, tl, rowb, nqb > 1 ? rowb + 16 : INT_MIN, lds);

  f32x4 ak[D / 16], av[D / 16];
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) {
    ak[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    av[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int r = rowb + n;                               // this lane's key row

  // ---- window pairs: query blocks rowb + 16b, b = 2p, 2p + 1
  for (int p = 0; p < nwp; ++p) {
    if (p > 0)
      stage_two<D>(sq, sg, tl, rowb + 32 * p, 2 * p + 1 < nqb ? rowb + 32 * p + 16 : INT_MIN, lds);
    // {L2, Delta} of queries ib+4g .. ib+4g+3 of both blocks, one 8-byte load
    // each, issued with the stage so that one wait covers both (the buffer
    // range check rejects a whole access that crosses the slab edge, so a
    // wider load would lose a valid query next to row -1 or T)
    uint2 qld[2][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        qld[hf][j] = bld8(rd, (rowb + 16 * (2 * p + hf) + 4 * g + j) * 8);
    wait_vm<0>();
    __builtin_amdgcn_wave_barrier();
    float pv[8], dsv[8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int b = 2 * p + hf;
      const int ib = rowb + 16 * b;
      u32x4 qa[D / 32], ga[D / 32];
      nat_operand<D>(lds + hf * Tl::kBlockBytes, tl, qa);
      nat_operand<D>(lds + (2 + hf) * Tl::kBlockBytes, tl, ga);
      const f32x4 s = mfma_rows<D>(qa, kb);
      const f32x4 d = mfma_rows<D>(ga, vb);
      float qL[4], qD[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qL[j] = __uint_as_float(qld[hf][j].x);
        qD[j] = __uint_as_float(qld[hf][j].y);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int iq = ib + 4 * g + j;
        const int rel = iq - r;
        const bool ok = b < nqb && iq < T && r >= 0 && rel >= 0 && rel < W;
        const float pe = ok ? ex2(s[j] * c2 - qL[j]) : 0.f;
        pv[4 * hf + j] = pe;
        dsv[4 * hf + j] = ok ? pe * (d[j] - qD[j]) : 0.f;
      }
    }
    u32x4 phi, plo, shi, slo;
    split8(pv, &phi, &plo);
    split8(dsv, &shi, &slo);
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      const u32x4 aq = tr_operand<D>(lds, lds + Tl::kBlockBytes, tl, mb);
      ak[mb] = mfma(aq, shi, ak[mb]);
      ak[mb] = mfma(aq, slo, ak[mb]);
      const u32x4 ag = tr_operand<D>(lds + 2 * Tl::kBlockBytes, lds + 3 * Tl::kBlockBytes, tl, mb);
      av[mb] = mfma(ag, phi, av[mb]);
      av[mb] = mfma(ag, plo, av[mb]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }

  // ---- tap pairs: query blocks rowb + c_t, t = 2tp, 2tp + 1
  const TapLane tv = tap_lane(taps);
  const int jj = n - 4 * g;                             // register of query n
  const bool diag = jj >= 0 && jj < 4 && n < kTileQ;    // lane holds a query
  const bool s0b = jj & 1, s1b = jj & 2;                // select register jj
  const bool u0b = (jj - 1) & 1, u1b = (jj - 1) & 2;    // select register jj - 1
  const TapSel ks = key_tap_sel(n, g);
  for (int tp = 0; 2 * tp < ntap; ++tp) {
    const int t0 = 2 * tp, t1 = t0 + 1;
    const bool has1 = t1 < ntap;
    const int c0 = rl_i(tv.c, t0), c1 = rl_i(tv.c, t1);
    const float wl0 = rl_f(tv.wl, t0), wh0 = rl_f(tv.wh, t0);
    const float wl1 = rl_f(tv.wl, t1), wh1 = rl_f(tv.wh, t1);
    const int ib0 = rowb + c0, ib1 = rowb + c1;
    stage_two<D>(sq, sg, tl, ib0, has1 ? ib1 : INT_MIN, lds);
    const uint2 ld0 = bld8(rd, (ib0 + n) * 8);          // {L2, Delta} of query n
    const uint2 ld1 = bld8(rd, (ib1 + n) * 8);
    wait_vm<0>();
    __builtin_amdgcn_wave_barrier();
    const TileLane<D> tl = refresh(tl_);
    // one block at a time (its four score fragments die before the next
    // block's are formed)
    float ps[2], pd[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const float wl = hf ? wl1 : wl0, wh = hf ? wh1 : wh0;
      u32x4 qa[D / 32];
      nat_operand<D>(lds + hf * Tl::kBlockBytes, tl, qa);
      const f32x4 sx = mfma_rows<D>(qa, kb);
      nat_operand<D>(lds + (2 + hf) * Tl::kBlockBytes, tl, qa);
      const f32x4 dx = mfma_rows<D>(qa, vb);
      ps[hf] = wl * pick4(sx, s0b, s1b) + wh * row_next(pick4(sx, u0b, u1b));
      pd[hf] = wl * pick4(dx, s0b, s1b) + wh * row_next(pick4(dx, u0b, u1b));
      __builtin_amdgcn_sched_barrier(0);
    }
    const float ps0 = ps[0], ps1 = ps[1], pd0 = pd[0], pd1 = pd[1];
    const int iq0 = ib0 + n, iq1 = ib1 + n;
    const bool ok0 = diag && iq0 < T && iq0 >= c0;
    const bool ok1 = diag && has1 && iq1 < T && iq1 >= c1;
    const float pe0 = ok0 ? ex2(ps0 * c2 - __uint_as_float(ld0.x)) : 0.f;
    const float pe1 = ok1 ? ex2(ps1 * c2 - __uint_as_float(ld1.x)) : 0.f;
    const float ds0 = ok0 ? pe0 * (pd0 - __uint_as_float(ld0.y)) : 0.f;
    const float ds1 = ok1 ? pe1 * (pd1 - __uint_as_float(ld1.y)) : 0.f;
    // dv first, then dk: one pair of hi/lo operands live at a time
    u32x4 ohi, olo;
    tap_operands(wl0 * pe0, wh0 * row_prev(pe0), wl1 * pe1, wh1 * row_prev(pe1), ks, &ohi, &olo);
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      const u32x4 ag = tr_operand<D>(lds + 2 * Tl::kBlockBytes, lds + 3 * Tl::kBlockBytes, tl, mb);
      av[mb] = mfma(ag, ohi, av[mb]);
      av[mb] = mfma(ag, olo, av[mb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    tap_operands(wl0 * ds0, wh0 * row_prev(ds0), wl1 * ds1, wh1 * row_prev(ds1), ks, &ohi, &olo);
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      const u32x4 aq = tr_operand<D>(lds, lds + Tl::kBlockBytes, tl, mb);
      ak[mb] = mfma(aq, ohi, ak[mb]);
      ak[mb] = mfma(aq, olo, ak[mb]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  }

  // rows 1 .. kTileK of the block are this tile's keys (0 and 15 are halos);
  // dv first, so that its accumulators are free while dk is scaled (and
  // turned back when RoPE is fused)
  auto key_ok = [&](int r) { return r >= 1 && r <= kTileK && rowb + r < T; };
  store_tile<D>(lds, av, dv + base + static_cast<size_t>(rowb) * D, lane, key_ok);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) ak[mb][j] *= scale;
  if (kRope)                          // the gradient of the rows before rotation
    rope_tile<D>(ak, g, rope_row0(rope, bh, pr.H) + r, rope, -1.f);
  store_tile<D>(lds, ak, dk + base + static_cast<size_t>(rowb) * D, lane, key_ok);
}

}  // namespace

bool mfma_supported(const Problem& pr, int dtype) {
  return dtype == FSA_DTYPE_BF16 && (pr.D == 64 || pr.D == 128);
}

// Heads interleaved per XCD by the query-side kernels: at most as many as
// keep their K and V rows within half of the XCD's 4 MB L2, and at most
// `cap`.
static int head_group(const Problem& pr, int cap) {
  const long long kv_head = 4LL * pr.T * pr.D;
  const long long fit = (2LL << 20) / std::max(1LL, kv_head);
  return static_cast<int>(std::max(1LL, std::min<long long>(
      std::min<long long>((pr.B * pr.H) / 8, fit), cap)));
}

hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v,
                           const Problem& pr, const TapsArg& taps, void* out,
                           bool out_bf16, float* lse, hipStream_t s,
                           const RopeArg& rope) {
  const int n_tiles = (pr.T + kTileQ - 1) / kTileQ;
  const dim3 grid(n_tiles * pr.B * pr.H);
  const int hg = head_group(pr, 8);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  auto* of = static_cast<float*>(out);
  auto* ob = static_cast<uint16_t*>(out);
#define FSA_FWD(DD, OT, R, O)                                                     \
  hipLaunchKernelGGL((fwd_mfma_kernel<DD, OT, R>), grid, dim3(64), 0, s, qq, kk, vv, \
                     pr, taps, n_tiles, hg, O, lse, rope)
  if (pr.D == 64) {
    if (rope.on) {
      if (out_bf16) FSA_FWD(64, uint16_t, true, ob); else FSA_FWD(64, float, true, of);
    } else {
      if (out_bf16) FSA_FWD(64, uint16_t, false, ob); else FSA_FWD(64, float, false, of);
    }
  } else {
    if (rope.on) {
      if (out_bf16) FSA_FWD(128, uint16_t, true, ob); else FSA_FWD(128, float, true, of);
    } else {
      if (out_bf16) FSA_FWD(128, uint16_t, false, ob); else FSA_FWD(128, float, false, of);
    }
  }
#undef FSA_FWD
  return hipGetLastError();
}

}  // namespace fsa

namespace fsa {

size_t bwd_partials_used_mfma(const Problem& pr) {
  return static_cast<size_t>((pr.T + kTileQ - 1) / kTileQ) * pr.B * pr.H;
}

hipError_t launch_bwd_dq_mfma(const void* q, const void* k, const void* v,
                              const void* dout, const float* lse,
                              const Problem& pr, const TapsArg& taps, float* dq,
                              float* delta, float* partials, hipStream_t s,
                              const RopeArg& rope) {
  const int n_tiles = (pr.T + kTileQ - 1) / kTileQ;
  const dim3 grid(n_tiles * pr.B * pr.H);
  const int hg = head_group(pr, 8);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  const auto* gg = static_cast<const uint16_t*>(dout);
#define FSA_DQ(DD, R)                                                                  \
  hipLaunchKernelGGL((bwd_dq_mfma_kernel<DD, R>), grid, dim3(64), 0, s, qq, kk, vv, gg, \
                     lse, pr, taps, n_tiles, hg, dq, delta, partials, rope)
  if (pr.D == 64) {
    if (rope.on) FSA_DQ(64, true); else FSA_DQ(64, false);
  } else {
    if (rope.on) FSA_DQ(128, true); else FSA_DQ(128, false);
  }
#undef FSA_DQ
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_mfma(const void* q, const void* k, const void* v,
                                const void* dout, const float* lse,
                                const float* delta, const float* partials,
                                size_t n_partials, const Problem& pr,
                                const TapsArg& taps, float* dk, float* dv,
                                float* dalpha, hipStream_t s, const RopeArg& rope) {
  const int n_tiles = (pr.T + kTileK - 1) / kTileK;
  const dim3 grid(n_tiles * pr.B * pr.H);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  const auto* gg = static_cast<const uint16_t*>(dout);
  const int np = static_cast<int>(n_partials);
#define FSA_DKDV(DD, R)                                                                  \
  hipLaunchKernelGGL((bwd_dkdv_mfma_kernel<DD, R>), grid, dim3(64), 0, s, qq, kk, vv, gg, \
                     lse, delta, partials, np, pr, taps, n_tiles, dk, dv, dalpha, rope)
  if (pr.D == 64) {
    if (rope.on) FSA_DKDV(64, true); else FSA_DKDV(64, false);
  } else {
    if (rope.on) FSA_DKDV(128, true); else FSA_DKDV(128, false);
  }
#undef FSA_DKDV
  return hipGetLastError();
}

}  // namespace fsa
