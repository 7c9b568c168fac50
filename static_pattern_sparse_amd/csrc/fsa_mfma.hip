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
// (v_mfma_f32_16x16x32_bf16, K rows as the A operand straight from global
// memory, Q rows as the B operand held in registers). For a tap block only the
// diagonal (weight 1-t) and the super-diagonal (weight t) of S^T are used.
//
// MFMA lane layout (16x16x32 bf16): lane l holds A[m=l%16][k=8(l/16)+e],
// B[k=8(l/16)+e][n=l%16] and C[m=4(l/16)+j][n=l%16]. With n = l%16 the query of
// the tile and g = l/16, lane (g, n) therefore holds the scores of query n
// against block rows 4g..4g+3.
//
// The softmax is not online: a tile's whole attended set (at most
// 16*nwb + 15 entries per query) fits in registers, so scores are formed
// first, then max, sum and lse, then P.V.
//
// P.V is the product O^T = V_blk^T P^T over pairs of key blocks (32 MFMA
// k-slots: slots 8g..8g+3 are rows 4g..4g+3 of block X, slots 8g+4..8g+7 rows
// 4g..4g+3 of block Y), so the P values come straight from the score layout.
// V^T is staged through LDS: each lane loads a 4x4 (row x column) bf16 patch,
// transposes it with byte permutes and writes 4 keys per column. P is split
// into bf16 hi + lo parts (two MFMAs) so its rounding stays near 2^-17.
#include <hip/hip_runtime.h>

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
constexpr int kMaxWinBlocks = 3;    // window blocks: W <= 33
constexpr int kLdsRowBytes = 72;    // one d-row of V^T: 32 keys (64 B) + pad

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

__device__ __forceinline__ float xsum4(float x) {   // sum over g = 0..3
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float xmax4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// bf16 hi/lo split of 8 fp32 values into two B operands.
__device__ __forceinline__ void split_hi_lo(const float* p, u32x4* hi, u32x4* lo) {
  bf16x8 h, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 he = static_cast<__bf16>(p[e]);
    h[e] = he;
    l[e] = static_cast<__bf16>(p[e] - static_cast<float>(he));
  }
  *hi = __builtin_bit_cast(u32x4, h);
  *lo = __builtin_bit_cast(u32x4, l);
}

// Map the 1-D workgroup id to (head, tile). Workgroups are dispatched
// round-robin over the 8 XCDs; when the head count allows, all tiles of one
// head go to one XCD, in order, so the rows its taps re-read stay in that
// XCD's L2.
__device__ __forceinline__ void map_tile(int bid, int BH, int n_tiles, int* bh,
                                         int* tile) {
  if ((BH & 7) == 0) {
    const int xcd = bid & 7;
    const int slot = bid >> 3;
    *bh = (slot / n_tiles) * 8 + xcd;
    *tile = slot % n_tiles;
  } else {
    *bh = bid / n_tiles;
    *tile = bid % n_tiles;
  }
}

// S^T block (16 rows from row0) x Q tile: lane (g, n) gets q_n . K[row0+4g+j].
template <int D>
__device__ __forceinline__ f32x4 score_block(const uint16_t* K, int row0, int T,
                                             const u32x4* qb, int n, int g) {
  const int row = clampi(row0 + n, 0, T - 1);
  const uint16_t* p = K + static_cast<size_t>(row) * D + 8 * g;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < D / 32; ++s) acc = mfma(ld16(p + 32 * s), qb[s], acc);
  return acc;
}

// Stage rows row0..row0+15 of X (clamped to the sequence) transposed into the
// X (half = 0) or Y (half = 1) half of an LDS pair buffer; lane (cc, rg)
// handles rows 4rg..4rg+3 and columns 4cc..4cc+3 (+64h). A missing block
// (row0 == INT_MIN) is written as zeros.
template <int D>
__device__ __forceinline__ void stage_t(const uint16_t* X, int row0, int T,
                                         char* lds, int half, int lane) {
  const int cc = lane >> 2, rg = lane & 3;
#pragma unroll
  for (int h = 0; h < D / 64; ++h) {
    uint2 r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (row0 == INT_MIN) {
        r[i] = make_uint2(0u, 0u);
      } else {
        const int row = clampi(row0 + 4 * rg + i, 0, T - 1);
        r[i] = *reinterpret_cast<const uint2*>(X + static_cast<size_t>(row) * D +
                                               64 * h + 4 * cc);
      }
    }
    const uint32_t sel_lo = 0x05040100u, sel_hi = 0x07060302u;
    uint2 col[4];
    col[0] = make_uint2(__builtin_amdgcn_perm(r[1].x, r[0].x, sel_lo),
                        __builtin_amdgcn_perm(r[3].x, r[2].x, sel_lo));
    col[1] = make_uint2(__builtin_amdgcn_perm(r[1].x, r[0].x, sel_hi),
                        __builtin_amdgcn_perm(r[3].x, r[2].x, sel_hi));
    col[2] = make_uint2(__builtin_amdgcn_perm(r[1].y, r[0].y, sel_lo),
                        __builtin_amdgcn_perm(r[3].y, r[2].y, sel_lo));
    col[3] = make_uint2(__builtin_amdgcn_perm(r[1].y, r[0].y, sel_hi),
                        __builtin_amdgcn_perm(r[3].y, r[2].y, sel_hi));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d = 64 * h + 4 * cc + c;
      *reinterpret_cast<uint2*>(lds + d * kLdsRowBytes + 32 * half + 8 * rg) = col[c];
    }
  }
}

// A operand X^T of a product over rows (d-block mb): lane (g, n) reads
// d = 16mb + n, rows 4g..4g+3 of block X and of block Y.
__device__ __forceinline__ u32x4 t_operand(const char* lds, int mb, int n, int g) {
  const char* row = lds + (16 * mb + n) * kLdsRowBytes + 8 * g;
  const uint2 x = *reinterpret_cast<const uint2*>(row);
  const uint2 y = *reinterpret_cast<const uint2*>(row + 32);
  u32x4 a;
  a[0] = x.x; a[1] = x.y; a[2] = y.x; a[3] = y.y;
  return a;
}

// ---------------------------------------------------------------- forward
template <int D>
__global__ __launch_bounds__(64) void fwd_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, Problem pr, Taps taps, int n_tiles,
    float* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) char lds[D * kLdsRowBytes];
  const int lane = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;
  const int T = pr.T, W = pr.W;
  int bh, tile;
  map_tile(blockIdx.x, pr.B * pr.H, n_tiles, &bh, &tile);
  const int i0 = tile * kTileQ;
  const size_t base = static_cast<size_t>(bh) * T * D;
  const uint16_t* Q = q + base;
  const uint16_t* K = k + base;
  const uint16_t* V = v + base;
  const int i = i0 + n;                                  // this lane's query
  const bool qvalid = n < kTileQ && i < T;

  u32x4 qb[D / 32];
  {
    const uint16_t* p = Q + static_cast<size_t>(clampi(i, 0, T - 1)) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qb[s] = ld16(p + 32 * s);
  }
  const float scale = pr.scale;
  const int nwb = (W + kTileQ - 1) / 16 + 1;             // window blocks in use
  // taps some query of the tile reaches
  const int last = min(i0 + kTileQ - 1, T - 1);
  int ntap = 0;
  while (ntap < taps.n && taps.c[ntap] <= last) ++ntap;

  // ---- scores
  float sw[kMaxWinBlocks][4];
  float st[kNumTaps];
  float m = -INFINITY;
#pragma unroll
  for (int b = 0; b < kMaxWinBlocks; ++b) {
    if (b < nwb) {
      const f32x4 s = score_block<D>(K, i0 - 16 * b, T, qb, n, g);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rel = 4 * g + j - 16 * b;              // key - i0
        const bool ok = qvalid && rel <= n && rel > n - W && i0 + rel >= 0;
        sw[b][j] = ok ? s[j] * scale : -INFINITY;
        m = fmaxf(m, sw[b][j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) sw[b][j] = -INFINITY;
    }
  }
#pragma unroll
  for (int t = 0; t < kNumTaps; ++t) {
    st[t] = -INFINITY;
    if (t < ntap) {
      const int c = taps.c[t];
      const f32x4 s = score_block<D>(K, i0 - c, T, qb, n, g);
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = 4 * g + j;
        part += key == n ? taps.w_lo[t] * s[j] : 0.f;
        part += key == n + 1 ? taps.w_hi[t] * s[j] : 0.f;
      }
      const float sc = xsum4(part) * scale;
      st[t] = (qvalid && i >= c) ? sc : -INFINITY;
      m = fmaxf(m, st[t]);
    }
  }
  m = xmax4(m);
  const float mm = m == -INFINITY ? 0.f : m;
  float zw = 0.f;
#pragma unroll
  for (int b = 0; b < kMaxWinBlocks; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) zw += __expf(sw[b][j] - mm);
  float z = xsum4(zw);
#pragma unroll
  for (int t = 0; t < kNumTaps; ++t) z += __expf(st[t] - mm);
  const float L = qvalid ? mm + __logf(z) : 0.f;

  // ---- P.V over pairs of key blocks: window blocks first, then taps
  f32x4 acc[D / 16];
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nblk = nwb + ntap;
  for (int pb = 0; pb < nblk; pb += 2) {
    float pv[8];
    int rows[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int blk = pb + hf;
      if (blk >= nblk) {
        rows[hf] = INT_MIN;
#pragma unroll
        for (int j = 0; j < 4; ++j) pv[4 * hf + j] = 0.f;
      } else if (blk < nwb) {
        rows[hf] = i0 - 16 * blk;
        // select the window block's scores (blk is wave-uniform)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float s = sw[0][j];
#pragma unroll
          for (int b = 1; b < kMaxWinBlocks; ++b) s = blk == b ? sw[b][j] : s;
          pv[4 * hf + j] = __expf(s - L);
        }
      } else {
        const int t = blk - nwb;
        float s = st[0], wl = taps.w_lo[0], wh = taps.w_hi[0];
        int c = taps.c[0];
#pragma unroll
        for (int u = 1; u < kNumTaps; ++u) {
          if (t == u) { s = st[u]; wl = taps.w_lo[u]; wh = taps.w_hi[u]; c = taps.c[u]; }
        }
        rows[hf] = i0 - c;
        const float p = __expf(s - L);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = 4 * g + j;
          pv[4 * hf + j] = key == n ? p * wl : (key == n + 1 ? p * wh : 0.f);
        }
      }
    }
    __syncthreads();
    stage_t<D>(V, rows[0], T, lds, 0, lane);
    stage_t<D>(V, rows[1], T, lds, 1, lane);
    __syncthreads();
    u32x4 bhi, blo;
    split_hi_lo(pv, &bhi, &blo);
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      const u32x4 a = t_operand(lds, mb, n, g);
      acc[mb] = mfma(a, bhi, acc[mb]);
      acc[mb] = mfma(a, blo, acc[mb]);
    }
  }

  if (qvalid) {
    float* o = out + base + static_cast<size_t>(i) * D + 4 * g;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb)
      *reinterpret_cast<float4*>(o + 16 * mb) =
          make_float4(acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]);
    if (g == 0) lse[static_cast<size_t>(bh) * T + i] = L;
  }
}


// ---------------------------------------------------------------- backward
// Query side, one wavefront per 15-query tile (same key blocks as the
// forward). For every attended entry e of query i, with p = exp(s - lse_i):
//   dP_e = dout_i . value_e,  Delta_i = sum_e p_e dP_e,  dS_e = p_e (dP_e - Delta_i),
//   dq_i = scale * sum_e dS_e key_e.
// S^T and dP^T of a block come from two MFMA products (K and V rows as A,
// the tile's q and dout rows as B). dq^T = K^T dS^T runs over pairs of
// blocks with K^T staged through LDS, like V^T in the forward. A tap entry's
// alpha gradient is -f * [dS * scale * q.(K[a+1]-K[a]) + p * dout.(V[a+1]-V[a])]
// (moving alpha moves the sample point i - alpha*f; Depth-Staggered Fibonacci
// Spacing, Methodology > Architecture and attention > Implementation); one
// partial per wavefront goes to `partials`, Delta_i to `delta`.
template <int D>
__global__ __launch_bounds__(64) void bwd_dq_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, Problem pr, Taps taps, int n_tiles,
    float* __restrict__ dq, float* __restrict__ delta,
    float* __restrict__ partials) {
  __shared__ __attribute__((aligned(16))) char lds[D * kLdsRowBytes];
  const int lane = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;
  const int T = pr.T, W = pr.W;
  int bh, tile;
  map_tile(blockIdx.x, pr.B * pr.H, n_tiles, &bh, &tile);
  const int i0 = tile * kTileQ;
  const size_t base = static_cast<size_t>(bh) * T * D;
  const uint16_t* Q = q + base;
  const uint16_t* K = k + base;
  const uint16_t* V = v + base;
  const uint16_t* G = dout + base;
  const int i = i0 + n;
  const bool qvalid = n < kTileQ && i < T;
  const int ic = clampi(i, 0, T - 1);

  u32x4 qb[D / 32], gb[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    qb[s] = ld16(Q + static_cast<size_t>(ic) * D + 8 * g + 32 * s);
    gb[s] = ld16(G + static_cast<size_t>(ic) * D + 8 * g + 32 * s);
  }
  const float L = qvalid ? lse[static_cast<size_t>(bh) * T + i] : 0.f;
  const float scale = pr.scale;
  const int nwb = (W + kTileQ - 1) / 16 + 1;
  const int last = min(i0 + kTileQ - 1, T - 1);
  int ntap = 0;
  while (ntap < taps.n && taps.c[ntap] <= last) ++ntap;

  // ---- p and dP of every entry, Delta
  float pw[kMaxWinBlocks][4], gw[kMaxWinBlocks][4];
  float pt[kNumTaps], gt[kNumTaps], sdf[kNumTaps], gdf[kNumTaps];
  float dpart = 0.f;
#pragma unroll
  for (int b = 0; b < kMaxWinBlocks; ++b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) { pw[b][j] = 0.f; gw[b][j] = 0.f; }
    if (b < nwb) {
      const f32x4 s = score_block<D>(K, i0 - 16 * b, T, qb, n, g);
      const f32x4 d = score_block<D>(V, i0 - 16 * b, T, gb, n, g);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rel = 4 * g + j - 16 * b;
        const bool ok = qvalid && rel <= n && rel > n - W && i0 + rel >= 0;
        pw[b][j] = ok ? __expf(s[j] * scale - L) : 0.f;
        gw[b][j] = d[j];
        dpart += pw[b][j] * d[j];
      }
    }
  }
  float Dl = xsum4(dpart);
#pragma unroll
  for (int t = 0; t < kNumTaps; ++t) {
    pt[t] = 0.f; gt[t] = 0.f; sdf[t] = 0.f; gdf[t] = 0.f;
    if (t < ntap) {
      const int c = taps.c[t];
      const float wl = taps.w_lo[t], wh = taps.w_hi[t];
      const f32x4 s = score_block<D>(K, i0 - c, T, qb, n, g);
      const f32x4 d = score_block<D>(V, i0 - c, T, gb, n, g);
      float ps = 0.f, pd = 0.f, ds = 0.f, dd = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = 4 * g + j;
        const float lo = key == n ? 1.f : 0.f, hi = key == n + 1 ? 1.f : 0.f;
        ps += (wl * lo + wh * hi) * s[j];
        pd += (wl * lo + wh * hi) * d[j];
        ds += (hi - lo) * s[j];
        dd += (hi - lo) * d[j];
      }
      ps = xsum4(ps); pd = xsum4(pd); ds = xsum4(ds); dd = xsum4(dd);
      const bool ok = qvalid && i >= c;
      pt[t] = ok ? __expf(ps * scale - L) : 0.f;
      gt[t] = pd;
      sdf[t] = ds;
      gdf[t] = dd;
      Dl += pt[t] * pd;
    }
  }

  // ---- dS, dalpha, dq^T = K^T dS^T
  float dal = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nblk = nwb + ntap;
  for (int pb = 0; pb < nblk; pb += 2) {
    float dsv[8];
    int rows[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int blk = pb + hf;
      if (blk >= nblk) {
        rows[hf] = INT_MIN;
#pragma unroll
        for (int j = 0; j < 4; ++j) dsv[4 * hf + j] = 0.f;
      } else if (blk < nwb) {
        rows[hf] = i0 - 16 * blk;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float p = pw[0][j], d = gw[0][j];
#pragma unroll
          for (int b = 1; b < kMaxWinBlocks; ++b) {
            p = blk == b ? pw[b][j] : p;
            d = blk == b ? gw[b][j] : d;
          }
          dsv[4 * hf + j] = p * (d - Dl);
        }
      } else {
        const int t = blk - nwb;
        float p = pt[0], d = gt[0], sd = sdf[0], gd = gdf[0];
        float wl = taps.w_lo[0], wh = taps.w_hi[0], nf = taps.neg_f[0];
        int c = taps.c[0];
#pragma unroll
        for (int u = 1; u < kNumTaps; ++u) {
          if (t == u) {
            p = pt[u]; d = gt[u]; sd = sdf[u]; gd = gdf[u];
            wl = taps.w_lo[u]; wh = taps.w_hi[u]; nf = taps.neg_f[u]; c = taps.c[u];
          }
        }
        rows[hf] = i0 - c;
        const float ds = p * (d - Dl);
        if (g == 0) dal += nf * (ds * scale * sd + p * gd);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = 4 * g + j;
          dsv[4 * hf + j] = key == n ? ds * wl : (key == n + 1 ? ds * wh : 0.f);
        }
      }
    }
    __syncthreads();
    stage_t<D>(K, rows[0], T, lds, 0, lane);
    stage_t<D>(K, rows[1], T, lds, 1, lane);
    __syncthreads();
    u32x4 bhi, blo;
    split_hi_lo(dsv, &bhi, &blo);
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      const u32x4 a = t_operand(lds, mb, n, g);
      acc[mb] = mfma(a, bhi, acc[mb]);
      acc[mb] = mfma(a, blo, acc[mb]);
    }
  }

  if (qvalid) {
    float* o = dq + base + static_cast<size_t>(i) * D + 4 * g;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb)
      *reinterpret_cast<float4*>(o + 16 * mb) =
          make_float4(acc[mb][0] * scale, acc[mb][1] * scale,
                      acc[mb][2] * scale, acc[mb][3] * scale);
    if (g == 0) delta[static_cast<size_t>(bh) * T + i] = Dl;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) dal += __shfl_xor(dal, off);
  if (lane == 0) partials[blockIdx.x] = dal;
}

// Key side, one wavefront per tile of kTileK = 14 key rows j0..j0+13, handled
// as the 16-row block rowb = j0-1 .. j0+14 (the two end rows are halos whose
// sums are discarded). Row r of the block collects
//   window: dk_r += scale dS_ir q_i, dv_r += p_ir dout_i for i = r..r+W-1;
//   tap:    the same with weight 1-t from query r + c and weight t from query
//           r + c - 1 (r is then the upper interpolation row).
// For a tap, the 15 queries ib = j0+c-1 .. ib+14 use block rows n' and n'+1,
// exactly the forward's tile/block geometry with the roles swapped. Their
// scores are recomputed with S = Q_span K_blk^T (query rows as A, the block's
// key rows as B held in registers), so lane (g, m) holds query 4g+j against
// key m: a tap score needs lanes m and m+1 of the same 16-lane row. The
// weighted dS (and p) blocks are then exactly the B operand of
// dk^T += Q_span^T (W o dS), dv^T += dout_span^T (W o P), over pairs of blocks,
// with Q^T and dout^T staged through LDS.
constexpr int kTileK = 14;

template <int D>
__global__ __launch_bounds__(64) void bwd_dkdv_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, Problem pr,
    Taps taps, int n_tiles, float* __restrict__ dk, float* __restrict__ dv) {
  __shared__ __attribute__((aligned(16))) char ldq[D * kLdsRowBytes];
  __shared__ __attribute__((aligned(16))) char ldg[D * kLdsRowBytes];
  const int lane = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;          // n: key row m of the block
  const int T = pr.T, W = pr.W;
  int bh, tile;
  map_tile(blockIdx.x, pr.B * pr.H, n_tiles, &bh, &tile);
  const int j0 = tile * kTileK;
  const int rowb = j0 - 1;
  const size_t base = static_cast<size_t>(bh) * T * D;
  const size_t rbase = static_cast<size_t>(bh) * T;
  const uint16_t* Q = q + base;
  const uint16_t* K = k + base;
  const uint16_t* V = v + base;
  const uint16_t* G = dout + base;
  const float scale = pr.scale;

  u32x4 kb[D / 32], vb[D / 32];
  {
    const int r = clampi(rowb + n, 0, T - 1);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      kb[s] = ld16(K + static_cast<size_t>(r) * D + 8 * g + 32 * s);
      vb[s] = ld16(V + static_cast<size_t>(r) * D + 8 * g + 32 * s);
    }
  }
  const int nqb = (W + kTileK + 15) / 16;          // window query blocks
  int ntap = 0;                                     // taps with a query < T
  while (ntap < taps.n && j0 + taps.c[ntap] - 1 <= T - 1) ++ntap;

  f32x4 ak[D / 16], av[D / 16];
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) {
    ak[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    av[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int nblk = nqb + ntap;
  for (int pb = 0; pb < nblk; pb += 2) {
    float pv[8], dsv[8];
    int rows[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int blk = pb + hf;
      if (blk >= nblk) {
        rows[hf] = INT_MIN;
#pragma unroll
        for (int j = 0; j < 4; ++j) { pv[4 * hf + j] = 0.f; dsv[4 * hf + j] = 0.f; }
      } else if (blk < nqb) {
        // window: queries ib + 4g + j against key rowb + n
        const int ib = rowb + 16 * blk;
        rows[hf] = ib;
        const f32x4 s = score_block<D>(Q, ib, T, kb, n, g);
        const f32x4 d = score_block<D>(G, ib, T, vb, n, g);
        const int r = rowb + n;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int iq = ib + 4 * g + j;
          const int rel = iq - r;
          const bool ok = iq < T && r >= 0 && rel >= 0 && rel < W;
          const int ii = clampi(iq, 0, T - 1);
          const float p = ok ? __expf(s[j] * scale - lse[rbase + ii]) : 0.f;
          pv[4 * hf + j] = p;
          dsv[4 * hf + j] = p * (d[j] - (ok ? delta[rbase + ii] : 0.f));
        }
      } else {
        const int t = blk - nqb;
        float wl = taps.w_lo[0], wh = taps.w_hi[0];
        int c = taps.c[0];
#pragma unroll
        for (int u = 1; u < kNumTaps; ++u) {
          if (t == u) { wl = taps.w_lo[u]; wh = taps.w_hi[u]; c = taps.c[u]; }
        }
        const int ib = j0 + c - 1;                 // query of span row 0
        rows[hf] = ib;
        const f32x4 s = score_block<D>(Q, ib, T, kb, n, g);
        const f32x4 d = score_block<D>(G, ib, T, vb, n, g);
        // query m (this lane's column) reads key rows m (lo) and m + 1 (hi)
        float s_lo = 0.f, s_hi = 0.f, d_lo = 0.f, d_hi = 0.f;
        const int jj = n - 4 * g;                  // reg holding query m here
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float su = __shfl_down(s[j], 1, 16);
          const float du = __shfl_down(d[j], 1, 16);
          if (jj == j) { s_lo = s[j]; s_hi = su; d_lo = d[j]; d_hi = du; }
        }
        const int iq = ib + n;
        const bool ok = jj >= 0 && jj < 4 && n < kTileQ && iq < T && iq >= c;
        const int ii = clampi(iq, 0, T - 1);
        const float p = ok ? __expf((wl * s_lo + wh * s_hi) * scale - lse[rbase + ii]) : 0.f;
        const float ds = ok ? p * (wl * d_lo + wh * d_hi - delta[rbase + ii]) : 0.f;
        const float p_up = __shfl_up(p, 1, 16);     // query m-1's values
        const float ds_up = __shfl_up(ds, 1, 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int qn = 4 * g + j;                 // query of reg j
          pv[4 * hf + j] = n == qn ? wl * p : (n == qn + 1 ? wh * p_up : 0.f);
          dsv[4 * hf + j] = n == qn ? wl * ds : (n == qn + 1 ? wh * ds_up : 0.f);
        }
      }
    }
    __syncthreads();
    stage_t<D>(Q, rows[0], T, ldq, 0, lane);
    stage_t<D>(Q, rows[1], T, ldq, 1, lane);
    stage_t<D>(G, rows[0], T, ldg, 0, lane);
    stage_t<D>(G, rows[1], T, ldg, 1, lane);
    __syncthreads();
    u32x4 phi, plo, shi, slo;
    split_hi_lo(pv, &phi, &plo);
    split_hi_lo(dsv, &shi, &slo);
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      const u32x4 aq = t_operand(ldq, mb, n, g);
      ak[mb] = mfma(aq, shi, ak[mb]);
      ak[mb] = mfma(aq, slo, ak[mb]);
      const u32x4 ag = t_operand(ldg, mb, n, g);
      av[mb] = mfma(ag, phi, av[mb]);
      av[mb] = mfma(ag, plo, av[mb]);
    }
  }

  const int r = rowb + n;
  if (n >= 1 && n <= kTileK && r < T) {
    float* ok_ = dk + base + static_cast<size_t>(r) * D + 4 * g;
    float* ov = dv + base + static_cast<size_t>(r) * D + 4 * g;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      *reinterpret_cast<float4*>(ok_ + 16 * mb) =
          make_float4(ak[mb][0] * scale, ak[mb][1] * scale, ak[mb][2] * scale,
                      ak[mb][3] * scale);
      *reinterpret_cast<float4*>(ov + 16 * mb) =
          make_float4(av[mb][0], av[mb][1], av[mb][2], av[mb][3]);
    }
  }
}

}  // namespace

bool mfma_supported(const Problem& pr, int dtype) {
  // the window of query i0 reaches back W-1 rows: ceil((W-1)/16) + 1 blocks
  return dtype == FSA_DTYPE_BF16 && (pr.D == 64 || pr.D == 128) &&
         pr.W <= 16 * (kMaxWinBlocks - 1) + 1;
}

hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v,
                           const Problem& pr, const Taps& taps, float* out,
                           float* lse, hipStream_t s) {
  const int n_tiles = (pr.T + kTileQ - 1) / kTileQ;
  const dim3 grid(n_tiles * pr.B * pr.H);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  if (pr.D == 64)
    hipLaunchKernelGGL(fwd_mfma_kernel<64>, grid, dim3(64), 0, s, qq, kk, vv, pr,
                       taps, n_tiles, out, lse);
  else
    hipLaunchKernelGGL(fwd_mfma_kernel<128>, grid, dim3(64), 0, s, qq, kk, vv, pr,
                       taps, n_tiles, out, lse);
  return hipGetLastError();
}

}  // namespace fsa

namespace fsa {

size_t bwd_partials_used_mfma(const Problem& pr) {
  return static_cast<size_t>((pr.T + kTileQ - 1) / kTileQ) * pr.B * pr.H;
}

hipError_t launch_bwd_dq_mfma(const void* q, const void* k, const void* v,
                              const void* dout, const float* lse,
                              const Problem& pr, const Taps& taps, float* dq,
                              float* delta, float* partials, hipStream_t s) {
  const int n_tiles = (pr.T + kTileQ - 1) / kTileQ;
  const dim3 grid(n_tiles * pr.B * pr.H);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  const auto* gg = static_cast<const uint16_t*>(dout);
  if (pr.D == 64)
    hipLaunchKernelGGL(bwd_dq_mfma_kernel<64>, grid, dim3(64), 0, s, qq, kk, vv,
                       gg, lse, pr, taps, n_tiles, dq, delta, partials);
  else
    hipLaunchKernelGGL(bwd_dq_mfma_kernel<128>, grid, dim3(64), 0, s, qq, kk, vv,
                       gg, lse, pr, taps, n_tiles, dq, delta, partials);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_mfma(const void* q, const void* k, const void* v,
                                const void* dout, const float* lse,
                                const float* delta, const Problem& pr,
                                const Taps& taps, float* dk, float* dv,
                                hipStream_t s) {
  const int n_tiles = (pr.T + kTileK - 1) / kTileK;
  const dim3 grid(n_tiles * pr.B * pr.H);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  const auto* gg = static_cast<const uint16_t*>(dout);
  if (pr.D == 64)
    hipLaunchKernelGGL(bwd_dkdv_mfma_kernel<64>, grid, dim3(64), 0, s, qq, kk, vv,
                       gg, lse, delta, pr, taps, n_tiles, dk, dv);
  else
    hipLaunchKernelGGL(bwd_dkdv_mfma_kernel<128>, grid, dim3(64), 0, s, qq, kk, vv,
                       gg, lse, delta, pr, taps, n_tiles, dk, dv);
  return hipGetLastError();
}

}  // namespace fsa
