// Decoding step of Fibonacci-spaced sparse attention: one new query per
// (batch, head) against the cached key and value rows of its slab.
//
// Method: Depth-Staggered Fibonacci Spacing for Sparse Attention (gist.science
// technical summary), Methodology > Architecture and attention (a query at
// position i attends the window rows i-W+1..i and the kept taps i - alpha*f_k,
// interpolating rows i - ceil(alpha*f_k) and the row after it). The page
// compares the latency of this step between learned and static spacing (Core
// contributions and results > 2. Learned dilation is inert, efficiency).
//
// Layout: q [B][H][D]; k_cache, v_cache [B][H][T_cap][D] (the training layout
// with T_cap rows per slab); pos [B] on the device. The step reads at most
// W + 2 * 15 rows per slab, so it is bound by memory latency, not bandwidth:
// every entry of the query is handed to its own group of 16 lanes (16 groups
// per workgroup), each group keeps an online softmax over its entries with the
// next entry's rows already in flight, and the groups are merged through LDS.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "fsa.h"
#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr int kDecBlock = 256;            // four wavefronts
constexpr int kGroups = kDecBlock / 16;   // entry groups of 16 lanes

// C consecutive elements of a row as fp32 (C = D / 16; one lane's share).
template <int C>
__device__ __forceinline__ void load_chunk(const uint16_t* p, float* r) {
  if constexpr (C == 4) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    r[0] = __uint_as_float(u.x << 16);
    r[1] = __uint_as_float(u.x & 0xffff0000u);
    r[2] = __uint_as_float(u.y << 16);
    r[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    static_assert(C == 8, "chunk of 4 or 8 elements");
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[2 * j] = __uint_as_float(w[j] << 16);
      r[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
}

template <int C>
__device__ __forceinline__ void load_chunk(const float* p, float* r) {
#pragma unroll
  for (int j = 0; j < C; j += 4) {
    const float4 a = *reinterpret_cast<const float4*>(p + j);
    r[j] = a.x;
    r[j + 1] = a.y;
    r[j + 2] = a.z;
    r[j + 3] = a.w;
  }
}

// Sum over the 16 lanes of a group, left in each of them.
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 8, 16);
  x += __shfl_xor(x, 4, 16);
  x += __shfl_xor(x, 2, 16);
  x += __shfl_xor(x, 1, 16);
  return x;
}

// The tap table in lanes: lane t (< kNumTaps) holds tap t's distance and
// weights (lanes past the table hold tap 0's), written with v_writelane so
// that no per-lane select turns into an indexed copy of the argument block.
struct TapLanes {
  int c;
  float wl, wh;
};

template <int L>
__device__ __forceinline__ void write_lane(int* x, int v) {
  asm("v_writelane_b32 %0, %1, %2" : "+v"(*x) : "s"(v), "n"(L));
}

template <int L>
__device__ __forceinline__ void fill_lanes(CTaps& taps, int* c, int* wl, int* wh) {
  if constexpr (L < kNumTaps) {
    write_lane<L>(c, taps.c[L]);
    write_lane<L>(wl, __float_as_int(taps.w_lo[L]));
    write_lane<L>(wh, __float_as_int(taps.w_hi[L]));
    fill_lanes<L + 1>(taps, c, wl, wh);
  }
}

__device__ __forceinline__ TapLanes tap_lanes(CTaps& taps) {
  int c = taps.c[0], wl = __float_as_int(taps.w_lo[0]), wh = __float_as_int(taps.w_hi[0]);
  fill_lanes<1>(taps, &c, &wl, &wh);
  return TapLanes{c, __int_as_float(wl), __int_as_float(wh)};
}

// Entry en of the query at position i: window entries first (row i - en),
// then the reaching taps in ascending distance (rows i - c and i - c + 1).
// Every lane of a 16-lane group asks for the same entry; the tap's values come
// from lane t < 15 of the wavefront (a lane shuffle). Those lanes belong to the
// wavefront's first group, which takes the lowest entries and so is active
// whenever any group of its wavefront is: the source lanes are always live.
struct Entry {
  int row;       // lower (or only) row
  float w0, w1;  // weights of row and row + 1 (w1 = 0 for a window entry)
};

__device__ __forceinline__ Entry entry_of(int en, int i, int nw, const TapLanes& tl) {
  const int t = max(en - nw, 0);
  const int c = __shfl(tl.c, t);
  const float wl = __shfl(tl.wl, t), wh = __shfl(tl.wh, t);
  if (en < nw) return Entry{i - en, 1.f, 0.f};
  return Entry{i - c, wl, wh};
}

// The lane's share of the K and V rows of an entry. An entry with no upper
// row (weight 0) reads its own row twice, so that every load is issued
// unconditionally and no row past the query is touched.
template <typename Tin, int C>
__device__ __forceinline__ void fetch(const Tin* K, const Tin* V, int D, const Entry& e,
                                      float* k0, float* v0, float* k1, float* v1) {
  const size_t r0 = static_cast<size_t>(e.row) * D;
  const size_t r1 = e.w1 != 0.f ? r0 + D : r0;
  load_chunk<C>(K + r0, k0);
  load_chunk<C>(V + r0, v0);
  load_chunk<C>(K + r1, k1);
  load_chunk<C>(V + r1, v1);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void put(float* o, float x) { *o = x; }
// bf16 bits, round to nearest even
__device__ __forceinline__ void put(uint16_t* o, float x) {
  *o = static_cast<uint16_t>(
      __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, 0.f}, bf16x2)));
}

template <typename Tin, int D, typename OutT>
__global__ __launch_bounds__(kDecBlock) void decode_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ kc,
    const Tin* __restrict__ vc, const int* __restrict__ pos, int H, int Tcap,
    int W, float c2, TapsArg taps_arg, OutT* __restrict__ out, float* __restrict__ lse) {
  CTaps& taps = taps_of(taps_arg);
  constexpr int C = D / 16;
  constexpr float kLn2 = 0.6931471805599453f;
  __shared__ float s_m[kGroups], s_l[kGroups];
  __shared__ __attribute__((aligned(16))) float s_acc[kGroups][D];
  const int tid = threadIdx.x;
  const int grp = tid >> 4, e = tid & 15;
  const int bh = blockIdx.x;
  const int i = pos[bh / H];
  OutT* o = out + static_cast<size_t>(bh) * D;
  if (i < 0 || i >= Tcap) {              // the same for the whole workgroup
    if (tid < D) put(o + tid, NAN);
    if (tid == 0) lse[bh] = NAN;
    return;
  }
  const TapLanes tl = tap_lanes(taps);
  const int lane = tid & 63;
  // taps sorted by distance: the reaching ones are a prefix
  const int ntap = __builtin_popcountll(
      __builtin_amdgcn_ballot_w64(lane < taps.n && tl.c <= i));
  const int nw = min(W, i + 1);
  const int ne = nw + ntap;

  float qv[C];
  load_chunk<C>(q + static_cast<size_t>(bh) * D + e * C, qv);
  const size_t slab = static_cast<size_t>(bh) * Tcap * D + e * C;
  const Tin* K = kc + slab;
  const Tin* V = vc + slab;

  float m = -INFINITY, l = 0.f;
  float acc[C];
#pragma unroll
  for (int j = 0; j < C; ++j) acc[j] = 0.f;
  float k0[C], v0[C], k1[C], v1[C];
  Entry cur{0, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < C; ++j) k0[j] = v0[j] = k1[j] = v1[j] = 0.f;
  int en = grp;
  if (en < ne) {
    cur = entry_of(en, i, nw, tl);
    fetch<Tin, C>(K, V, D, cur, k0, v0, k1, v1);
  }
  for (; en < ne; en += kGroups) {
    // next entry's rows in flight while this one is reduced
    const int nx = en + kGroups;
    Entry nxt{0, 0.f, 0.f};
    float nk0[C], nv0[C], nk1[C], nv1[C];
    if (nx < ne) {
      nxt = entry_of(nx, i, nw, tl);
      fetch<Tin, C>(K, V, D, nxt, nk0, nv0, nk1, nv1);
    } else {
#pragma unroll
      for (int j = 0; j < C; ++j) nk0[j] = nv0[j] = nk1[j] = nv1[j] = 0.f;
    }
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      s0 = fmaf(qv[j], k0[j], s0);
      s1 = fmaf(qv[j], k1[j], s1);
    }
    const float s = sum16(fmaf(cur.w1, s1, cur.w0 * s0)) * c2;
    const float mn = fmaxf(m, s);
    const float corr = exp2f(m - mn);    // 0 on the first entry
    const float p = exp2f(s - mn);
    l = l * corr + p;
    m = mn;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const float val = fmaf(cur.w1, v1[j], cur.w0 * v0[j]);
      acc[j] = fmaf(p, val, acc[j] * corr);
    }
    cur = nxt;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      k0[j] = nk0[j];
      v0[j] = nv0[j];
      k1[j] = nk1[j];
      v1[j] = nv1[j];
    }
  }

  // merge the groups: out = sum_g acc_g 2^(m_g - M) / sum_g l_g 2^(m_g - M)
  if (e == 0) {
    s_m[grp] = m;
    s_l[grp] = l;
  }
#pragma unroll
  for (int j = 0; j < C; ++j) s_acc[grp][e * C + j] = acc[j];
  __syncthreads();
  if (tid < D) {
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) M = fmaxf(M, s_m[g]);
    float L = 0.f, od = 0.f;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const float f = exp2f(s_m[g] - M);  // 0 for a group with no entry
      L = fmaf(s_l[g], f, L);
      od = fmaf(s_acc[g][tid], f, od);
    }
    put(o + tid, od / L);
    if (tid == 0) lse[bh] = (M + log2f(L)) * kLn2;
  }
}

template <typename Tin, int D>
hipError_t decode_typed(const void* q, const void* k, const void* v,
                        const int* pos, int B, int H, int Tcap, int W,
                        const TapsArg& taps, void* out, bool out_bf16, float* lse,
                        hipStream_t s) {
  const float c2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(D)));
  if (out_bf16)
    hipLaunchKernelGGL((decode_kernel<Tin, D, uint16_t>), dim3(B * H), dim3(kDecBlock), 0, s,
                       static_cast<const Tin*>(q), static_cast<const Tin*>(k),
                       static_cast<const Tin*>(v), pos, H, Tcap, W, c2, taps,
                       static_cast<uint16_t*>(out), lse);
  else
    hipLaunchKernelGGL((decode_kernel<Tin, D, float>), dim3(B * H), dim3(kDecBlock), 0, s,
                       static_cast<const Tin*>(q), static_cast<const Tin*>(k),
                       static_cast<const Tin*>(v), pos, H, Tcap, W, c2, taps,
                       static_cast<float*>(out), lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const void* q, const void* k, const void* v, int dtype,
                         const int* pos, int B, int H, int Tcap, int D, int W,
                         const TapsArg& taps, void* out, bool out_bf16, float* lse,
                         hipStream_t s) {
  if (dtype == FSA_DTYPE_F32)
    return D == 64 ? decode_typed<float, 64>(q, k, v, pos, B, H, Tcap, W, taps, out, out_bf16, lse, s)
                   : decode_typed<float, 128>(q, k, v, pos, B, H, Tcap, W, taps, out, out_bf16, lse, s);
  return D == 64 ? decode_typed<uint16_t, 64>(q, k, v, pos, B, H, Tcap, W, taps, out, out_bf16, lse, s)
                 : decode_typed<uint16_t, 128>(q, k, v, pos, B, H, Tcap, W, taps, out, out_bf16, lse, s);
}

}  // namespace fsa
