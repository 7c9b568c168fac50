// Lane-per-row kernels of Fibonacci-spaced sparse attention.
//
// Each lane owns one query (forward, dq pass) or one key row (dk/dv pass) and
// walks that row's attended entries with fp32 arithmetic. These kernels serve
// the fp32 inputs; they read rows straight from global memory (L1/L2 cached).
//
// Method: Depth-Staggered Fibonacci Spacing for Sparse Attention (gist.science
// technical summary), Methodology > Architecture and attention: the attended
// set (window of W keys plus Fibonacci taps), the per-layer scale alpha of the
// tap distances, and linear interpolation of key and value rows at fractional
// distances, which gives the gradient with respect to alpha.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fsa.h"
#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr int kVecBlock = 64;  // one wavefront per workgroup

// ---- result rows: fp32, or bf16 rounded to nearest even --------------------
template <int D>
__device__ __forceinline__ void store_row(float* o, const float* acc) {
#pragma unroll
  for (int d = 0; d < D; d += 4)
    *reinterpret_cast<float4*>(o + d) = make_float4(acc[d], acc[d + 1], acc[d + 2], acc[d + 3]);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int D>
__device__ __forceinline__ void store_row(uint16_t* o, const float* acc) {
#pragma unroll
  for (int d = 0; d < D; d += 8) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                              f32x2{acc[d + 2 * e], acc[d + 2 * e + 1]}, bf16x2));
    *reinterpret_cast<uint4*>(o + d) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---- row access, converted to fp32 ----------------------------------------
__device__ __forceinline__ void load8(const float* p, float* r) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
}

__device__ __forceinline__ void load8(const uint16_t* p, float* r) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = __uint_as_float(w[i] << 16);
    r[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <typename Tin, int D>
__device__ __forceinline__ void load_row(const Tin* p, float* r) {
#pragma unroll
  for (int d = 0; d < D; d += 8) load8(p + d, r + d);
}

// x . row, the row streamed from memory
template <typename Tin, int D>
__device__ __forceinline__ float dot_row(const float* x, const Tin* p) {
  float acc = 0.f;
#pragma unroll
  for (int d = 0; d < D; d += 8) {
    float r[8];
    load8(p + d, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(x[d + e], r[e], acc);
  }
  return acc;
}

// acc += a * row
template <typename Tin, int D>
__device__ __forceinline__ void axpy_row(float a, const Tin* p, float* acc) {
#pragma unroll
  for (int d = 0; d < D; d += 8) {
    float r[8];
    load8(p + d, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[d + e] = fmaf(a, r[e], acc[d + e]);
  }
}

// ---- forward ---------------------------------------------------------------
// out_i = sum_e softmax(s)_e * value_e over the window entries j = i-w
// (w < W, j >= 0) and the kept taps with i >= c (rows a = i-c, a+1).
template <typename Tin, int D, typename OutT>
__global__ __launch_bounds__(kVecBlock) void fwd_vec_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, Problem pr, TapsArg taps_arg, OutT* __restrict__ out,
    float* __restrict__ lse) {
  CTaps& taps = taps_of(taps_arg);
  const int i = blockIdx.x * kVecBlock + threadIdx.x;
  const int T = pr.T;
  if (i >= T) return;
  const size_t base = static_cast<size_t>(blockIdx.y) * T * D;
  const Tin* K = k + base;
  const Tin* V = v + base;
  float qr[D];
  load_row<Tin, D>(q + base + static_cast<size_t>(i) * D, qr);
#pragma unroll
  for (int d = 0; d < D; ++d) qr[d] *= pr.scale;

  // pass 1: running max and denominator
  float m = -INFINITY, l = 0.f;
  const int wn = min(pr.W, i + 1);
  for (int w = 0; w < wn; ++w) {
    const float s = dot_row<Tin, D>(qr, K + static_cast<size_t>(i - w) * D);
    if (s > m) { l = l * expf(m - s) + 1.f; m = s; } else { l += expf(s - m); }
  }
  for (int n = 0; n < taps.n; ++n) {
    const int c = taps.c[n];
    if (i < c) break;
    const Tin* ka = K + static_cast<size_t>(i - c) * D;
    float s = taps.w_lo[n] * dot_row<Tin, D>(qr, ka);
    if (taps.w_hi[n] != 0.f) s += taps.w_hi[n] * dot_row<Tin, D>(qr, ka + D);
    if (s > m) { l = l * expf(m - s) + 1.f; m = s; } else { l += expf(s - m); }
  }
  const float L = m + logf(l);

  // pass 2: weighted values
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  for (int w = 0; w < wn; ++w) {
    const size_t j = static_cast<size_t>(i - w) * D;
    const float p = expf(dot_row<Tin, D>(qr, K + j) - L);
    axpy_row<Tin, D>(p, V + j, acc);
  }
  for (int n = 0; n < taps.n; ++n) {
    const int c = taps.c[n];
    if (i < c) break;
    const size_t a = static_cast<size_t>(i - c) * D;
    const float wl = taps.w_lo[n], wh = taps.w_hi[n];
    float s = wl * dot_row<Tin, D>(qr, K + a);
    if (wh != 0.f) s += wh * dot_row<Tin, D>(qr, K + a + D);
    const float p = expf(s - L);
    axpy_row<Tin, D>(p * wl, V + a, acc);
    if (wh != 0.f) axpy_row<Tin, D>(p * wh, V + a + D, acc);
  }
  store_row<D>(out + base + static_cast<size_t>(i) * D, acc);
  lse[static_cast<size_t>(blockIdx.y) * T + i] = L;
}

// ---- backward, query side --------------------------------------------------
// Delta_i = sum_e p_e dP_e, dS_e = p_e (dP_e - Delta_i), dq_i = scale sum_e
// dS_e key_e, and the alpha gradient of every tap entry:
//   -f * [dS (s_hi - s_lo) + p (dP_hi - dP_lo)],
// s_lo/s_hi the scaled scores against rows a and a+1, dP_lo/dP_hi the dout
// products with rows a and a+1. One partial per workgroup.
template <typename Tin, int D>
__global__ __launch_bounds__(kVecBlock) void bwd_dq_vec_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ dout,
    const float* __restrict__ lse, Problem pr, TapsArg taps_arg,
    float* __restrict__ dq, float* __restrict__ delta,
    float* __restrict__ partials) {
  CTaps& taps = taps_of(taps_arg);
  const int i = blockIdx.x * kVecBlock + threadIdx.x;
  const int T = pr.T;
  float dal = 0.f;
  if (i < T) {
    const size_t base = static_cast<size_t>(blockIdx.y) * T * D;
    const Tin* K = k + base;
    const Tin* V = v + base;
    float qr[D], gr[D];
    load_row<Tin, D>(q + base + static_cast<size_t>(i) * D, qr);
    load_row<Tin, D>(dout + base + static_cast<size_t>(i) * D, gr);
#pragma unroll
    for (int d = 0; d < D; ++d) qr[d] *= pr.scale;
    const float L = lse[static_cast<size_t>(blockIdx.y) * T + i];
    const int wn = min(pr.W, i + 1);

    float Dsum = 0.f;
    for (int w = 0; w < wn; ++w) {
      const size_t j = static_cast<size_t>(i - w) * D;
      const float p = expf(dot_row<Tin, D>(qr, K + j) - L);
      Dsum += p * dot_row<Tin, D>(gr, V + j);
    }
    for (int n = 0; n < taps.n; ++n) {
      const int c = taps.c[n];
      if (i < c) break;
      const size_t a = static_cast<size_t>(i - c) * D;
      const float wl = taps.w_lo[n], wh = taps.w_hi[n];
      const float s = wl * dot_row<Tin, D>(qr, K + a) + wh * dot_row<Tin, D>(qr, K + a + D);
      const float dp = wl * dot_row<Tin, D>(gr, V + a) + wh * dot_row<Tin, D>(gr, V + a + D);
      Dsum += expf(s - L) * dp;
    }

    float acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = 0.f;
    for (int w = 0; w < wn; ++w) {
      const size_t j = static_cast<size_t>(i - w) * D;
      const float p = expf(dot_row<Tin, D>(qr, K + j) - L);
      const float ds = p * (dot_row<Tin, D>(gr, V + j) - Dsum);
      axpy_row<Tin, D>(ds, K + j, acc);
    }
    for (int n = 0; n < taps.n; ++n) {
      const int c = taps.c[n];
      if (i < c) break;
      const size_t a = static_cast<size_t>(i - c) * D;
      const float wl = taps.w_lo[n], wh = taps.w_hi[n];
      const float s_lo = dot_row<Tin, D>(qr, K + a);
      const float s_hi = dot_row<Tin, D>(qr, K + a + D);
      const float g_lo = dot_row<Tin, D>(gr, V + a);
      const float g_hi = dot_row<Tin, D>(gr, V + a + D);
      const float p = expf(wl * s_lo + wh * s_hi - L);
      const float ds = p * (wl * g_lo + wh * g_hi - Dsum);
      axpy_row<Tin, D>(ds * wl, K + a, acc);
      axpy_row<Tin, D>(ds * wh, K + a + D, acc);
      dal += taps.neg_f[n] * (ds * (s_hi - s_lo) + p * (g_hi - g_lo));
    }
    float* o = dq + base + static_cast<size_t>(i) * D;
#pragma unroll
    for (int d = 0; d < D; d += 4)
      *reinterpret_cast<float4*>(o + d) =
          make_float4(acc[d] * pr.scale, acc[d + 1] * pr.scale,
                      acc[d + 2] * pr.scale, acc[d + 3] * pr.scale);
    delta[static_cast<size_t>(blockIdx.y) * T + i] = Dsum;
  }
  // fixed-order wavefront reduction of the alpha gradient
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) dal += __shfl_xor(dal, off);
  if (threadIdx.x == 0)
    partials[static_cast<size_t>(blockIdx.y) * gridDim.x + blockIdx.x] = dal;
}

// ---- backward, key side ----------------------------------------------------
// Row j collects the gradient of every entry that gathered it: window queries
// i = j + w; tap queries i = j + c (row j is the lower row, weight 1 - t) and
// i = j + c - 1 (row j is the upper row, weight t, needs j >= 1).
template <typename Tin, int D>
__global__ __launch_bounds__(kVecBlock) void bwd_dkdv_vec_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, Problem pr,
    TapsArg taps_arg, float* __restrict__ dk, float* __restrict__ dv) {
  CTaps& taps = taps_of(taps_arg);
  const int j = blockIdx.x * kVecBlock + threadIdx.x;
  const int T = pr.T;
  if (j >= T) return;
  const size_t base = static_cast<size_t>(blockIdx.y) * T * D;
  const size_t rbase = static_cast<size_t>(blockIdx.y) * T;
  const Tin* Q = q + base;
  const Tin* K = k + base;
  const Tin* V = v + base;
  const Tin* G = dout + base;
  float kr[D], vr[D];
  load_row<Tin, D>(K + static_cast<size_t>(j) * D, kr);
  load_row<Tin, D>(V + static_cast<size_t>(j) * D, vr);
  float gk[D], gv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { gk[d] = 0.f; gv[d] = 0.f; }

  for (int w = 0; w < pr.W; ++w) {
    const int i = j + w;
    if (i >= T) break;
    const size_t qi = static_cast<size_t>(i) * D;
    const float p = expf(pr.scale * dot_row<Tin, D>(kr, Q + qi) - lse[rbase + i]);
    const float ds = p * (dot_row<Tin, D>(vr, G + qi) - delta[rbase + i]);
    axpy_row<Tin, D>(ds * pr.scale, Q + qi, gk);
    axpy_row<Tin, D>(p, G + qi, gv);
  }
  for (int n = 0; n < taps.n; ++n) {
    const int c = taps.c[n];
    const float wl = taps.w_lo[n], wh = taps.w_hi[n];
    // row j as the lower row of query i = j + c
    {
      const int i = j + c;
      if (i < T) {
        const size_t qi = static_cast<size_t>(i) * D;
        const Tin* up = K + static_cast<size_t>(j + 1) * D;
        const Tin* upv = V + static_cast<size_t>(j + 1) * D;
        float s = wl * dot_row<Tin, D>(kr, Q + qi);
        float g = wl * dot_row<Tin, D>(vr, G + qi);
        if (wh != 0.f) {
          float qq[D];
          load_row<Tin, D>(Q + qi, qq);
          s += wh * dot_row<Tin, D>(qq, up);
          float gg[D];
          load_row<Tin, D>(G + qi, gg);
          g += wh * dot_row<Tin, D>(gg, upv);
        }
        const float p = expf(pr.scale * s - lse[rbase + i]);
        const float ds = p * (g - delta[rbase + i]);
        axpy_row<Tin, D>(ds * wl * pr.scale, Q + qi, gk);
        axpy_row<Tin, D>(p * wl, G + qi, gv);
      }
    }
    // row j as the upper row of query i = j + c - 1 (lower row j - 1)
    if (wh != 0.f && j >= 1) {
      const int i = j + c - 1;
      if (i < T) {
        const size_t qi = static_cast<size_t>(i) * D;
        const Tin* lo = K + static_cast<size_t>(j - 1) * D;
        const Tin* lov = V + static_cast<size_t>(j - 1) * D;
        float qq[D], gg[D];
        load_row<Tin, D>(Q + qi, qq);
        load_row<Tin, D>(G + qi, gg);
        const float s = wl * dot_row<Tin, D>(qq, lo) + wh * dot_row<Tin, D>(kr, Q + qi);
        const float g = wl * dot_row<Tin, D>(gg, lov) + wh * dot_row<Tin, D>(vr, G + qi);
        const float p = expf(pr.scale * s - lse[rbase + i]);
        const float ds = p * (g - delta[rbase + i]);
        axpy_row<Tin, D>(ds * wh * pr.scale, Q + qi, gk);
        axpy_row<Tin, D>(p * wh, G + qi, gv);
      }
    }
  }
  float* ok = dk + base + static_cast<size_t>(j) * D;
  float* ov = dv + base + static_cast<size_t>(j) * D;
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    *reinterpret_cast<float4*>(ok + d) = make_float4(gk[d], gk[d + 1], gk[d + 2], gk[d + 3]);
    *reinterpret_cast<float4*>(ov + d) = make_float4(gv[d], gv[d + 1], gv[d + 2], gv[d + 3]);
  }
}

}  // namespace

// ---- dalpha: deterministic sum of the per-tile partials ---------------------
__global__ __launch_bounds__(256) void dalpha_reduce_kernel(
    const float* __restrict__ partials, size_t n, float* __restrict__ dalpha) {
  __shared__ double sh[256];
  double acc = 0.0;
  for (size_t x = threadIdx.x; x < n; x += 256) acc += partials[x];
  sh[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) dalpha[0] = static_cast<float>(sh[0]);
}

hipError_t launch_dalpha_reduce(const float* partials, size_t n, float* dalpha,
                                hipStream_t s) {
  hipLaunchKernelGGL(dalpha_reduce_kernel, dim3(1), dim3(256), 0, s, partials,
                     n, dalpha);
  return hipGetLastError();
}

namespace {
template <typename Tin, int D>
hipError_t fwd_vec_typed(const void* q, const void* k, const void* v,
                         const Problem& pr, const TapsArg& taps, void* out,
                         bool out_bf16, float* lse, hipStream_t s) {
  dim3 grid((pr.T + kVecBlock - 1) / kVecBlock, pr.B * pr.H);
  if (out_bf16)
    hipLaunchKernelGGL((fwd_vec_kernel<Tin, D, uint16_t>), grid, dim3(kVecBlock), 0, s,
                       static_cast<const Tin*>(q), static_cast<const Tin*>(k),
                       static_cast<const Tin*>(v), pr, taps, static_cast<uint16_t*>(out), lse);
  else
    hipLaunchKernelGGL((fwd_vec_kernel<Tin, D, float>), grid, dim3(kVecBlock), 0, s,
                       static_cast<const Tin*>(q), static_cast<const Tin*>(k),
                       static_cast<const Tin*>(v), pr, taps, static_cast<float*>(out), lse);
  return hipGetLastError();
}

template <typename Tin, int D>
hipError_t bwd_dq_vec_typed(const void* q, const void* k, const void* v,
                            const void* dout, const float* lse,
                            const Problem& pr, const TapsArg& taps, float* dq,
                            float* delta, float* partials, hipStream_t s) {
  dim3 grid((pr.T + kVecBlock - 1) / kVecBlock, pr.B * pr.H);
  hipLaunchKernelGGL((bwd_dq_vec_kernel<Tin, D>), grid, dim3(kVecBlock), 0, s,
                     static_cast<const Tin*>(q), static_cast<const Tin*>(k),
                     static_cast<const Tin*>(v), static_cast<const Tin*>(dout),
                     lse, pr, taps, dq, delta, partials);
  return hipGetLastError();
}

template <typename Tin, int D>
hipError_t bwd_dkdv_vec_typed(const void* q, const void* k, const void* v,
                              const void* dout, const float* lse,
                              const float* delta, const Problem& pr,
                              const TapsArg& taps, float* dk, float* dv,
                              hipStream_t s) {
  dim3 grid((pr.T + kVecBlock - 1) / kVecBlock, pr.B * pr.H);
  hipLaunchKernelGGL((bwd_dkdv_vec_kernel<Tin, D>), grid, dim3(kVecBlock), 0, s,
                     static_cast<const Tin*>(q), static_cast<const Tin*>(k),
                     static_cast<const Tin*>(v), static_cast<const Tin*>(dout),
                     lse, delta, pr, taps, dk, dv);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fwd_vec(const void* q, const void* k, const void* v,
                          int dtype, const Problem& pr, const TapsArg& taps,
                          void* out, bool out_bf16, float* lse, hipStream_t s) {
  if (dtype == FSA_DTYPE_F32) {
    return pr.D == 64 ? fwd_vec_typed<float, 64>(q, k, v, pr, taps, out, out_bf16, lse, s)
                      : fwd_vec_typed<float, 128>(q, k, v, pr, taps, out, out_bf16, lse, s);
  }
  return pr.D == 64 ? fwd_vec_typed<uint16_t, 64>(q, k, v, pr, taps, out, out_bf16, lse, s)
                    : fwd_vec_typed<uint16_t, 128>(q, k, v, pr, taps, out, out_bf16, lse, s);
}

size_t bwd_partials_used_vec(const Problem& pr) {
  return static_cast<size_t>((pr.T + kVecBlock - 1) / kVecBlock) * pr.B * pr.H;
}

hipError_t launch_bwd_dq_vec(const void* q, const void* k, const void* v,
                             const void* dout, const float* lse, int dtype,
                             const Problem& pr, const TapsArg& taps, float* dq,
                             float* delta, float* partials, hipStream_t s) {
  if (dtype == FSA_DTYPE_F32)
    return pr.D == 64 ? bwd_dq_vec_typed<float, 64>(q, k, v, dout, lse, pr, taps, dq, delta, partials, s)
                      : bwd_dq_vec_typed<float, 128>(q, k, v, dout, lse, pr, taps, dq, delta, partials, s);
  return pr.D == 64 ? bwd_dq_vec_typed<uint16_t, 64>(q, k, v, dout, lse, pr, taps, dq, delta, partials, s)
                    : bwd_dq_vec_typed<uint16_t, 128>(q, k, v, dout, lse, pr, taps, dq, delta, partials, s);
}

hipError_t launch_bwd_dkdv_vec(const void* q, const void* k, const void* v,
                               const void* dout, const float* lse,
                               const float* delta, int dtype,
                               const Problem& pr, const TapsArg& taps, float* dk,
                               float* dv, hipStream_t s) {
  if (dtype == FSA_DTYPE_F32)
    return pr.D == 64 ? bwd_dkdv_vec_typed<float, 64>(q, k, v, dout, lse, delta, pr, taps, dk, dv, s)
                      : bwd_dkdv_vec_typed<float, 128>(q, k, v, dout, lse, delta, pr, taps, dk, dv, s);
  return pr.D == 64 ? bwd_dkdv_vec_typed<uint16_t, 64>(q, k, v, dout, lse, delta, pr, taps, dk, dv, s)
                    : bwd_dkdv_vec_typed<uint16_t, 128>(q, k, v, dout, lse, delta, pr, taps, dk, dv, s);
}

}  // namespace fsa
