// Row-group kernels of Fibonacci-spaced sparse attention (fp32 inputs).
//
// Eight lanes share one query (forward, dq pass) or one key row (dk/dv pass);
// a wavefront owns eight consecutive rows. Lane e of a group holds the
// elements 32c + 4e .. 32c + 4e + 3 of a row (c < D/32), so one load
// instruction reads 128 contiguous bytes of each of the eight rows (a whole
// fp32 row of D = 64 in two instructions). A dot product is four FMAs per
// chunk per lane and a sum over the group's eight lanes (DPP). Rows are read
// straight from global memory (L1/L2 cached): consecutive rows of a
// wavefront read overlapping rows, which the L1 serves. Every entry is taken
// once, with an online softmax (forward) or with the two sums
// sum p dP key and sum p key that Delta combines at the end (dq).
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

constexpr int kVecBlock = 64;      // one wavefront per workgroup
constexpr int kGroup = 8;          // lanes per row
constexpr int kRowsPerWave = kVecBlock / kGroup;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---- row parts, converted to fp32 ------------------------------------------
__device__ __forceinline__ void load4(const float* p, float* r) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
}

__device__ __forceinline__ void load4(const uint16_t* p, float* r) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  r[0] = __uint_as_float(u.x << 16);
  r[1] = __uint_as_float(u.x & 0xffff0000u);
  r[2] = __uint_as_float(u.y << 16);
  r[3] = __uint_as_float(u.y & 0xffff0000u);
}

// The lane's part of a row: elements 32c + 4e .. + 3, c < D/32.
template <typename Tin, int D>
__device__ __forceinline__ void load_part(const Tin* row, int e, float* r) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c) load4(row + 32 * c + 4 * e, r + 4 * c);
}

// Sum over the eight lanes of a group, left in each of them: two quad swaps
// and the half-row mirror.
template <int Ctrl>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xf, 0xf, false));
}
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f<0xB1>(x);             // quad_perm(1, 0, 3, 2)
  x += dpp_f<0x4E>(x);             // quad_perm(2, 3, 0, 1)
  x += dpp_f<0x141>(x);            // row_half_mirror
  return x;
}

// x . row over the group (x: the lane's part)
template <typename Tin, int D>
__device__ __forceinline__ float dot_row(const float* x, const Tin* row, int e) {
  float r[D / 8];
  load_part<Tin, D>(row, e, r);
  float acc = 0.f;
#pragma unroll
  for (int d = 0; d < D / 8; ++d) acc = fmaf(x[d], r[d], acc);
  return group_sum(acc);
}

// acc += a * row (the lane's part)
template <typename Tin, int D>
__device__ __forceinline__ void axpy_row(float a, const Tin* row, int e, float* acc) {
  float r[D / 8];
  load_part<Tin, D>(row, e, r);
#pragma unroll
  for (int d = 0; d < D / 8; ++d) acc[d] = fmaf(a, r[d], acc[d]);
}

template <int D>
__device__ __forceinline__ void store_part(float* row, int e, const float* x) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    *reinterpret_cast<float4*>(row + 32 * c + 4 * e) =
        make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
}

template <int D>
__device__ __forceinline__ void store_part(uint16_t* row, int e, const float* x) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[4 * c], x[4 * c + 1]}, bf16x2));
    const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[4 * c + 2], x[4 * c + 3]}, bf16x2));
    *reinterpret_cast<uint2*>(row + 32 * c + 4 * e) = make_uint2(w0, w1);
  }
}

// ---- forward ---------------------------------------------------------------
// out_i = sum_e softmax(s)_e * value_e over the window entries j = i-w
// (w < W, j >= 0) and the kept taps with i >= c (rows a = i-c, a+1), one pass
// with a running max: each entry rescales the sum and the accumulator.
template <typename Tin, int D, typename OutT>
__global__ __launch_bounds__(kVecBlock) void fwd_vec_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, Problem pr, TapsArg taps_arg, OutT* __restrict__ out,
    float* __restrict__ lse) {
  CTaps& taps = taps_of(taps_arg);
  const int e = threadIdx.x % kGroup;
  const int i = blockIdx.x * kRowsPerWave + threadIdx.x / kGroup;
  const int T = pr.T;
  if (i >= T) return;                       // whole groups leave together
  const size_t base = static_cast<size_t>(blockIdx.y) * T * D;
  const Tin* K = k + base;
  const Tin* V = v + base;
  float qr[D / 8];
  load_part<Tin, D>(q + base + static_cast<size_t>(i) * D, e, qr);
#pragma unroll
  for (int d = 0; d < D / 8; ++d) qr[d] *= pr.scale;

  float m = -INFINITY, l = 0.f;
  float acc[D / 8];
#pragma unroll
  for (int d = 0; d < D / 8; ++d) acc[d] = 0.f;
  // one entry of score s whose value is wl V[a] (+ wh V[a+1])
  auto take = [&](float s, size_t a, float wl, float wh) {
    const float mn = fmaxf(m, s);
    const float corr = expf(m - mn);
    const float p = expf(s - mn);
    l = l * corr + p;
    m = mn;
#pragma unroll
    for (int d = 0; d < D / 8; ++d) acc[d] *= corr;
    axpy_row<Tin, D>(p * wl, V + a, e, acc);
    if (wh != 0.f) axpy_row<Tin, D>(p * wh, V + a + D, e, acc);
  };
  const int wn = min(pr.W, i + 1);
  for (int w = 0; w < wn; ++w) {
    const size_t j = static_cast<size_t>(i - w) * D;
    take(dot_row<Tin, D>(qr, K + j, e), j, 1.f, 0.f);
  }
  for (int n = 0; n < taps.n; ++n) {
    const int c = taps.c[n];
    if (i < c) break;
    const size_t a = static_cast<size_t>(i - c) * D;
    const float wl = taps.w_lo[n], wh = taps.w_hi[n];
    float s = wl * dot_row<Tin, D>(qr, K + a, e);
    if (wh != 0.f) s += wh * dot_row<Tin, D>(qr, K + a + D, e);
    take(s, a, wl, wh);
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < D / 8; ++d) acc[d] *= inv;
  store_part<D>(out + base + static_cast<size_t>(i) * D, e, acc);
  if (e == 0) lse[static_cast<size_t>(blockIdx.y) * T + i] = m + logf(l);
}

// ---- backward, query side --------------------------------------------------
// Delta_i = sum_e p_e dP_e, dS_e = p_e (dP_e - Delta_i), dq_i = scale sum_e
// dS_e key_e = scale (sum_e p_e dP_e key_e - Delta_i sum_e p_e key_e), and
// the alpha gradient of every tap entry,
//   -f * [dS (s_hi - s_lo) + p (dP_hi - dP_lo)]
//   = -f * p * [dP (s_hi - s_lo) + (dP_hi - dP_lo)] - Delta_i * (-f * p * (s_hi - s_lo)),
// s_lo/s_hi the scaled scores against rows a and a+1, dP_lo/dP_hi the dout
// products with rows a and a+1: one pass over the entries. One partial per
// workgroup (eight query rows).
template <typename Tin, int D>
__global__ __launch_bounds__(kVecBlock) void bwd_dq_vec_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ dout,
    const float* __restrict__ lse, Problem pr, TapsArg taps_arg,
    float* __restrict__ dq, float* __restrict__ delta,
    float* __restrict__ partials) {
  CTaps& taps = taps_of(taps_arg);
  const int e = threadIdx.x % kGroup;
  const int i = blockIdx.x * kRowsPerWave + threadIdx.x / kGroup;
  const int T = pr.T;
  float dal = 0.f;
  if (i < T) {
    const size_t base = static_cast<size_t>(blockIdx.y) * T * D;
    const Tin* K = k + base;
    const Tin* V = v + base;
    float qr[D / 8], gr[D / 8];
    load_part<Tin, D>(q + base + static_cast<size_t>(i) * D, e, qr);
    load_part<Tin, D>(dout + base + static_cast<size_t>(i) * D, e, gr);
#pragma unroll
    for (int d = 0; d < D / 8; ++d) qr[d] *= pr.scale;
    const float L = lse[static_cast<size_t>(blockIdx.y) * T + i];
    float a1[D / 8], a2[D / 8];
#pragma unroll
    for (int d = 0; d < D / 8; ++d) { a1[d] = 0.f; a2[d] = 0.f; }
    float Dsum = 0.f, al_a = 0.f, al_b = 0.f;
    const int wn = min(pr.W, i + 1);
    for (int w = 0; w < wn; ++w) {
      const size_t j = static_cast<size_t>(i - w) * D;
      const float p = expf(dot_row<Tin, D>(qr, K + j, e) - L);
      const float dp = dot_row<Tin, D>(gr, V + j, e);
      Dsum += p * dp;
      axpy_row<Tin, D>(p * dp, K + j, e, a1);
      axpy_row<Tin, D>(p, K + j, e, a2);
    }
    for (int n = 0; n < taps.n; ++n) {
      const int c = taps.c[n];
      if (i < c) break;
      const size_t a = static_cast<size_t>(i - c) * D;
      const float wl = taps.w_lo[n], wh = taps.w_hi[n];
      const float s_lo = dot_row<Tin, D>(qr, K + a, e);
      const float s_hi = dot_row<Tin, D>(qr, K + a + D, e);
      const float g_lo = dot_row<Tin, D>(gr, V + a, e);
      const float g_hi = dot_row<Tin, D>(gr, V + a + D, e);
      const float p = expf(wl * s_lo + wh * s_hi - L);
      const float dp = wl * g_lo + wh * g_hi;
      Dsum += p * dp;
      axpy_row<Tin, D>(p * dp * wl, K + a, e, a1);
      axpy_row<Tin, D>(p * wl, K + a, e, a2);
      if (wh != 0.f) {
        axpy_row<Tin, D>(p * dp * wh, K + a + D, e, a1);
        axpy_row<Tin, D>(p * wh, K + a + D, e, a2);
      }
      const float nf = taps.neg_f[n];
      al_a += nf * p * (dp * (s_hi - s_lo) + (g_hi - g_lo));
      al_b += nf * p * (s_hi - s_lo);
    }
    float o[D / 8];
#pragma unroll
    for (int d = 0; d < D / 8; ++d) o[d] = pr.scale * (a1[d] - Dsum * a2[d]);
    store_part<D>(dq + base + static_cast<size_t>(i) * D, e, o);
    if (e == 0) {
      delta[static_cast<size_t>(blockIdx.y) * T + i] = Dsum;
      dal = al_a - Dsum * al_b;                 // one lane of the group contributes
    }
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
// i = j + c - 1 (row j is the upper row, weight t, needs j >= 1). The group
// holds rows j - 1, j and j + 1 of K and V (the other row of a tap entry).
template <typename Tin, int D>
__global__ __launch_bounds__(kVecBlock) void bwd_dkdv_vec_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k,
    const Tin* __restrict__ v, const Tin* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, Problem pr,
    TapsArg taps_arg, float* __restrict__ dk, float* __restrict__ dv) {
  CTaps& taps = taps_of(taps_arg);
  const int e = threadIdx.x % kGroup;
  const int j = blockIdx.x * kRowsPerWave + threadIdx.x / kGroup;
  const int T = pr.T;
  if (j >= T) return;
  const size_t base = static_cast<size_t>(blockIdx.y) * T * D;
  const size_t rbase = static_cast<size_t>(blockIdx.y) * T;
  const Tin* Q = q + base;
  const Tin* K = k + base;
  const Tin* V = v + base;
  const Tin* G = dout + base;
  float kr[D / 8], vr[D / 8], kn[D / 8], vn[D / 8], kp[D / 8], vp[D / 8];
  load_part<Tin, D>(K + static_cast<size_t>(j) * D, e, kr);
  load_part<Tin, D>(V + static_cast<size_t>(j) * D, e, vr);
  // neighbouring rows, clamped into the slab (used only where they exist)
  const size_t jn = static_cast<size_t>(min(j + 1, T - 1)) * D;
  const size_t jp = static_cast<size_t>(max(j - 1, 0)) * D;
  load_part<Tin, D>(K + jn, e, kn);
  load_part<Tin, D>(V + jn, e, vn);
  load_part<Tin, D>(K + jp, e, kp);
  load_part<Tin, D>(V + jp, e, vp);
  float gk[D / 8], gv[D / 8];
#pragma unroll
  for (int d = 0; d < D / 8; ++d) { gk[d] = 0.f; gv[d] = 0.f; }
  const float sc = pr.scale;

  for (int w = 0; w < pr.W; ++w) {
    const int i = j + w;
    if (i >= T) break;
    const size_t qi = static_cast<size_t>(i) * D;
    float qq[D / 8], gg[D / 8];
    load_part<Tin, D>(Q + qi, e, qq);
    load_part<Tin, D>(G + qi, e, gg);
    float s = 0.f, g = 0.f;
#pragma unroll
    for (int d = 0; d < D / 8; ++d) { s = fmaf(kr[d], qq[d], s); g = fmaf(vr[d], gg[d], g); }
    s = group_sum(s);
    g = group_sum(g);
    const float p = expf(sc * s - lse[rbase + i]);
    const float ds = p * (g - delta[rbase + i]);
#pragma unroll
    for (int d = 0; d < D / 8; ++d) {
      gk[d] = fmaf(ds * sc, qq[d], gk[d]);
      gv[d] = fmaf(p, gg[d], gv[d]);
    }
  }
  for (int n = 0; n < taps.n; ++n) {
    const int c = taps.c[n];
    const float wl = taps.w_lo[n], wh = taps.w_hi[n];
    // row j as the lower row of query i = j + c, and as the upper row of
    // query j + c - 1 (lower row j - 1)
#pragma unroll
    for (int up = 0; up < 2; ++up) {
      if (up == 1 && (wh == 0.f || j < 1)) break;
      const int i = j + c - up;
      if (i >= T) continue;
      const size_t qi = static_cast<size_t>(i) * D;
      float qq[D / 8], gg[D / 8];
      load_part<Tin, D>(Q + qi, e, qq);
      load_part<Tin, D>(G + qi, e, gg);
      const float* klo = up ? kp : kr;
      const float* khi = up ? kr : kn;
      const float* vlo = up ? vp : vr;
      const float* vhi = up ? vr : vn;
      float slo = 0.f, shi = 0.f, glo = 0.f, ghi = 0.f;
#pragma unroll
      for (int d = 0; d < D / 8; ++d) {
        slo = fmaf(klo[d], qq[d], slo);
        shi = fmaf(khi[d], qq[d], shi);
        glo = fmaf(vlo[d], gg[d], glo);
        ghi = fmaf(vhi[d], gg[d], ghi);
      }
      const float s = wl * group_sum(slo) + wh * group_sum(shi);
      const float g = wl * group_sum(glo) + wh * group_sum(ghi);
      const float p = expf(sc * s - lse[rbase + i]);
      const float ds = p * (g - delta[rbase + i]);
      const float w = up ? wh : wl;
#pragma unroll
      for (int d = 0; d < D / 8; ++d) {
        gk[d] = fmaf(ds * w * sc, qq[d], gk[d]);
        gv[d] = fmaf(p * w, gg[d], gv[d]);
      }
    }
  }
  store_part<D>(dk + base + static_cast<size_t>(j) * D, e, gk);
  store_part<D>(dv + base + static_cast<size_t>(j) * D, e, gv);
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
  dim3 grid((pr.T + kRowsPerWave - 1) / kRowsPerWave, pr.B * pr.H);
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
  dim3 grid((pr.T + kRowsPerWave - 1) / kRowsPerWave, pr.B * pr.H);
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
  dim3 grid((pr.T + kRowsPerWave - 1) / kRowsPerWave, pr.B * pr.H);
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
  return static_cast<size_t>((pr.T + kRowsPerWave - 1) / kRowsPerWave) * pr.B * pr.H;
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
