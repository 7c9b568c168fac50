// Rotary position embedding of query or key rows, the pass that precedes the
// gather of Fibonacci-spaced sparse attention.
//
// Method: Depth-Staggered Fibonacci Spacing for Sparse Attention (gist.science
// technical summary), Methodology > Architecture and attention > Implementation
// (RoPE is applied before the gather, so the attention kernels take rotated q
// and k rows) and Significance and claims (native RoPE, no scaling). The page
// fixes neither the pairing nor the frequencies; this pass uses the
// rotate-half pairing (m, m + D/2) with frequency theta_m = base^(-2m/D), the
// same rotation the input generator applies.
//
// Row t of slab (b, h) stands at position p = pos0[b] + t (p = t without
// pos0). For m < D/2 the pair (x_m, x_{m+D/2}) turns by the angle p*theta_m:
//   y_m       = x_m cos(p theta_m) - x_{m+D/2} sin(p theta_m)
//   y_{m+D/2} = x_m sin(p theta_m) + x_{m+D/2} cos(p theta_m)
// The inverse turns by -p*theta_m (the transpose): it maps the gradient with
// respect to rotated rows to the gradient with respect to the rows before
// rotation.
//
// The pass reads and writes each element once, so it is bound by HBM
// bandwidth. One thread rotates 4 consecutive pairs of row t in up to 4
// heads of one batch entry (two 8-byte (bf16) or 16-byte (fp32) loads per
// head, consecutive threads on consecutive addresses); the heads share the
// row's angles. The angle is reduced in fp64 (p * theta_m / 2pi minus its
// nearest integer) before the fp32 sine and cosine, so positions far beyond
// 2^24 radians keep full fp32 accuracy.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "fsa.h"
#include "fsa_internal.h"

namespace fsa {
namespace {

constexpr int kRopeBlock = 256;
constexpr int kPairsPerThread = 4;
constexpr int kHeads = 4;               // heads of one batch entry per thread

__device__ __forceinline__ void load4(const float* p, float* r) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  r[0] = a.x;
  r[1] = a.y;
  r[2] = a.z;
  r[3] = a.w;
}

__device__ __forceinline__ void load4(const uint16_t* p, float* r) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  r[0] = __uint_as_float(u.x << 16);
  r[1] = __uint_as_float(u.x & 0xffff0000u);
  r[2] = __uint_as_float(u.y << 16);
  r[3] = __uint_as_float(u.y & 0xffff0000u);
}

__device__ __forceinline__ void store4(float* p, const float* r) {
  *reinterpret_cast<float4*>(p) = make_float4(r[0], r[1], r[2], r[3]);
}

// fp32 -> bf16 bits, round to nearest even (finite values)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void store4(uint16_t* p, const float* r) {
  *reinterpret_cast<uint2*>(p) = make_uint2(bf16_rne(r[0]) | (bf16_rne(r[1]) << 16),
                                            bf16_rne(r[2]) | (bf16_rne(r[3]) << 16));
}

// Frequencies: theta_{m0+j} = theta_{m0} * ratio^j with
// theta_{m0} = 2^(-(2 m0 / D) log2(base)) and ratio = base^(-2/D), in fp64.
// A thread takes 4 pairs of row t in up to kHeads heads of one batch entry:
// those rows share the position, so the sines and cosines are formed once
// for all of them. All loads of a thread are issued before its first store
// (y may alias x).
template <typename Tin, typename Tout>
__global__ __launch_bounds__(kRopeBlock) void rope_kernel(
    const Tin* x, Tout* y, int H, int T, int D, double log2_base, double ratio,
    const int* __restrict__ pos0, float sgn, long long n_threads) {
  const long long gid = static_cast<long long>(blockIdx.x) * kRopeBlock + threadIdx.x;
  if (gid >= n_threads) return;
  const int per_row = D / (2 * kPairsPerThread);
  const long long r = gid / per_row;                 // (b, head group, t)
  const int m0 = static_cast<int>(gid - r * per_row) * kPairsPerThread;
  const long long bg = r / T;
  const int t = static_cast<int>(r - bg * T);
  const int groups = (H + kHeads - 1) / kHeads;
  const int b = static_cast<int>(bg / groups);
  const int h0 = static_cast<int>(bg - static_cast<long long>(b) * groups) * kHeads;
  const int nh = min(kHeads, H - h0);
  const long long p = (pos0 ? static_cast<long long>(pos0[b]) : 0LL) + t;
  const int half = D / 2;
  const long long slab = static_cast<long long>(T) * D;
  const long long off0 = (static_cast<long long>(b) * H + h0) * slab +
                         static_cast<long long>(t) * D + m0;

  float xa[kHeads][kPairsPerThread], xb[kHeads][kPairsPerThread];
#pragma unroll
  for (int h = 0; h < kHeads; ++h)
    if (h < nh) {
      load4(x + off0 + h * slab, xa[h]);
      load4(x + off0 + h * slab + half, xb[h]);
    }

  constexpr double kInv2Pi = 0.15915494309189533577;   // 1 / (2 pi)
  double theta = exp2(-(2.0 * m0 / D) * log2_base);
  const double pd = static_cast<double>(p);
  float cs[kPairsPerThread], sn[kPairsPerThread];
#pragma unroll
  for (int j = 0; j < kPairsPerThread; ++j) {
    double rev = pd * theta * kInv2Pi;                 // turns
    rev -= rint(rev);                                  // in [-1/2, 1/2]
    sincospif(static_cast<float>(2.0 * rev), &sn[j], &cs[j]);   // angle 2 pi rev
    sn[j] *= sgn;
    theta *= ratio;
  }

#pragma unroll
  for (int h = 0; h < kHeads; ++h)
    if (h < nh) {
      float ya[kPairsPerThread], yb[kPairsPerThread];
#pragma unroll
      for (int j = 0; j < kPairsPerThread; ++j) {
        // one rounding order, written out (the fused rotation in the
        // attention kernels uses the same, so both give the same bits)
        ya[j] = fmaf(xa[h][j], cs[j], -(xb[h][j] * sn[j]));
        yb[j] = fmaf(xa[h][j], sn[j], xb[h][j] * cs[j]);
      }
      store4(y + off0 + h * slab, ya);
      store4(y + off0 + h * slab + half, yb);
    }
}

long long rope_threads(int B, int H, int T, int D) {
  return static_cast<long long>(B) * ((H + kHeads - 1) / kHeads) * T *
         (D / (2 * kPairsPerThread));
}

template <typename Tin, typename Tout>
hipError_t launch_typed(const void* x, void* y, int B, int H, int T, int D,
                        double base, const int* pos0, bool inverse, hipStream_t s) {
  const long long n_threads = rope_threads(B, H, T, D);
  const long long blocks = (n_threads + kRopeBlock - 1) / kRopeBlock;
  hipLaunchKernelGGL((rope_kernel<Tin, Tout>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kRopeBlock), 0, s, static_cast<const Tin*>(x),
                     static_cast<Tout*>(y), H, T, D, std::log2(base),
                     std::pow(base, -2.0 / D), pos0, inverse ? -1.f : 1.f, n_threads);
  return hipGetLastError();
}

}  // namespace

long long rope_blocks(int B, int H, int T, int D) {
  return (rope_threads(B, H, T, D) + kRopeBlock - 1) / kRopeBlock;
}

hipError_t launch_rope(const void* x, int in_dtype, int B, int H, int T, int D,
                       double base, const int* pos0, bool inverse, void* y,
                       int out_dtype, hipStream_t s) {
  const bool in_bf = in_dtype == FSA_DTYPE_BF16, out_bf = out_dtype == FSA_DTYPE_BF16;
  if (in_bf && out_bf)
    return launch_typed<uint16_t, uint16_t>(x, y, B, H, T, D, base, pos0, inverse, s);
  if (in_bf)
    return launch_typed<uint16_t, float>(x, y, B, H, T, D, base, pos0, inverse, s);
  if (out_bf)
    return launch_typed<float, uint16_t>(x, y, B, H, T, D, base, pos0, inverse, s);
  return launch_typed<float, float>(x, y, B, H, T, D, base, pos0, inverse, s);
}

}  // namespace fsa
