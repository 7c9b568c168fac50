// Learned per-layer alpha on the device: theta -> alpha and the layer's tap
// table, and the optimizer update of every layer's theta from its dL/dalpha,
// each in one launch, so that a training step never brings alpha to the host.
//
// Method: Depth-Staggered Fibonacci Spacing for Sparse Attention (gist.science
// technical summary), Methodology > Experimental variables, Learned: one free
// parameter theta per layer, initialised at alpha = 1, trained by gradient
// descent; Architecture and attention > Scaling: alpha in [0.5, 1.5]. The page
// names neither the map nor the optimizer; this library offers
//   FSA_THETA_CLAMP  alpha = clip(theta, 0.5, 1.5), theta projected back onto
//                    [0.5, 1.5] after each update (projected gradient descent);
//   FSA_THETA_TANH   alpha = 1 + tanh(theta) / 2, theta unconstrained;
// and plain gradient descent or Adam (bias-corrected). alpha is the map in
// fp64 rounded once to fp32; the chain rule takes that rounding as the
// identity: dL/dtheta = dL/dalpha * dalpha/dtheta.
#include <hip/hip_runtime.h>

#include <cmath>

#include "fsa.h"
#include "fsa_internal.h"
#include "fsa_taps.h"

namespace fsa {
namespace {

constexpr int kMaxLayers = 1024;   // one workgroup, a thread per layer
static_assert(sizeof(Taps) <= FSA_TAP_TABLE_BYTES, "tap table slot");

__device__ double map_alpha(double th, int theta_map) {
  if (theta_map == FSA_THETA_CLAMP) return th < 0.5 ? 0.5 : (th > 1.5 ? 1.5 : th);
  return 1.0 + 0.5 * tanh(th);
}

__device__ double map_slope(double th, int theta_map) {
  if (theta_map == FSA_THETA_CLAMP) return (th >= 0.5 && th <= 1.5) ? 1.0 : 0.0;
  const double t = tanh(th);
  return 0.5 * (1.0 - t * t);
}

// alpha of one layer (fp32) and its tap table, written in place (a table
// built in a private copy would sit in scratch memory: its slots are indexed
// by a running count). A NaN theta gives a NaN alpha, whose table keeps no tap.
__device__ void layer_alpha(float theta, int theta_map, int window, int pattern,
                            float* alpha, char* table) {
  const double th = theta;
  const float a = th != th ? __int_as_float(0x7fc00000)
                           : static_cast<float>(map_alpha(th, theta_map));
  build_taps(pattern, a, window, reinterpret_cast<Taps*>(table));
  *alpha = a;
}

__global__ __launch_bounds__(kMaxLayers) void theta_alpha_kernel(
    const float* __restrict__ theta, int L, int theta_map, int window,
    int pattern, float* __restrict__ alpha, char* __restrict__ tables) {
  const int l = threadIdx.x;
  if (l < L)
    layer_alpha(theta[l], theta_map, window, pattern, alpha + l,
                tables + static_cast<size_t>(l) * FSA_TAP_TABLE_BYTES);
}

// One update of every layer's theta. state = [m: L floats][v: L floats]
// [step: int32], step = the number of updates made so far.
__global__ __launch_bounds__(kMaxLayers) void theta_step_kernel(
    float* __restrict__ theta, const float* __restrict__ dalpha, int L,
    int theta_map, int optimizer, float lr, float beta1, float beta2, float eps,
    char* __restrict__ state, int window, int pattern, float* __restrict__ alpha,
    char* __restrict__ tables) {
  const int l = threadIdx.x;
  float* m = reinterpret_cast<float*>(state);
  float* v = m + L;
  int* step = reinterpret_cast<int*>(state + 8 * static_cast<size_t>(L));
  const int t = *step + 1;                            // 1-based step of this update
  __syncthreads();                                    // every thread has read it
  if (l == 0) *step = t;
  if (l >= L) return;
  double th = theta[l];
  const double g = static_cast<double>(dalpha[l]) * map_slope(th, theta_map);
  if (optimizer == FSA_OPT_SGD) {
    th = th - static_cast<double>(lr) * g;
  } else {
    const double b1 = beta1, b2 = beta2;
    const double mm = b1 * m[l] + (1.0 - b1) * g;
    const double vv = b2 * v[l] + (1.0 - b2) * g * g;
    const double mh = mm / (1.0 - pow(b1, static_cast<double>(t)));
    const double vh = vv / (1.0 - pow(b2, static_cast<double>(t)));
    th = th - static_cast<double>(lr) * mh / (sqrt(vh) + static_cast<double>(eps));
    m[l] = static_cast<float>(mm);
    v[l] = static_cast<float>(vv);
  }
  if (theta_map == FSA_THETA_CLAMP) th = th < 0.5 ? 0.5 : (th > 1.5 ? 1.5 : th);
  const float th32 = static_cast<float>(th);
  theta[l] = th32;
  layer_alpha(th32, theta_map, window, pattern, alpha + l,
              tables + static_cast<size_t>(l) * FSA_TAP_TABLE_BYTES);
}

bool aligned(const void* p, unsigned a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

bool table_pattern_ok(int pattern) {
  return (pattern & ~(FSA_BASE_MASK | FSA_MODE_MASK)) == 0;
}

}  // namespace
}  // namespace fsa

using namespace fsa;

extern "C" {

int fsa_theta_alpha(const float* theta, int num_layers, int theta_map, int window,
                    int pattern, float* alpha, void* tap_tables, void* stream) {
  if (num_layers < 1 || num_layers > kMaxLayers || window < 1 ||
      (theta_map != FSA_THETA_CLAMP && theta_map != FSA_THETA_TANH) ||
      !table_pattern_ok(pattern))
    return FSA_ERR_INVALID_ARG;
  if (!theta || !alpha || !tap_tables || !aligned(theta, 4) || !aligned(alpha, 4) ||
      !aligned(tap_tables, 256))
    return FSA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(theta_alpha_kernel, dim3(1), dim3(num_layers), 0,
                     static_cast<hipStream_t>(stream), theta, num_layers, theta_map,
                     window, pattern, alpha, static_cast<char*>(tap_tables));
  return status_of(hipGetLastError());
}

int fsa_theta_step(float* theta, const float* dalpha, int num_layers, int theta_map,
                   int optimizer, float lr, float beta1, float beta2, float eps,
                   void* state, int window, int pattern, float* alpha,
                   void* tap_tables, void* stream) {
  if (num_layers < 1 || num_layers > kMaxLayers || window < 1 ||
      (theta_map != FSA_THETA_CLAMP && theta_map != FSA_THETA_TANH) ||
      (optimizer != FSA_OPT_SGD && optimizer != FSA_OPT_ADAM) ||
      !table_pattern_ok(pattern) || !std::isfinite(lr) || lr < 0.f)
    return FSA_ERR_INVALID_ARG;
  if (optimizer == FSA_OPT_ADAM &&
      (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f) ||
       !std::isfinite(eps) || !(eps > 0.f)))
    return FSA_ERR_INVALID_ARG;
  if (!theta || !dalpha || !state || !alpha || !tap_tables || !aligned(theta, 4) ||
      !aligned(dalpha, 4) || !aligned(state, 16) || !aligned(alpha, 4) ||
      !aligned(tap_tables, 256))
    return FSA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(theta_step_kernel, dim3(1), dim3(num_layers), 0,
                     static_cast<hipStream_t>(stream), theta, dalpha, num_layers,
                     theta_map, optimizer, lr, beta1, beta2, eps,
                     static_cast<char*>(state), window, pattern, alpha,
                     static_cast<char*>(tap_tables));
  return status_of(hipGetLastError());
}

}  // extern "C"
