// C ABI of libfsa: argument checks, the per-layer tap table and dispatch.
//
// Method: Depth-Staggered Fibonacci Spacing for Sparse Attention (gist.science
// technical summary), sections Methodology > Architecture and attention and
// Methodology > Experimental variables.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "fsa.h"
#include "fsa_internal.h"

namespace fsa {

namespace {

// Methodology > Architecture and attention > Attended set: Fibonacci distances
// 1 .. 987 with the leading 1 taken once.
constexpr int kFib[kNumTaps] = {1,  2,  3,   5,   8,   13,  21, 34,
                                55, 89, 144, 233, 377, 610, 987};

thread_local int g_last_hip_error = 0;

bool alpha_ok(float a) { return std::isfinite(a) && a >= 0.5f && a <= 1.5f; }

int gcd(int a, int b) {
  while (b) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a < 0 ? -a : a;
}

// Tap table of one layer. The distance alpha*f is formed in fp64 from the fp32
// alpha; 24 + 10 significant bits fit in fp64, so it is exact, and so are
// ceil(d) - d and 1 - (ceil(d) - d). Each weight is then rounded once to fp32.
void build_taps(float alpha, int window, Taps* t) {
  t->n = 0;
  for (int k = 0; k < kNumTaps; ++k) {
    const double d = static_cast<double>(alpha) * kFib[k];
    if (d < static_cast<double>(window)) continue;   // inside the window
    const double c = std::ceil(d);
    const double hi = c - d;
    const int n = t->n++;
    t->c[n] = static_cast<int>(c);
    t->w_hi[n] = static_cast<float>(hi);
    t->w_lo[n] = static_cast<float>(1.0 - hi);
    t->neg_f[n] = -static_cast<float>(kFib[k]);
  }
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Shared shape/argument checks. Returns FSA_OK, or the status to report.
int check_shape(int dtype, int B, int H, int T, int D, float alpha, int window) {
  if (B < 0 || H < 0 || T < 0 || window < 1 || !alpha_ok(alpha))
    return FSA_ERR_INVALID_ARG;
  if (dtype != FSA_DTYPE_F32 && dtype != FSA_DTYPE_BF16) return FSA_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return FSA_ERR_UNSUPPORTED;
  // grid limits: heads on grid.y, 64-bit element offsets inside the kernels
  if (static_cast<long long>(B) * H > 65535) return FSA_ERR_UNSUPPORTED;
  return FSA_OK;
}

}  // namespace

BwdWorkspace bwd_workspace_layout(int B, int H, int T, int D, int dtype) {
  (void)D;
  (void)dtype;
  BwdWorkspace w{};
  const size_t rows = static_cast<size_t>(B) * H * T;
  // one dalpha partial per 8 query rows is an upper bound for every kernel
  // tiling used by the backward pass
  w.n_partials = static_cast<size_t>(B) * H * ((static_cast<size_t>(T) + 7) / 8);
  w.delta_off = 0;
  w.partial_off = align256(rows * sizeof(float));
  w.total = align256(w.partial_off + w.n_partials * sizeof(float));
  return w;
}

}  // namespace fsa

using namespace fsa;

extern "C" {

int fsa_schedule(int kind, int num_layers, float alpha_min, float alpha_max,
                 int stride, float* alpha_out) {
  if (alpha_out == nullptr || num_layers < 1) return FSA_ERR_INVALID_ARG;
  if (kind == FSA_SCHEDULE_FIXED) {
    for (int l = 0; l < num_layers; ++l) alpha_out[l] = 1.0f;
    return FSA_OK;
  }
  if (kind != FSA_SCHEDULE_LINEAR && kind != FSA_SCHEDULE_COPRIME)
    return FSA_ERR_INVALID_ARG;
  if (!alpha_ok(alpha_min) || !alpha_ok(alpha_max) || alpha_min > alpha_max)
    return FSA_ERR_INVALID_ARG;
  if (kind == FSA_SCHEDULE_COPRIME && gcd(stride, num_layers) != 1)
    return FSA_ERR_INVALID_ARG;
  const double lo = alpha_min, hi = alpha_max;
  for (int l = 0; l < num_layers; ++l) {
    const double frac =
        num_layers == 1 ? 0.0 : static_cast<double>(l) / (num_layers - 1);
    const float a = static_cast<float>(lo + (hi - lo) * frac);
    if (kind == FSA_SCHEDULE_LINEAR) {
      alpha_out[l] = a;
    } else {
      const long long dst =
          ((static_cast<long long>(stride) * l) % num_layers + num_layers) %
          num_layers;
      alpha_out[dst] = a;
    }
  }
  return FSA_OK;
}

int fsa_offsets(float alpha, int window, int32_t* c_out, float* t_out,
                uint8_t* keep_out) {
  if (!c_out || !t_out || !keep_out || window < 1 || !alpha_ok(alpha))
    return FSA_ERR_INVALID_ARG;
  for (int k = 0; k < kNumTaps; ++k) {
    const double d = static_cast<double>(alpha) * kFib[k];
    const double c = std::ceil(d);
    c_out[k] = static_cast<int32_t>(c);
    t_out[k] = static_cast<float>(c - d);
    keep_out[k] = d >= static_cast<double>(window) ? 1 : 0;
  }
  return FSA_OK;
}

int fsa_forward(const void* q, const void* k, const void* v, int dtype, int B,
                int H, int T, int D, float alpha, int window, float* out,
                float* lse, void* stream) {
  int st = check_shape(dtype, B, H, T, D, alpha, window);
  if (st != FSA_OK) return st;
  if (static_cast<long long>(B) * H * T == 0) return FSA_OK;
  if (!q || !k || !v || !out || !lse) return FSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(lse))
    return FSA_ERR_INVALID_ARG;
  Taps taps;
  build_taps(alpha, window, &taps);
  Problem pr{B, H, T, D, window, static_cast<float>(1.0 / std::sqrt(double(D)))};
  hipError_t e = launch_fwd_vec(q, k, v, dtype, pr, taps, out, lse,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return FSA_ERR_HIP;
  }
  return FSA_OK;
}

size_t fsa_backward_workspace_size(int B, int H, int T, int D, int dtype) {
  if (check_shape(dtype, B, H, T, D, 1.0f, 1) != FSA_OK) return 0;
  if (static_cast<long long>(B) * H * T == 0) return 0;
  return bwd_workspace_layout(B, H, T, D, dtype).total;
}

int fsa_backward(const void* q, const void* k, const void* v,
                 const void* dout, const float* lse, int dtype, int B, int H,
                 int T, int D, float alpha, int window, float* dq, float* dk,
                 float* dv, float* dalpha, void* workspace,
                 size_t workspace_bytes, void* stream) {
  int st = check_shape(dtype, B, H, T, D, alpha, window);
  if (st != FSA_OK) return st;
  if (dalpha == nullptr) return FSA_ERR_INVALID_ARG;
  const bool empty = static_cast<long long>(B) * H * T == 0;
  if (!empty) {
    if (!q || !k || !v || !dout || !lse || !dq || !dk || !dv)
      return FSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) ||
        !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
      return FSA_ERR_INVALID_ARG;
  }
  BwdWorkspace ws{};
  if (!empty) {
    ws = bwd_workspace_layout(B, H, T, D, dtype);
    if (workspace == nullptr || workspace_bytes < ws.total ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return FSA_ERR_WORKSPACE;
  }
  Taps taps;
  build_taps(alpha, window, &taps);
  Problem pr{B, H, T, D, window, static_cast<float>(1.0 / std::sqrt(double(D)))};
  char* wsb = static_cast<char*>(workspace);
  float* delta = empty ? nullptr : reinterpret_cast<float*>(wsb + ws.delta_off);
  float* partials = empty ? nullptr : reinterpret_cast<float*>(wsb + ws.partial_off);
  hipError_t e = launch_bwd_vec(q, k, v, dout, lse, dtype, pr, taps, dq, dk, dv,
                                delta, partials, ws.n_partials, dalpha,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return FSA_ERR_HIP;
  }
  return FSA_OK;
}

const char* fsa_status_string(int status) {
  switch (status) {
    case FSA_OK: return "ok";
    case FSA_ERR_INVALID_ARG: return "invalid argument";
    case FSA_ERR_UNSUPPORTED: return "unsupported head dimension, dtype or size";
    case FSA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case FSA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int fsa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
