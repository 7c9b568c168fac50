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
#include "fsa_taps.h"

namespace fsa {

namespace {

bool pattern_ok(int pattern) {
  return (pattern & ~(FSA_BASE_MASK | FSA_MODE_MASK | FSA_OUT_BF16)) == 0 &&
         (pattern & FSA_BASE_MASK) <= FSA_BASE_POW2;
}

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
  // grid limits: heads on grid.y of the row-group kernels, one tile per
  // workgroup on grid.x of the tile kernels
  if (static_cast<long long>(B) * H > 65535) return FSA_ERR_UNSUPPORTED;
  if ((static_cast<long long>(T) + 13) / 14 * B * H > 0x7fffffffLL)
    return FSA_ERR_UNSUPPORTED;
  // byte offsets within one (b, h) slab are 32-bit in the kernels
  if (static_cast<long long>(T) * D >= (1LL << 29)) return FSA_ERR_UNSUPPORTED;
  return FSA_OK;
}

Problem make_problem(int B, int H, int T, int D, int window) {
  return Problem{B, H, T, D, window,
                 static_cast<float>(1.0 / std::sqrt(static_cast<double>(D)))};
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FSA_OK;
  g_last_hip_error = static_cast<int>(e);
  return FSA_ERR_HIP;
}

struct BwdArgs {
  bool empty = false;
  Problem pr{};
  TapsArg taps{};
  float* delta = nullptr;
  float* partials = nullptr;
};

BwdWorkspace bwd_layout(int B, int H, int T, int D, int dtype);

// Checks shared by the backward stages; fills *a on success. The tap table
// comes from alpha and the pattern, or from `table` (device memory) when that
// is not null; alpha and the pattern are then not used.
int check_bwd(const void* q, const void* k, const void* v, const void* dout,
              const float* lse, int dtype, int B, int H, int T, int D,
              float alpha, int window, int pattern, void* workspace,
              size_t workspace_bytes, BwdArgs* a, const Taps* table = nullptr) {
  if (table != nullptr) {
    alpha = 1.0f;
    pattern = FSA_PATTERN_FIB;
  }
  if (!pattern_ok(pattern)) return FSA_ERR_INVALID_ARG;
  int st = check_shape(dtype, B, H, T, D, alpha, window);
  if (st != FSA_OK) return st;
  a->empty = static_cast<long long>(B) * H * T == 0;
  if (a->empty) return FSA_OK;
  if (!q || !k || !v || !dout || !lse) return FSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) ||
      !aligned16(lse))
    return FSA_ERR_INVALID_ARG;
  const BwdWorkspace ws = bwd_layout(B, H, T, D, dtype);
  if (workspace == nullptr || workspace_bytes < ws.total ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return FSA_ERR_WORKSPACE;
  if (table != nullptr) {
    a->taps.v = Taps{};
    a->taps.dev = table;
  } else {
    build_taps(pattern, alpha, window, &a->taps.v);
    a->taps.dev = nullptr;
  }
  a->pr = make_problem(B, H, T, D, window);
  char* wsb = static_cast<char*>(workspace);
  a->delta = reinterpret_cast<float*>(wsb + ws.delta_off);
  a->partials = reinterpret_cast<float*>(wsb + ws.partial_off);
  return FSA_OK;
}

BwdWorkspace bwd_layout(int B, int H, int T, int D, int dtype) {
  return bwd_workspace_layout(B, H, T, D, dtype);
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
  // per row: (lse * log2(e), Delta) as two floats
  w.partial_off = align256(rows * 2 * sizeof(float));
  w.total = align256(w.partial_off + w.n_partials * sizeof(float));
  return w;
}

// Kernel family: bf16 inputs take the MFMA tile kernels, fp32 inputs the
// row-group kernels.
hipError_t launch_forward(const void* q, const void* k, const void* v,
                          int dtype, const Problem& pr, const TapsArg& taps,
                          void* out, bool out_bf16, float* lse, hipStream_t s) {
  if (mfma_supported(pr, dtype))
    return launch_fwd_mfma(q, k, v, pr, taps, out, out_bf16, lse, s);
  return launch_fwd_vec(q, k, v, dtype, pr, taps, out, out_bf16, lse, s);
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v,
                         const void* dout, const float* lse, int dtype,
                         const Problem& pr, const TapsArg& taps, float* dq,
                         float* delta, float* partials, hipStream_t s) {
  if (mfma_supported(pr, dtype))
    return launch_bwd_dq_mfma(q, k, v, dout, lse, pr, taps, dq, delta, partials, s);
  return launch_bwd_dq_vec(q, k, v, dout, lse, dtype, pr, taps, dq, delta,
                           partials, s);
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v,
                           const void* dout, const float* lse,
                           const float* delta, const float* partials,
                           int dtype, const Problem& pr, const TapsArg& taps,
                           float* dk, float* dv, float* dalpha, hipStream_t s) {
  const size_t np = bwd_partials_used(pr, dtype);
  if (mfma_supported(pr, dtype))
    return launch_bwd_dkdv_mfma(q, k, v, dout, lse, delta, partials, np, pr,
                                taps, dk, dv, dalpha, s);
  hipError_t e = launch_bwd_dkdv_vec(q, k, v, dout, lse, delta, dtype, pr, taps,
                                     dk, dv, s);
  if (e != hipSuccess) return e;
  return launch_dalpha_reduce(partials, np, dalpha, s);
}

size_t bwd_partials_used(const Problem& pr, int dtype) {
  return mfma_supported(pr, dtype) ? bwd_partials_used_mfma(pr)
                                   : bwd_partials_used_vec(pr);
}

int check_backward_call(const void* q, const void* k, const void* v,
                        const void* dout, const float* lse, int dtype, int B,
                        int H, int T, int D, float alpha, int window,
                        int pattern, const float* dq, const float* dk,
                        const float* dv, const float* dalpha, bool* empty) {
  if (!pattern_ok(pattern)) return FSA_ERR_INVALID_ARG;
  int st = check_shape(dtype, B, H, T, D, alpha, window);
  if (st != FSA_OK) return st;
  if (dalpha == nullptr) return FSA_ERR_INVALID_ARG;
  *empty = static_cast<long long>(B) * H * T == 0;
  if (*empty) return FSA_OK;
  if (!q || !k || !v || !dout || !lse || !dq || !dk || !dv) return FSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FSA_ERR_INVALID_ARG;
  return FSA_OK;
}

int status_of(hipError_t e) { return hip_status(e); }

int backward_both(const void* q, const void* k, const void* v, const void* dout,
                  const float* lse, int dtype, int B, int H, int T, int D,
                  float alpha, int window, int pattern, const Taps* table,
                  float* dq, float* dk, float* dv, float* dalpha, void* workspace,
                  size_t workspace_bytes, void* stream) {
  bool empty = false;
  int st = check_backward_call(q, k, v, dout, lse, dtype, B, H, T, D,
                               table ? 1.0f : alpha, window,
                               table ? FSA_PATTERN_FIB : pattern, dq, dk, dv,
                               dalpha, &empty);
  if (st != FSA_OK) return st;
  BwdArgs a;
  st = check_bwd(q, k, v, dout, lse, dtype, B, H, T, D, alpha, window, pattern,
                 workspace, workspace_bytes, &a, table);
  if (st != FSA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.empty) return hip_status(launch_dalpha_reduce(nullptr, 0, dalpha, s));
  st = hip_status(launch_bwd_dq(q, k, v, dout, lse, dtype, a.pr, a.taps, dq,
                                a.delta, a.partials, s));
  if (st != FSA_OK) return st;
  return hip_status(launch_bwd_dkdv(q, k, v, dout, lse, a.delta, a.partials,
                                    dtype, a.pr, a.taps, dk, dv, dalpha, s));
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

int fsa_offsets_ex(int pattern, float alpha, int window, int32_t* c_out,
                   float* t_out, uint8_t* keep_out) {
  if (!c_out || !t_out || !keep_out || window < 1 || !alpha_ok(alpha) ||
      !pattern_ok(pattern))
    return FSA_ERR_INVALID_ARG;
  for (int k = 0; k < kNumTaps; ++k) {
    const double f = base_term(pattern, k);
    const double d = static_cast<double>(alpha) * f;
    double c, t, slope;
    tap_of(pattern, d, f, &c, &t, &slope);
    c_out[k] = static_cast<int32_t>(c);
    t_out[k] = static_cast<float>(t);
    keep_out[k] = d >= static_cast<double>(window) ? 1 : 0;
  }
  return FSA_OK;
}

int fsa_offsets(float alpha, int window, int32_t* c_out, float* t_out,
                uint8_t* keep_out) {
  return fsa_offsets_ex(FSA_PATTERN_FIB, alpha, window, c_out, t_out, keep_out);
}

int fsa_forward_ex(const void* q, const void* k, const void* v, int dtype,
                   int B, int H, int T, int D, float alpha, int window,
                   int pattern, void* out, float* lse, void* stream) {
  if (!pattern_ok(pattern)) return FSA_ERR_INVALID_ARG;
  int st = check_shape(dtype, B, H, T, D, alpha, window);
  if (st != FSA_OK) return st;
  if (static_cast<long long>(B) * H * T == 0) return FSA_OK;
  if (!q || !k || !v || !out || !lse) return FSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(lse))
    return FSA_ERR_INVALID_ARG;
  TapsArg taps{};
  build_taps(pattern, alpha, window, &taps.v);
  const Problem pr = make_problem(B, H, T, D, window);
  return hip_status(launch_forward(q, k, v, dtype, pr, taps, out,
                                   (pattern & FSA_OUT_BF16) != 0, lse,
                                   static_cast<hipStream_t>(stream)));
}

int fsa_forward(const void* q, const void* k, const void* v, int dtype, int B,
                int H, int T, int D, float alpha, int window, float* out,
                float* lse, void* stream) {
  return fsa_forward_ex(q, k, v, dtype, B, H, T, D, alpha, window,
                        FSA_PATTERN_FIB, out, lse, stream);
}

size_t fsa_backward_workspace_size(int B, int H, int T, int D, int dtype) {
  if (check_shape(dtype, B, H, T, D, 1.0f, 1) != FSA_OK) return 0;
  if (static_cast<long long>(B) * H * T == 0) return 0;
  return bwd_workspace_layout(B, H, T, D, dtype).total;
}

int fsa_backward_dq_ex(const void* q, const void* k, const void* v,
                       const void* dout, const float* lse, int dtype, int B,
                       int H, int T, int D, float alpha, int window,
                       int pattern, float* dq, void* workspace,
                       size_t workspace_bytes, void* stream) {
  BwdArgs a;
  int st = check_bwd(q, k, v, dout, lse, dtype, B, H, T, D, alpha, window,
                     pattern, workspace, workspace_bytes, &a);
  if (st != FSA_OK || a.empty) return st;
  if (!dq || !aligned16(dq)) return FSA_ERR_INVALID_ARG;
  return hip_status(launch_bwd_dq(q, k, v, dout, lse, dtype, a.pr, a.taps, dq,
                                  a.delta, a.partials,
                                  static_cast<hipStream_t>(stream)));
}

int fsa_backward_dkdv_ex(const void* q, const void* k, const void* v,
                         const void* dout, const float* lse, int dtype, int B,
                         int H, int T, int D, float alpha, int window,
                         int pattern, float* dk, float* dv, float* dalpha,
                         void* workspace, size_t workspace_bytes,
                         void* stream) {
  BwdArgs a;
  int st = check_bwd(q, k, v, dout, lse, dtype, B, H, T, D, alpha, window,
                     pattern, workspace, workspace_bytes, &a);
  if (st != FSA_OK) return st;
  if (dalpha == nullptr) return FSA_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.empty) return hip_status(launch_dalpha_reduce(nullptr, 0, dalpha, s));
  if (!dk || !dv || !aligned16(dk) || !aligned16(dv)) return FSA_ERR_INVALID_ARG;
  return hip_status(launch_bwd_dkdv(q, k, v, dout, lse, a.delta, a.partials,
                                    dtype, a.pr, a.taps, dk, dv, dalpha, s));
}

int fsa_backward_ex(const void* q, const void* k, const void* v,
                    const void* dout, const float* lse, int dtype, int B, int H,
                    int T, int D, float alpha, int window, int pattern,
                    float* dq, float* dk, float* dv, float* dalpha,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return fsa::backward_both(q, k, v, dout, lse, dtype, B, H, T, D, alpha, window,
                            pattern, nullptr, dq, dk, dv, dalpha, workspace,
                            workspace_bytes, stream);
}

namespace {

// Checks of the fused-RoPE calls beyond those of the plain ones: bf16 rows
// (the tile kernels), a finite base above 1, pos0 4-byte aligned or null.
int check_rope(int dtype, int D, float base, const int32_t* pos0) {
  if (!std::isfinite(base) || !(base > 1.f)) return FSA_ERR_INVALID_ARG;
  if (pos0 != nullptr && (reinterpret_cast<uintptr_t>(pos0) & 3u) != 0)
    return FSA_ERR_INVALID_ARG;
  if (dtype != FSA_DTYPE_BF16 || (D != 64 && D != 128)) return FSA_ERR_UNSUPPORTED;
  return FSA_OK;
}

RopeArg rope_arg(float base, int D, const int32_t* pos0, void* q_out) {
  RopeArg r{};
  r.on = 1;
  // as the RoPE pass forms them (fsa_rope), so that both turn by the same bits
  r.log2_base = std::log2(static_cast<double>(base));
  r.ratio = std::pow(static_cast<double>(base), -2.0 / D);
  r.pos0 = pos0;
  r.q_out = static_cast<uint16_t*>(q_out);
  return r;
}

}  // namespace

int fsa_forward_rope(const void* q_pre, const void* k, const void* v, int dtype,
                     int B, int H, int T, int D, float alpha, int window,
                     int pattern, float base, const int32_t* pos0, void* out,
                     float* lse, void* q_rot, void* stream) {
  if (!pattern_ok(pattern)) return FSA_ERR_INVALID_ARG;
  int st = check_shape(dtype, B, H, T, D, alpha, window);
  if (st != FSA_OK) return st;
  if ((st = check_rope(dtype, D, base, pos0)) != FSA_OK) return st;
  if (static_cast<long long>(B) * H * T == 0) return FSA_OK;
  if (!q_pre || !k || !v || !out || !lse) return FSA_ERR_INVALID_ARG;
  if (!aligned16(q_pre) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(lse) || (q_rot != nullptr && !aligned16(q_rot)))
    return FSA_ERR_INVALID_ARG;
  TapsArg taps{};
  build_taps(pattern, alpha, window, &taps.v);
  const Problem pr = make_problem(B, H, T, D, window);
  return hip_status(launch_fwd_mfma(q_pre, k, v, pr, taps, out,
                                    (pattern & FSA_OUT_BF16) != 0, lse,
                                    static_cast<hipStream_t>(stream),
                                    rope_arg(base, D, pos0, q_rot)));
}

int fsa_backward_rope(const void* q, const void* k, const void* v,
                      const void* dout, const float* lse, int dtype, int B, int H,
                      int T, int D, float alpha, int window, int pattern,
                      float base, const int32_t* pos0, float* dq_pre,
                      float* dk_pre, float* dv, float* dalpha, void* workspace,
                      size_t workspace_bytes, void* stream) {
  bool empty = false;
  int st = fsa::check_backward_call(q, k, v, dout, lse, dtype, B, H, T, D, alpha,
                                    window, pattern, dq_pre, dk_pre, dv, dalpha,
                                    &empty);
  if (st != FSA_OK) return st;
  if ((st = check_rope(dtype, D, base, pos0)) != FSA_OK) return st;
  BwdArgs a;
  st = check_bwd(q, k, v, dout, lse, dtype, B, H, T, D, alpha, window, pattern,
                 workspace, workspace_bytes, &a);
  if (st != FSA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.empty) return hip_status(launch_dalpha_reduce(nullptr, 0, dalpha, s));
  const RopeArg rope = rope_arg(base, D, pos0, nullptr);
  st = hip_status(launch_bwd_dq_mfma(q, k, v, dout, lse, a.pr, a.taps, dq_pre,
                                     a.delta, a.partials, s, rope));
  if (st != FSA_OK) return st;
  return hip_status(launch_bwd_dkdv_mfma(q, k, v, dout, lse, a.delta, a.partials,
                                         bwd_partials_used(a.pr, dtype), a.pr,
                                         a.taps, dk_pre, dv, dalpha, s, rope));
}

int fsa_forward_dev(const void* q, const void* k, const void* v, int dtype,
                    int B, int H, int T, int D, const void* tap_table,
                    int window, int flags, void* out, float* lse, void* stream) {
  if ((flags & ~FSA_OUT_BF16) != 0) return FSA_ERR_INVALID_ARG;
  int st = check_shape(dtype, B, H, T, D, 1.0f, window);
  if (st != FSA_OK) return st;
  if (static_cast<long long>(B) * H * T == 0) return FSA_OK;
  if (!q || !k || !v || !out || !lse || !tap_table) return FSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(lse) || !aligned16(tap_table))
    return FSA_ERR_INVALID_ARG;
  TapsArg taps{};
  taps.dev = static_cast<const Taps*>(tap_table);
  const Problem pr = make_problem(B, H, T, D, window);
  return hip_status(launch_forward(q, k, v, dtype, pr, taps, out,
                                   (flags & FSA_OUT_BF16) != 0, lse,
                                   static_cast<hipStream_t>(stream)));
}

int fsa_backward_dev(const void* q, const void* k, const void* v,
                     const void* dout, const float* lse, int dtype, int B, int H,
                     int T, int D, const void* tap_table, int window, float* dq,
                     float* dk, float* dv, float* dalpha, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (tap_table == nullptr || !aligned16(tap_table)) return FSA_ERR_INVALID_ARG;
  return fsa::backward_both(q, k, v, dout, lse, dtype, B, H, T, D, 1.0f, window,
                            FSA_PATTERN_FIB, static_cast<const Taps*>(tap_table),
                            dq, dk, dv, dalpha, workspace, workspace_bytes, stream);
}

int fsa_backward_dq(const void* q, const void* k, const void* v,
                    const void* dout, const float* lse, int dtype, int B, int H,
                    int T, int D, float alpha, int window, float* dq,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return fsa_backward_dq_ex(q, k, v, dout, lse, dtype, B, H, T, D, alpha,
                            window, FSA_PATTERN_FIB, dq, workspace,
                            workspace_bytes, stream);
}

int fsa_backward_dkdv(const void* q, const void* k, const void* v,
                      const void* dout, const float* lse, int dtype, int B,
                      int H, int T, int D, float alpha, int window, float* dk,
                      float* dv, float* dalpha, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return fsa_backward_dkdv_ex(q, k, v, dout, lse, dtype, B, H, T, D, alpha,
                              window, FSA_PATTERN_FIB, dk, dv, dalpha,
                              workspace, workspace_bytes, stream);
}

int fsa_backward(const void* q, const void* k, const void* v,
                 const void* dout, const float* lse, int dtype, int B, int H,
                 int T, int D, float alpha, int window, float* dq, float* dk,
                 float* dv, float* dalpha, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return fsa_backward_ex(q, k, v, dout, lse, dtype, B, H, T, D, alpha, window,
                         FSA_PATTERN_FIB, dq, dk, dv, dalpha, workspace,
                         workspace_bytes, stream);
}

int fsa_decode(const void* q, const void* k_cache, const void* v_cache,
               int dtype, int B, int H, int T_cap, int D, const int32_t* pos,
               float alpha, int window, int pattern, void* out, float* lse,
               void* stream) {
  if (!pattern_ok(pattern) || T_cap < 1) return FSA_ERR_INVALID_ARG;
  int st = check_shape(dtype, B, H, T_cap, D, alpha, window);
  if (st != FSA_OK) return st;
  if (static_cast<long long>(B) * H == 0) return FSA_OK;
  if (!q || !k_cache || !v_cache || !pos || !out || !lse)
    return FSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(out) || (reinterpret_cast<uintptr_t>(pos) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return FSA_ERR_INVALID_ARG;
  TapsArg taps{};
  build_taps(pattern, alpha, window, &taps.v);
  return hip_status(launch_decode(q, k_cache, v_cache, dtype, pos, B, H, T_cap,
                                  D, window, taps, out,
                                  (pattern & FSA_OUT_BF16) != 0, lse,
                                  static_cast<hipStream_t>(stream)));
}

int fsa_rope(const void* x, int in_dtype, int B, int H, int T, int D,
             float base, const int32_t* pos0, int inverse, void* y,
             int out_dtype, void* stream) {
  if (B < 0 || H < 0 || T < 0 || D < 2 || (D & 1) != 0 || !std::isfinite(base) ||
      !(base > 1.f))
    return FSA_ERR_INVALID_ARG;
  if ((in_dtype != FSA_DTYPE_F32 && in_dtype != FSA_DTYPE_BF16) ||
      (out_dtype != FSA_DTYPE_F32 && out_dtype != FSA_DTYPE_BF16))
    return FSA_ERR_UNSUPPORTED;
  // one thread per 4 pairs of a row; the grid is one-dimensional
  if ((D & 7) != 0 || D > 1024) return FSA_ERR_UNSUPPORTED;
  if (rope_blocks(B, H, T, D) > 0x7fffffffLL) return FSA_ERR_UNSUPPORTED;
  if (static_cast<long long>(B) * H * T == 0) return FSA_OK;
  if (!x || !y || !aligned16(x) || !aligned16(y) ||
      (pos0 != nullptr && (reinterpret_cast<uintptr_t>(pos0) & 3u) != 0))
    return FSA_ERR_INVALID_ARG;
  // in place only with one element size: rows of different widths would
  // overlap other threads' rows
  if (x == y && in_dtype != out_dtype) return FSA_ERR_INVALID_ARG;
  return hip_status(launch_rope(x, in_dtype, B, H, T, D, static_cast<double>(base),
                                pos0, inverse != 0, y, out_dtype,
                                static_cast<hipStream_t>(stream)));
}

const char* fsa_status_string(int status) {
  switch (status) {
    case FSA_OK: return "ok";
    case FSA_ERR_INVALID_ARG: return "invalid argument";
    case FSA_ERR_UNSUPPORTED: return "unsupported head dimension, dtype or size";
    case FSA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case FSA_ERR_HIP: return "HIP launch failed";
    case FSA_ERR_SCRATCH:
      return "problem needs more scratch than fsa_backward_noalloc's fixed device array";
    default: return "unknown status";
  }
}

int fsa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
