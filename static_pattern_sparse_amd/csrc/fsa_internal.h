// Internal declarations shared by the host planner and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fsa {

constexpr int kNumTaps = 15;

// Kept taps of one layer, ascending distance. Built on the host in fp64 from
// the fp32 alpha (Depth-Staggered Fibonacci Spacing for Sparse Attention,
// Methodology > Architecture and attention > Scaling, Implementation) and
// passed to the kernels by value.
struct Taps {
  int n;                   // number of kept taps (d_k >= W)
  int c[kNumTaps];         // ceil(d_k): distance of the lower row
  float w_lo[kNumTaps];    // 1 - t_k, weight of the lower row
  float w_hi[kNumTaps];    // t_k = ceil(d_k) - d_k, weight of the upper row
  float neg_f[kNumTaps];   // -f_k, d(position)/d(alpha) of the tap
};

// A layer's tap table as the kernels receive it: by value from the host
// planner, or, when `dev` is not null, from device memory -- a table written
// on the device from a device-resident alpha (fsa_theta_alpha,
// fsa_theta_step), so that a learned alpha never travels to the host.
struct TapsArg {
  Taps v;
  const Taps* dev;
};

// The table a kernel reads, in the constant address space: the kernel's own
// argument copy or the device table, both read with scalar loads.
typedef __attribute__((address_space(4))) const Taps CTaps;
__device__ __forceinline__ CTaps& taps_of(const TapsArg& a) {
  return a.dev ? *(CTaps*)a.dev : *(CTaps*)&a.v;
}

// RoPE fused into the bf16 tile kernels: the forward turns its query tile in
// registers (and writes the turned rows when q_out is set), the backward
// turns dq and dk back at store time (the transpose), so only the key rows
// need a pass of their own. Row t of batch entry b stands at position
// pos0[b] + t (t without pos0); frequencies base^(-2m/D), pairs (m, m + D/2).
struct RopeArg {
  int on;               // 0: the rows are already rotated; nothing is turned
  double log2_base;     // log2 of the frequency base
  double ratio;         // base^(-2/D): frequency m+1 over frequency m
  const int* pos0;      // device int32[B], or null
  uint16_t* q_out;      // forward: rotated q rows (bf16) written here if set
};

struct Problem {
  int B, H, T, D, W;
  float scale;  // 1/sqrt(D)
};

// Workspace layout of the backward pass (offsets in bytes, 256-aligned).
struct BwdWorkspace {
  size_t delta_off;     // per row i: Delta_i = sum_e p_ie dP_ie (and, for the
                        // tile kernels, float2 {lse_i * log2(e), Delta_i})
  size_t partial_off;   // float[n_partials]: per-tile dalpha partial sums
  size_t n_partials;
  size_t total;
};
BwdWorkspace bwd_workspace_layout(int B, int H, int T, int D, int dtype);

// Argument checks of the backward entry points apart from the workspace:
// pattern, shape, alpha, window, and the pointers (null, 16-byte alignment).
// FSA_OK when the call may proceed; *empty is set for B*H*T == 0 (then only
// dalpha is written).
int check_backward_call(const void* q, const void* k, const void* v,
                        const void* dout, const float* lse, int dtype, int B,
                        int H, int T, int D, float alpha, int window,
                        int pattern, const float* dq, const float* dk,
                        const float* dv, const float* dalpha, bool* empty);
// fsa_status of a HIP error (FSA_ERR_HIP, recorded for fsa_last_hip_error)
int status_of(hipError_t e);
// The whole backward (dq stage, then dk/dv stage) after every check; the tap
// table from (alpha, pattern), or from `table` in device memory when that is
// not null.
int backward_both(const void* q, const void* k, const void* v, const void* dout,
                  const float* lse, int dtype, int B, int H, int T, int D,
                  float alpha, int window, int pattern, const Taps* table,
                  float* dq, float* dk, float* dv, float* dalpha, void* workspace,
                  size_t workspace_bytes, void* stream);

// Launchers; each returns the hipError_t of its launch. The kernel family is
// chosen from dtype: fp32 inputs use the row-group kernels, bf16 inputs the
// MFMA tile kernels. `out` is fp32, or bf16 (round to nearest even) when
// out_bf16.
hipError_t launch_forward(const void* q, const void* k, const void* v,
                          int dtype, const Problem& pr, const TapsArg& taps,
                          void* out, bool out_bf16, float* lse, hipStream_t s);
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v,
                         const void* dout, const float* lse, int dtype,
                         const Problem& pr, const TapsArg& taps, float* dq,
                         float* delta, float* partials, hipStream_t s);
// dk, dv, and dalpha[0] = fixed-order sum of the dq stage's partials
hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v,
                           const void* dout, const float* lse,
                           const float* delta, const float* partials,
                           int dtype, const Problem& pr, const TapsArg& taps,
                           float* dk, float* dv, float* dalpha, hipStream_t s);
// number of dalpha partials the dq stage writes for this problem
size_t bwd_partials_used(const Problem& pr, int dtype);
hipError_t launch_dalpha_reduce(const float* partials, size_t n, float* dalpha,
                                hipStream_t s);

// decoding step (fsa_decode.hip): one query per (b, h) at position pos[b]
// against rows 0..pos[b] of the cached slabs [B][H][Tcap][D]
hipError_t launch_decode(const void* q, const void* k, const void* v, int dtype,
                         const int* pos, int B, int H, int Tcap, int D, int W,
                         const TapsArg& taps, void* out, bool out_bf16, float* lse,
                         hipStream_t s);

// rotary position embedding pass (fsa_rope.hip): rows [B][H][T][D] of
// in_dtype -> out_dtype, row t of batch entry b at position pos0[b] + t
// (pos0 may be null: position t); inverse turns by the negated angles
hipError_t launch_rope(const void* x, int in_dtype, int B, int H, int T, int D,
                       double base, const int* pos0, bool inverse, void* y,
                       int out_dtype, hipStream_t s);
// workgroups the pass launches (the 1-D grid must stay below 2^31)
long long rope_blocks(int B, int H, int T, int D);

// row-group kernels (fsa_vec.hip): eight lanes per row
hipError_t launch_fwd_vec(const void* q, const void* k, const void* v,
                          int dtype, const Problem& pr, const TapsArg& taps,
                          void* out, bool out_bf16, float* lse, hipStream_t s);
hipError_t launch_bwd_dq_vec(const void* q, const void* k, const void* v,
                             const void* dout, const float* lse, int dtype,
                             const Problem& pr, const TapsArg& taps, float* dq,
                             float* delta, float* partials, hipStream_t s);
hipError_t launch_bwd_dkdv_vec(const void* q, const void* k, const void* v,
                               const void* dout, const float* lse,
                               const float* delta, int dtype,
                               const Problem& pr, const TapsArg& taps, float* dk,
                               float* dv, hipStream_t s);
size_t bwd_partials_used_vec(const Problem& pr);

// MFMA tile kernels (fsa_mfma.hip): bf16 inputs, D in {64, 128}, any window
bool mfma_supported(const Problem& pr, int dtype);
hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v,
                           const Problem& pr, const TapsArg& taps, void* out,
                           bool out_bf16, float* lse, hipStream_t s,
                           const RopeArg& rope = RopeArg{});
hipError_t launch_bwd_dq_mfma(const void* q, const void* k, const void* v,
                              const void* dout, const float* lse,
                              const Problem& pr, const TapsArg& taps, float* dq,
                              float* delta, float* partials, hipStream_t s,
                              const RopeArg& rope = RopeArg{});
hipError_t launch_bwd_dkdv_mfma(const void* q, const void* k, const void* v,
                                const void* dout, const float* lse,
                                const float* delta, const float* partials,
                                size_t n_partials, const Problem& pr,
                                const TapsArg& taps, float* dk, float* dv,
                                float* dalpha, hipStream_t s,
                                const RopeArg& rope = RopeArg{});
size_t bwd_partials_used_mfma(const Problem& pr);

}  // namespace fsa
