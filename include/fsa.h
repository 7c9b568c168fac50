/*
 * fsa.h -- C ABI of libfsa, Fibonacci-spaced sparse attention for AMD Instinct
 * MI355X (gfx950).
 *
 * Method: "Depth-Staggered Fibonacci Spacing for Sparse Attention" (C. A.
 * Capps; gist.science technical summary), cited below as [DSFS: <section>].
 * Each query at position i attends a dense causal window of W keys plus up to
 * fifteen keys at distances d_k = alpha * f_k, f = 1, 2, 3, 5, ..., 987, with
 * one scalar alpha per layer in [0.5, 1.5]; a fractional distance linearly
 * interpolates the two neighbouring key rows and value rows, so the loss has a
 * gradient with respect to alpha; RoPE is applied before the gather
 * [DSFS: Methodology > Architecture and attention: Attended set, Scaling,
 * Implementation]. The schedules are those of [DSFS: Methodology >
 * Experimental variables].
 *
 * Conventions fixed by this library where the page is silent:
 *   - window: key offsets 0..W-1 (the query itself included), cut at row 0;
 *   - a tap with alpha*f_k < W is dropped (it lies inside the window);
 *   - a tap whose position i - alpha*f_k is negative is dropped for query i;
 *   - tap rows: lower a = i - ceil(alpha*f_k) with weight 1 - t, upper a + 1
 *     with weight t = ceil(alpha*f_k) - alpha*f_k;
 *   - one softmax over the union of window and tap entries, scale 1/sqrt(D);
 *   - alpha is taken as the given fp32 value; the distances are formed in fp64;
 *   - at an integer distance d(alpha) uses the slope K[a+1] - K[a], V[a+1] - V[a].
 *
 * Tensor layout: every q, k, v, dout, out, dq, dk, dv is a dense row-major
 * [B][H][T][D] array (element (b,h,t,d) at ((b*H + h)*T + t)*D + d); lse is
 * [B][H][T]. q and k are the post-RoPE rows.
 *
 * Memory and streams: every tensor pointer is a DEVICE pointer owned by the
 * caller; the library allocates no memory and never synchronises. `stream` is
 * a hipStream_t (NULL = the null stream); work is enqueued on it and the call
 * returns at once. Outputs are overwritten, never accumulated into.
 *
 * Errors: each call returns an fsa_status. Argument checks run before any HIP
 * call, so an invalid call enqueues nothing. FSA_ERR_HIP means a launch failed;
 * fsa_last_hip_error() gives the HIP error code of the calling thread. Faults
 * inside kernels surface later, at the caller's synchronisation.
 *
 * Thread safety: the library holds no mutable global state apart from the
 * thread-local last HIP error and fsa_backward_noalloc's per-device scratch
 * address (looked up once under a lock); calls from several threads are safe,
 * except fsa_backward_noalloc calls that overlap on one GPU (they share its
 * scratch array).
 */
#ifndef FSA_H_
#define FSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define FSA_OK 0
#define FSA_ERR_INVALID_ARG 1 /* null/misaligned pointer, bad size, bad alpha */
#define FSA_ERR_UNSUPPORTED 2 /* head dim, dtype or size with no kernel */
#define FSA_ERR_WORKSPACE 3   /* workspace missing or smaller than required */
#define FSA_ERR_HIP 4         /* a HIP launch failed; see fsa_last_hip_error() */
#define FSA_ERR_SCRATCH 5     /* beyond fsa_backward_noalloc's fixed scratch */

/* schedules [DSFS: Methodology > Experimental variables] */
#define FSA_SCHEDULE_FIXED 0   /* alpha = 1 for every layer */
#define FSA_SCHEDULE_LINEAR 1  /* alpha from alpha_min (layer 0) to alpha_max (last layer) */
#define FSA_SCHEDULE_COPRIME 2 /* linear values re-assigned by l -> stride*l mod L */

/* element types of q, k, v and dout */
#define FSA_DTYPE_F32 0
#define FSA_DTYPE_BF16 1

#define FSA_NUM_TAPS 15 /* base distances per pattern (both bases) */

/*
 * Tap patterns: a base list and a mode, or-ed together. The entry points
 * without the _ex suffix use FSA_PATTERN_FIB.
 *   FSA_BASE_FIBONACCI  f = 1, 2, 3, 5, ..., 987 [DSFS: Methodology >
 *                       Architecture and attention > Attended set].
 *   FSA_BASE_POW2       f = 1, 2, 4, ..., 16384, the power-of-two (log-sparse)
 *                       control [DSFS: Methodology > Control variables]; the
 *                       ladder runs past 987 because the page names 1024 and
 *                       2048 as offsets that a 4096-token evaluation reaches
 *                       [DSFS: Core contributions and results > 3. Length
 *                       extrapolation, base sensitivity]; fifteen terms, as
 *                       many as the Fibonacci list.
 *   FSA_MODE_LERP       fractional distances interpolate rows a = i - ceil(d)
 *                       and a + 1 [DSFS: Methodology > Architecture and
 *                       attention > Implementation].
 *   FSA_MODE_ROUND      integer offsets round(d) (nearest, ties to even), the
 *                       mask form of the static runs [DSFS: Core contributions
 *                       and results > 2. Learned dilation is inert,
 *                       efficiency]; the attended rows do not move with alpha,
 *                       so dalpha is 0.
 * In every pattern a term with alpha*f < W is dropped, and for query i a tap
 * applies when i >= c (c the distance of its lower row).
 */
#define FSA_BASE_FIBONACCI 0
#define FSA_BASE_POW2 1
#define FSA_BASE_MASK 1
#define FSA_MODE_LERP 0
#define FSA_MODE_ROUND 2
#define FSA_MODE_MASK 2
#define FSA_PATTERN_FIB (FSA_BASE_FIBONACCI | FSA_MODE_LERP)

/*
 * Output option, or-ed into the same argument of fsa_forward_ex and
 * fsa_decode: `out` holds bf16 (round to nearest even from the fp32 result)
 * instead of fp32, half the bytes written. lse stays fp32. The backward calls
 * ignore the bit (they do not take `out`).
 */
#define FSA_OUT_BF16 4

/*
 * fsa_schedule -- per-layer alpha table, host only.
 *   kind        FSA_SCHEDULE_*.
 *   num_layers  L >= 1.
 *   alpha_min, alpha_max  ends of the linear ladder, 0.5 <= min <= max <= 1.5
 *               (ignored for FIXED).
 *   stride      coprime stride, gcd(stride, L) = 1 (COPRIME only; 7 in the page).
 *   alpha_out   host array of L floats, written.
 * LINEAR: alpha_l = min + (max - min) * l / (L - 1), evaluated in fp64 and
 * rounded once to fp32 (alpha_0 = min when L = 1). COPRIME: out[(stride*l) mod L]
 * = linear[l]. Returns FSA_ERR_INVALID_ARG on a null pointer, L < 1, a range
 * outside [0.5, 1.5], min > max, or gcd(stride, L) != 1.
 */
int fsa_schedule(int kind, int num_layers, float alpha_min, float alpha_max,
                 int stride, float* alpha_out);

/*
 * fsa_offsets -- the tap table the kernels use, host only (for inspection).
 * [DSFS: Methodology > Architecture and attention > Scaling, Implementation]
 *   alpha     fp32 scale in [0.5, 1.5]; window W >= 1.
 *   c_out     host int32[15]: ceil(alpha*f_k), distance of the lower row.
 *   t_out     host float[15]: ceil(alpha*f_k) - alpha*f_k, weight of the upper
 *             row, rounded to fp32 from the exact fp64 value.
 *   keep_out  host uint8[15]: 1 when alpha*f_k >= W.
 * Returns FSA_ERR_INVALID_ARG on a null pointer, W < 1 or a bad alpha.
 */
int fsa_offsets(float alpha, int window, int32_t* c_out, float* t_out,
                uint8_t* keep_out);

/*
 * fsa_offsets_ex -- fsa_offsets for any tap pattern (FSA_BASE_* | FSA_MODE_*):
 * c_out[k] is the lower-row distance of base term k (round(alpha*f_k) in
 * FSA_MODE_ROUND), t_out[k] the upper-row weight (0 in FSA_MODE_ROUND),
 * keep_out[k] = (alpha*f_k >= W). Returns FSA_ERR_INVALID_ARG also for an
 * unknown pattern.
 */
int fsa_offsets_ex(int pattern, float alpha, int window, int32_t* c_out,
                   float* t_out, uint8_t* keep_out);

/*
 * fsa_forward -- out, lse of one layer.
 * [DSFS: Methodology > Architecture and attention]
 *   q, k, v   device [B][H][T][D] of `dtype` (q, k post-RoPE), 16-byte aligned.
 *   dtype     FSA_DTYPE_F32 or FSA_DTYPE_BF16.
 *   B, H, T   >= 0 (a zero product is a no-op); D in {64, 128}. Sizes past
 *             B*H = 65535 or T*D = 2^29 (the kernels' 32-bit offsets within a
 *             slab) return FSA_ERR_UNSUPPORTED.
 *   alpha     fp32 in [0.5, 1.5]; window W >= 1 (W >= T gives causal attention).
 *   out       device float [B][H][T][D], written (fp32 for every dtype).
 *   lse       device float [B][H][T], written: log of the softmax denominator
 *             (natural log, scores already scaled by 1/sqrt(D)).
 */
int fsa_forward(const void* q, const void* k, const void* v, int dtype, int B,
                int H, int T, int D, float alpha, int window, float* out,
                float* lse, void* stream);

/*
 * fsa_backward_workspace_size -- bytes of device scratch fsa_backward needs
 * (per-row softmax terms and per-tile dalpha partials). Returns 0 for an empty
 * problem or an unsupported shape.
 */
size_t fsa_backward_workspace_size(int B, int H, int T, int D, int dtype);

/*
 * fsa_backward -- gradients of one layer.
 * [DSFS: Methodology > Architecture and attention > Implementation (gradient
 * reaches alpha); Experimental variables > Learned]
 *   q, k, v, dout  device [B][H][T][D] of `dtype`; dout is dLoss/dout.
 *   lse       device float [B][H][T] from fsa_forward on the same inputs.
 *   dq, dk, dv  device float [B][H][T][D], written (gradients w.r.t. the
 *             post-RoPE q and k, and v).
 *   dalpha    device float[1], written: dLoss/dalpha summed over B, H and T.
 *   workspace device scratch of at least fsa_backward_workspace_size() bytes,
 *             256-byte aligned; its contents on entry do not matter.
 * The result is deterministic (fixed reduction order).
 */
int fsa_backward(const void* q, const void* k, const void* v,
                 const void* dout, const float* lse, int dtype, int B, int H,
                 int T, int D, float alpha, int window, float* dq, float* dk,
                 float* dv, float* dalpha, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * Split-phase backward: the same two stages fsa_backward runs, for callers
 * that interleave other work between them or time them separately. They must
 * run in this order on one stream, with the same arguments and workspace:
 *   fsa_backward_dq    writes dq, and the per-row softmax terms and per-tile
 *                      dalpha partials into the workspace;
 *   fsa_backward_dkdv  writes dk and dv (reads the per-row terms) and
 *                      dalpha[0] (sums the partials in a fixed order).
 * Arguments, layouts and errors are those of fsa_backward.
 */
int fsa_backward_dq(const void* q, const void* k, const void* v,
                    const void* dout, const float* lse, int dtype, int B, int H,
                    int T, int D, float alpha, int window, float* dq,
                    void* workspace, size_t workspace_bytes, void* stream);
int fsa_backward_dkdv(const void* q, const void* k, const void* v,
                      const void* dout, const float* lse, int dtype, int B,
                      int H, int T, int D, float alpha, int window, float* dk,
                      float* dv, float* dalpha, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * _ex variants: the same calls with a tap pattern (FSA_BASE_* | FSA_MODE_*,
 * and FSA_OUT_BF16 for fsa_forward_ex) after `window`; arguments, layouts and
 * errors as above, plus FSA_ERR_INVALID_ARG for an unknown bit. In
 * FSA_MODE_ROUND dalpha is written as 0. fsa_forward_ex's `out` is float
 * [B][H][T][D], or bf16 bits (uint16) [B][H][T][D] with FSA_OUT_BF16.
 */
int fsa_forward_ex(const void* q, const void* k, const void* v, int dtype,
                   int B, int H, int T, int D, float alpha, int window,
                   int pattern, void* out, float* lse, void* stream);
int fsa_backward_ex(const void* q, const void* k, const void* v,
                    const void* dout, const float* lse, int dtype, int B, int H,
                    int T, int D, float alpha, int window, int pattern,
                    float* dq, float* dk, float* dv, float* dalpha,
                    void* workspace, size_t workspace_bytes, void* stream);
int fsa_backward_dq_ex(const void* q, const void* k, const void* v,
                       const void* dout, const float* lse, int dtype, int B,
                       int H, int T, int D, float alpha, int window,
                       int pattern, float* dq, void* workspace,
                       size_t workspace_bytes, void* stream);
int fsa_backward_dkdv_ex(const void* q, const void* k, const void* v,
                         const void* dout, const float* lse, int dtype, int B,
                         int H, int T, int D, float alpha, int window,
                         int pattern, float* dk, float* dv, float* dalpha,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Learned alpha [DSFS: Methodology > Experimental variables, Learned: one free
 * parameter theta per layer, initialised at alpha = 1 and trained by gradient
 * descent; Architecture and attention > Scaling: alpha in [0.5, 1.5]; Core
 * contributions and results > 2. Learned dilation is inert]. The page fixes
 * neither the map from theta to alpha nor the optimizer; this library offers
 *   FSA_THETA_CLAMP  alpha = clip(theta, 0.5, 1.5); after each update theta is
 *                    projected back onto [0.5, 1.5] (projected gradient
 *                    descent). theta = 1 gives alpha = 1.
 *   FSA_THETA_TANH   alpha = 1 + tanh(theta)/2, theta unconstrained. theta = 0
 *                    gives alpha = 1.
 * alpha is the map evaluated in fp64 and rounded once to fp32. A layer's alpha
 * and its tap table live in device memory, written by fsa_theta_alpha or
 * fsa_theta_step; fsa_forward_dev and fsa_backward_dev read the table there,
 * so a training step never brings alpha to the host.
 */
#define FSA_THETA_CLAMP 0
#define FSA_THETA_TANH 1
#define FSA_OPT_SGD 0  /* theta <- theta - lr * g */
#define FSA_OPT_ADAM 1 /* Adam with bias correction (Kingma and Ba) */
/* bytes of one layer's tap table (an opaque device record); tables of
 * consecutive layers sit FSA_TAP_TABLE_BYTES apart from a 256-byte aligned base */
#define FSA_TAP_TABLE_BYTES 256
/* bytes of fsa_theta_step's optimizer state for L layers: m[L], v[L] (fp32)
 * and the update count (int32) */
#define FSA_THETA_STATE_BYTES(L) (8u * (unsigned)(L) + 16u)

/*
 * fsa_theta_alpha -- alpha and the tap table of every layer from its theta,
 * on the device (one launch).
 *   theta      device float[L], read; 1 <= L <= 1024.
 *   theta_map  FSA_THETA_CLAMP or FSA_THETA_TANH.
 *   window, pattern  the window and tap pattern (FSA_BASE_* | FSA_MODE_*) the
 *             tables are for; the attention calls must pass the same window.
 *   alpha      device float[L], written: the fp32 alpha of each layer (NaN
 *             for a NaN theta; that layer's table then keeps no tap).
 *   tap_tables device, L * FSA_TAP_TABLE_BYTES bytes, 256-byte aligned,
 *             written: layer l's table at byte l * FSA_TAP_TABLE_BYTES.
 * Returns FSA_ERR_INVALID_ARG for a bad L, map, window or pattern, or a null
 * or misaligned pointer.
 */
int fsa_theta_alpha(const float* theta, int num_layers, int theta_map, int window,
                    int pattern, float* alpha, void* tap_tables, void* stream);

/*
 * fsa_theta_step -- one optimizer update of every layer's theta from the
 * layers' dL/dalpha, then the new alpha and tap tables, on the device (one
 * launch, deterministic).
 *   theta      device float[L], updated in place.
 *   dalpha     device float[L]: dL/dalpha of each layer (fsa_backward_dev's
 *             dalpha, one float per layer).
 *   g_l = dalpha_l * dalpha/dtheta(theta_l): 1 on [0.5, 1.5] and 0 outside
 *   for the clip, (1 - tanh(theta)^2)/2 for the tanh map. Then
 *     FSA_OPT_SGD:  theta_l -= lr * g_l;
 *     FSA_OPT_ADAM: t = count + 1; m = beta1 m + (1 - beta1) g,
 *                   v = beta2 v + (1 - beta2) g^2,
 *                   theta_l -= lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps);
 *   with FSA_THETA_CLAMP theta is projected onto [0.5, 1.5]. The update is
 *   computed in fp64; theta, m and v are stored in fp32.
 *   state      device, FSA_THETA_STATE_BYTES(L) bytes, 16-byte aligned: m, v
 *             and the update count, zero before the first update (the caller
 *             clears it once); read and written.
 *   lr >= 0 and finite; for Adam 0 <= beta1, beta2 < 1 and eps > 0.
 *   window, pattern, alpha, tap_tables  as fsa_theta_alpha, for the new theta.
 */
int fsa_theta_step(float* theta, const float* dalpha, int num_layers, int theta_map,
                   int optimizer, float lr, float beta1, float beta2, float eps,
                   void* state, int window, int pattern, float* alpha,
                   void* tap_tables, void* stream);

/*
 * fsa_forward_dev, fsa_backward_dev -- fsa_forward_ex and fsa_backward_ex with
 * the layer's tap table read from device memory (one FSA_TAP_TABLE_BYTES
 * record written by fsa_theta_alpha or fsa_theta_step, 16-byte aligned)
 * instead of formed on the host from alpha. `window` must be the window the
 * table was written for. fsa_forward_dev's `flags` is 0 or FSA_OUT_BF16.
 * Arguments, layouts, results and errors otherwise as fsa_forward_ex and
 * fsa_backward_ex; dalpha[0] is dL/dalpha of the layer.
 */
int fsa_forward_dev(const void* q, const void* k, const void* v, int dtype,
                    int B, int H, int T, int D, const void* tap_table,
                    int window, int flags, void* out, float* lse, void* stream);
int fsa_backward_dev(const void* q, const void* k, const void* v,
                     const void* dout, const float* lse, int dtype, int B, int H,
                     int T, int D, const void* tap_table, int window, float* dq,
                     float* dk, float* dv, float* dalpha, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * fsa_backward_noalloc -- fsa_backward_ex with no workspace argument and no
 * allocation, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *   Arguments, layouts, results and errors as fsa_backward_ex. The per-row
 *   softmax terms and the per-tile dalpha partials go to a fixed device array
 *   of FSA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 *   on until the process ends (looked up at the first call on each device;
 *   the device is the stream's). A problem whose fsa_backward_workspace_size
 *   exceeds it returns FSA_ERR_SCRATCH before any HIP call (16 MiB covers
 *   B*H*T up to about 1.9 million rows, e.g. B1 H16 T65536 at D = 128).
 *   The array keeps the last call's contents; every element the kernels read
 *   is written earlier in the same call, so nothing is cleared. All calls on
 *   one GPU share the array: calls that overlap in time on one GPU (two
 *   streams, two threads) race and give wrong results; serialise them.
 *   The call itself allocates nothing (no hipMalloc, no library allocation).
 */
#define FSA_NOALLOC_SCRATCH_BYTES (16u << 20)
int fsa_backward_noalloc(const void* q, const void* k, const void* v,
                         const void* dout, const float* lse, int dtype, int B,
                         int H, int T, int D, float alpha, int window,
                         int pattern, float* dq, float* dk, float* dv,
                         float* dalpha, void* stream);

/*
 * fsa_decode -- one decoding step: a new query per (b, h) against the cached
 * rows of its slab.
 * [DSFS: Methodology > Architecture and attention > Attended set, Scaling,
 * Implementation; Core contributions and results > 2. Learned dilation is
 * inert, efficiency (the inference latency of this step)]
 *   q         device [B][H][D] of `dtype`: the post-RoPE query of position
 *             pos[b], 16-byte aligned.
 *   k_cache, v_cache  device [B][H][T_cap][D] of `dtype`, 16-byte aligned:
 *             rows 0..pos[b] of slab (b, h) hold the keys (post-RoPE) and
 *             values of positions 0..pos[b]; rows after pos[b] are never read.
 *   pos       device int32[B], 4-byte aligned: the query's position per batch
 *             entry. A position outside [0, T_cap) cannot be reported from the
 *             device: that entry's out and lse are written as NaN.
 *   alpha, window, pattern  as for fsa_forward_ex (FSA_OUT_BF16 included).
 *   out       device float [B][H][D] (bf16 bits with FSA_OUT_BF16), written;
 *   lse       device float [B][H], written.
 * The query attends exactly what row pos[b] of fsa_forward attends. Returns
 * FSA_ERR_INVALID_ARG for a null or misaligned pointer, T_cap < 1, a bad alpha,
 * window or pattern; FSA_ERR_UNSUPPORTED as fsa_forward.
 */
int fsa_decode(const void* q, const void* k_cache, const void* v_cache,
               int dtype, int B, int H, int T_cap, int D, const int32_t* pos,
               float alpha, int window, int pattern, void* out, float* lse,
               void* stream);

/*
 * fsa_rope -- rotary position embedding of query or key rows, the pass that
 * precedes the gather (the attention entry points take its output).
 * [DSFS: Methodology > Architecture and attention > Implementation (RoPE is
 * applied before the gather); Significance and claims (native RoPE, no
 * scaling); Core contributions and results > 3. Length extrapolation,
 * mechanism (a fixed offset keeps the same rotation angle at every position)]
 * The pages fix neither pairing nor frequencies; this library uses the
 * rotate-half pairing: for m < D/2 the pair (x[m], x[m + D/2]) of row t of
 * slab (b, h) turns by the angle p * base^(-2m/D) at position
 * p = pos0[b] + t:
 *   y[m]       = x[m] cos - x[m + D/2] sin,
 *   y[m + D/2] = x[m] sin + x[m + D/2] cos.
 *   x         device [B][H][T][D] of in_dtype (FSA_DTYPE_F32 or _BF16),
 *             16-byte aligned, read.
 *   y         device [B][H][T][D] of out_dtype, 16-byte aligned, written
 *             (bf16: round to nearest even from the fp32 result). y == x
 *             rotates in place when in_dtype == out_dtype; other overlaps
 *             are not allowed.
 *   pos0      device int32[B], 4-byte aligned: position of row 0 per batch
 *             entry (a decoding step passes T = 1 and its positions), or
 *             NULL for position t.
 *   base      frequency base (10000, 500000, ...), finite and > 1.
 *   inverse   nonzero: turn by the negated angles, the transpose of the
 *             rotation; applied to the gradient with respect to rotated rows
 *             (fsa_backward's dq, dk) it gives the gradient with respect to
 *             the rows before rotation.
 * Angles are reduced modulo 2 pi in fp64 and rotated in fp32. Returns
 * FSA_ERR_INVALID_ARG for a null or misaligned pointer, negative sizes, an odd
 * D or a bad base, or x == y with two dtypes; FSA_ERR_UNSUPPORTED for another
 * dtype, D not a multiple of 8 or above 1024, or a grid beyond 2^31
 * workgroups. B*H*T == 0 is a no-op.
 */
int fsa_rope(const void* x, int in_dtype, int B, int H, int T, int D,
             float base, const int32_t* pos0, int inverse, void* y,
             int out_dtype, void* stream);

/*
 * fsa_forward_rope, fsa_backward_rope -- the attention calls with RoPE fused
 * where the rows sit in registers [DSFS: Methodology > Architecture and
 * attention > Implementation (RoPE before the gather)], for bf16 rows
 * (D = 64 or 128; other dtypes return FSA_ERR_UNSUPPORTED, and take the
 * separate pass fsa_rope). Rotation as fsa_rope: pairs (m, m + D/2), angle
 * p * base^(-2m/D), row t of batch entry b at position p = pos0[b] + t (pos0
 * a device int32[B], 4-byte aligned, or NULL for p = t), base finite and > 1.
 *   fsa_forward_rope: fsa_forward_ex with q_pre the query rows BEFORE rotation
 *     (the kernel turns each query tile in fp32 and rounds it to bf16, nearest
 *     even); k must already be rotated (fsa_rope). When q_rot is not NULL
 *     (device bf16 [B][H][T][D], 16-byte aligned) the turned query rows are
 *     written there, the rows fsa_backward_rope reads as q.
 *   fsa_backward_rope: fsa_backward_ex on the rotated q and k, with dq_pre and
 *     dk_pre the gradients with respect to the rows BEFORE rotation (the
 *     kernels turn dq and dk back at store time, the transpose of the
 *     rotation); dv and dalpha as fsa_backward_ex.
 * Sines and cosines come from the hardware (argument in turns, reduced in
 * fp64); other arguments, layouts and errors as fsa_forward_ex and
 * fsa_backward_ex.
 */
int fsa_forward_rope(const void* q_pre, const void* k, const void* v, int dtype,
                     int B, int H, int T, int D, float alpha, int window,
                     int pattern, float base, const int32_t* pos0, void* out,
                     float* lse, void* q_rot, void* stream);
int fsa_backward_rope(const void* q, const void* k, const void* v,
                      const void* dout, const float* lse, int dtype, int B, int H,
                      int T, int D, float alpha, int window, int pattern,
                      float base, const int32_t* pos0, float* dq_pre,
                      float* dk_pre, float* dv, float* dalpha, void* workspace,
                      size_t workspace_bytes, void* stream);

/* fsa_status_string -- static text for a status code. */
const char* fsa_status_string(int status);

/* fsa_last_hip_error -- HIP error code of this thread's last FSA_ERR_HIP. */
int fsa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FSA_H_ */
