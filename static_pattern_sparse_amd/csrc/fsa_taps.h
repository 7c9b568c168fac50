// Tap table of one layer from its fp32 alpha, the window and the tap pattern.
// The same code runs on the host (the planner behind every entry point that
// takes alpha by value) and on the device (tables written from a device-
// resident alpha, for learned alpha), so the two tables agree bit for bit:
// every step is an exact fp64 operation (a product of a 24-bit and a 15-bit
// integer, ceil, floor, a difference of nearby values) followed by one
// rounding to fp32.
#pragma once

#include <hip/hip_runtime.h>

#include "fsa.h"
#include "fsa_internal.h"

namespace fsa {

// Base distance k of a pattern.
//   Fibonacci (Methodology > Architecture and attention > Attended set):
//     1, 2, 3, 5, ..., 987, the leading 1 taken once;
//   power of two (Methodology > Control variables): 1, 2, 4, ..., 16384,
//     fifteen terms, as many as the Fibonacci list. The page's examples of
//     offsets that only a longer evaluation reaches (1024 and 2048 at four
//     times a 1024 training length, Core contributions and results > 3.
//     Length extrapolation, base sensitivity) need a ladder that goes on past
//     987; terms beyond a sequence's length attend nothing.
__host__ __device__ inline int base_term(int pattern, int k) {
  if ((pattern & FSA_BASE_MASK) == FSA_BASE_POW2) return 1 << k;
  int a = 1, b = 2;                                   // f_0, f_1
  for (int i = 0; i < k; ++i) {
    const int c = a + b;
    a = b;
    b = c;
  }
  return a;
}

// Nearest integer to d >= 0, ties to the even neighbour.
__host__ __device__ inline double round_even(double d) {
  const double f = floor(d);
  const double r = d - f;
  if (r > 0.5) return f + 1.0;
  if (r < 0.5) return f;
  return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

// One base distance at scale alpha: the distance c of the lower row, the
// weight t of the upper row and the slope d(position)/d(alpha). The distance
// alpha*f is exact in fp64 (24 + 15 significant bits).
//   interpolated (Methodology > Architecture and attention > Implementation):
//     c = ceil(d), t = c - d, slope -f;
//   rounded (the integer offsets that let static runs take a fused mask path,
//   Core contributions and results > 2. Learned dilation is inert,
//   efficiency): c = round(d), t = 0, slope 0 -- the attended rows do not
//   move with alpha.
__host__ __device__ inline void tap_of(int pattern, double d, double f, double* c,
                                       double* t, double* slope) {
  if (pattern & FSA_MODE_ROUND) {
    *c = round_even(d);
    *t = 0.0;
    *slope = 0.0;
  } else {
    *c = ceil(d);
    *t = *c - d;
    *slope = -f;
  }
}

// The kept base distances (alpha*f >= W), ascending; each weight rounded
// once to fp32 from its exact fp64 value. A non-finite alpha keeps no tap.
__host__ __device__ inline void build_taps(int pattern, float alpha, int window, Taps* t) {
  *t = Taps{};                                        // unused slots zero
  for (int k = 0; k < kNumTaps; ++k) {
    const double f = base_term(pattern, k);
    const double d = static_cast<double>(alpha) * f;
    if (!(d >= static_cast<double>(window))) continue;   // inside the window
    double c, hi, slope;
    tap_of(pattern, d, f, &c, &hi, &slope);
    const int n = t->n++;
    t->c[n] = static_cast<int>(c);
    t->w_hi[n] = static_cast<float>(hi);
    t->w_lo[n] = static_cast<float>(1.0 - hi);
    t->neg_f[n] = static_cast<float>(slope);
  }
}

}  // namespace fsa
