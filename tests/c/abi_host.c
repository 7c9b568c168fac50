/*
 * Host-only calls of libfsa from plain C (no GPU needed): the schedules and
 * the tap table, checked against values worked out by hand from the page's
 * definitions [Depth-Staggered Fibonacci Spacing for Sparse Attention:
 * Methodology > Experimental variables; Architecture and attention > Scaling].
 * Prints "ok" and exits 0 when every check holds.
 */
#include <math.h>
#include <stdio.h>
#include <stdint.h>

#include "fsa.h"

static int fails = 0;
#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);     \
      ++fails;                                                \
    }                                                         \
  } while (0)

int main(void) {
  float a[16];
  /* linear: 0.5 + l/15, rounded to fp32 */
  CHECK(fsa_schedule(FSA_SCHEDULE_LINEAR, 16, 0.5f, 1.5f, 7, a) == FSA_OK);
  CHECK(a[0] == 0.5f && a[15] == 1.5f && a[3] == 0.7f);
  /* coprime with stride 7: out[7l mod 16] = linear[l]; out[7] = linear[1] */
  float c[16];
  CHECK(fsa_schedule(FSA_SCHEDULE_COPRIME, 16, 0.5f, 1.5f, 7, c) == FSA_OK);
  CHECK(c[0] == a[0] && c[7] == a[1] && c[14] == a[2] && c[5] == a[3]);
  CHECK(fsa_schedule(FSA_SCHEDULE_COPRIME, 16, 0.5f, 1.5f, 6, c) == FSA_ERR_INVALID_ARG);
  CHECK(fsa_schedule(FSA_SCHEDULE_FIXED, 4, 0.5f, 1.5f, 7, c) == FSA_OK && c[3] == 1.0f);

  /* tap table at alpha = 0.5, W = 12: distances 0.5 f */
  int32_t dist[FSA_NUM_TAPS];
  float t[FSA_NUM_TAPS];
  uint8_t keep[FSA_NUM_TAPS];
  CHECK(fsa_offsets(0.5f, 12, dist, t, keep) == FSA_OK);
  CHECK(dist[6] == 11 && t[6] == 0.5f && !keep[6]);   /* f = 21: d = 10.5 */
  CHECK(dist[7] == 17 && t[7] == 0.0f && keep[7]);    /* f = 34: d = 17   */
  CHECK(dist[14] == 494 && t[14] == 0.5f && keep[14]); /* f = 987: d = 493.5 */
  /* rounded mode, ties to even: 493.5 -> 494, 116.5 -> 116 */
  CHECK(fsa_offsets_ex(FSA_MODE_ROUND, 0.5f, 12, dist, t, keep) == FSA_OK);
  CHECK(dist[14] == 494 && dist[11] == 116 && t[11] == 0.0f);
  /* power-of-two base at alpha = 1.5: 1.5 * 2^k */
  CHECK(fsa_offsets_ex(FSA_BASE_POW2, 1.5f, 12, dist, t, keep) == FSA_OK);
  CHECK(dist[0] == 2 && t[0] == 0.5f && !keep[0]);     /* 1.5 */
  CHECK(dist[3] == 12 && keep[3]);                     /* 12 = W: kept */
  CHECK(dist[14] == 24576 && keep[14]);
  CHECK(fsa_offsets_ex(8, 1.0f, 12, dist, t, keep) == FSA_ERR_INVALID_ARG);

  /* argument checks run before any device call */
  CHECK(fsa_forward(NULL, NULL, NULL, FSA_DTYPE_BF16, 1, 1, 16, 64, 1.0f, 4,
                    NULL, NULL, NULL) == FSA_ERR_INVALID_ARG);
  CHECK(fsa_forward(NULL, NULL, NULL, FSA_DTYPE_BF16, 1, 1, 16, 96, 1.0f, 4,
                    NULL, NULL, NULL) == FSA_ERR_UNSUPPORTED);
  CHECK(fsa_backward_workspace_size(8, 8, 1024, 64, FSA_DTYPE_BF16) % 256 == 0);
  CHECK(fsa_rope(NULL, FSA_DTYPE_BF16, 1, 1, 16, 64, 10000.0f, NULL, 0, NULL,
                 FSA_DTYPE_BF16, NULL) == FSA_ERR_INVALID_ARG);
  CHECK(fsa_rope(NULL, FSA_DTYPE_BF16, 1, 1, 16, 60, 10000.0f, NULL, 0, NULL,
                 FSA_DTYPE_BF16, NULL) == FSA_ERR_UNSUPPORTED);
  CHECK(fsa_rope(NULL, FSA_DTYPE_F32, 1, 1, 0, 64, 10000.0f, NULL, 1, NULL,
                 FSA_DTYPE_F32, NULL) == FSA_OK);

  /* sweep the host planner (under a sanitizer build this checks its memory
   * use): every pattern bit combination, alphas across the range, windows */
  for (int pattern = -1; pattern < 9; ++pattern) {
    for (int ai = 0; ai <= 40; ++ai) {
      const float alpha = 0.5f + ai / 40.0f;
      for (int w = 0; w < 45; w += 4) {
        const int st = fsa_offsets_ex(pattern, alpha, w, dist, t, keep);
        const int valid = (pattern == 0 || pattern == 1 || pattern == 2 || pattern == 3 ||
                           pattern == 4 || pattern == 5 || pattern == 6 || pattern == 7) && w >= 1;
        CHECK(st == (valid ? FSA_OK : FSA_ERR_INVALID_ARG));
        if (st == FSA_OK)
          for (int k = 1; k < FSA_NUM_TAPS; ++k) CHECK(dist[k] >= dist[k - 1]);
      }
    }
  }
  float sched[64];
  for (int L = 1; L <= 64; ++L)
    for (int stride = 1; stride < 12; ++stride) {
      const int st = fsa_schedule(FSA_SCHEDULE_COPRIME, L, 0.5f, 1.5f, stride, sched);
      int a = stride, b = L;
      while (b) { const int r = a % b; a = b; b = r; }
      CHECK(st == (a == 1 ? FSA_OK : FSA_ERR_INVALID_ARG));
    }
  printf("%s\n", fails ? "failed" : "ok");
  return fails ? 1 : 0;
}
