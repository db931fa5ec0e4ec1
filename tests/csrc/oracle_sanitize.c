/* Every oracle routine on small edge-case inputs, for a build under
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize.py).
 * Buffers are allocated at exactly the sizes the routines' contracts give,
 * so a read or write past them, or any undefined operation, aborts the run.
 * The values are not checked here (the pins do that); the run must reach its
 * last line. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static void* xalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) abort();
  memset(p, 0x5A, n ? n : 1);
  return p;
}

static size_t esize(int dt) { return dt == ORACLE_F32 ? 4 : 2; }

/* rows x cols logits in element format dt: a ramp with the policy values
 * (+inf, a NaN, -inf) at a few places */
static void* make_x(int dt, int64_t rows, int64_t cols) {
  const int64_t n = rows * cols;
  double* v = (double*)xalloc(sizeof(double) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) v[i] = 3.0 * sin(0.7 * (double)i) + (double)(i % 5);
  if (n > 3) v[1] = INFINITY;
  if (n > 7) v[n - 2] = NAN;
  if (n > 11) v[n / 2] = -INFINITY;
  void* x = xalloc(esize(dt) * (size_t)n);
  oracle_encode(v, n, dt, x);
  free(v);
  return x;
}

static void masks(int64_t rows, int64_t cols, oracle_mask* mk, int32_t* vl, uint8_t* keep) {
  for (int64_t r = 0; r < rows; ++r) vl[r] = (int32_t)((r * 7) % (cols + 3)) - 1; /* -1 .. cols + 1 */
  for (int64_t i = 0; i < rows * cols; ++i) keep[i] = (uint8_t)((i * 5) % 3 != 0);
  mk[0] = (oracle_mask){ORACLE_MASK_NONE, NULL, 0, 0, NULL};
  mk[1] = (oracle_mask){ORACLE_MASK_VALID_LEN, vl, 0, 0, NULL};
  mk[2] = (oracle_mask){ORACLE_MASK_CAUSAL, NULL, 3, -2, NULL};
  mk[3] = (oracle_mask){ORACLE_MASK_KEEP, NULL, 0, 0, keep};
}

static void shape(int dt, int64_t rows, int64_t cols) {
  const int64_t n = rows * cols;
  void* x = make_x(dt, rows, cols);
  int32_t* vl = (int32_t*)xalloc(sizeof(int32_t) * (size_t)rows);
  uint8_t* keep = (uint8_t*)xalloc((size_t)n);
  oracle_mask mk[4];
  masks(rows, cols, mk, vl, keep);
  int32_t* tgt = (int32_t*)xalloc(sizeof(int32_t) * (size_t)rows);
  for (int64_t r = 0; r < rows; ++r) tgt[r] = (int32_t)(r % (cols + 2)) - 1; /* -1 .. cols */
  for (int k = 0; k < 4; ++k) {
    for (int64_t r0 = 0; r0 <= rows; r0 += rows > 1 ? rows - 1 : 1) {
      const int64_t r1 = rows;
      const int64_t m = r1 - r0;
      double* p = (double*)xalloc(sizeof(double) * (size_t)(m * cols));
      uint8_t* cls = (uint8_t*)xalloc((size_t)(m * cols));
      int32_t* st = (int32_t*)xalloc(sizeof(int32_t) * (size_t)m);
      if (oracle_softmax_rows(x, dt, rows, cols, &mk[k], r0, r1, p, cls, st) != 0) abort();
      double* lse = (double*)xalloc(sizeof(double) * (size_t)m);
      if (oracle_log_softmax_rows(x, dt, rows, cols, &mk[k], r0, r1, lse, p) != 0) abort();
      double* loss = (double*)xalloc(sizeof(double) * (size_t)m);
      if (oracle_cross_entropy_rows(x, dt, rows, cols, &mk[k], tgt, r0, r1, loss, p) != 0) abort();
      if (oracle_cross_entropy_rows(x, dt, rows, cols, &mk[k], tgt, r0, r1, loss, NULL) != 0) abort();
      const int64_t chunks[3] = {1, 3, cols + 5};
      for (int c = 0; c < 3; ++c) {
        const int64_t ch = chunks[c];
        const int64_t nch = cols ? (cols + ch - 1) / ch : 0;
        double* cm = (double*)xalloc(sizeof(double) * (size_t)(m * nch));
        double* cl = (double*)xalloc(sizeof(double) * (size_t)(m * nch));
        if (oracle_chunk_stats(x, dt, rows, cols, &mk[k], ch, r0, r1, cm, cl) != 0) abort();
        if (oracle_merge_normalize(x, dt, rows, cols, &mk[k], cm, cl, nch, r0, r1, p, cls, st) != 0) abort();
        double mm, ll;
        if (m > 0) oracle_merge_all(cm, cl, nch, &mm, &ll);
        free(cm);
        free(cl);
      }
      free(p);
      free(cls);
      free(st);
      free(lse);
      free(loss);
      if (m == 0) break;
    }
    /* the CPU baseline on every thread count up to past the row count */
    for (int th = 1; th <= (int)rows + 2; th += 1 + (int)rows / 3) {
      void* y = xalloc(esize(dt) * (size_t)n);
      if (oracle_softmax_rows_encode_mt(x, y, dt, rows, cols, &mk[k], th) != 0) abort();
      free(y);
    }
    /* weighted sums: values as [rows / rpg, cols, d] for rows_per_group 1
     * and rows (when it divides) */
    for (int64_t rpg = 1; rpg <= rows; rpg = rows) {
      if (rows % rpg != 0) break;
      const int64_t groups = rows / rpg, d = 3;
      void* v = make_x(dt == ORACLE_F32 ? ORACLE_BF16 : dt, groups * cols, d);
      double* out = (double*)xalloc(sizeof(double) * (size_t)(rows * d));
      int32_t* st2 = (int32_t*)xalloc(sizeof(int32_t) * (size_t)rows);
      const int wdt = dt == ORACLE_F32 ? ORACLE_BF16 : dt;
      void* s16 = make_x(wdt, rows, cols);
      if (oracle_softmax_weighted_rows(s16, v, wdt, rows, cols, d, rpg, &mk[k], 0, rows, out, st2) != 0) abort();
      const int64_t ch = 2, nch = cols ? (cols + ch - 1) / ch : 0;
      double* wm = (double*)xalloc(sizeof(double) * (size_t)(rows * nch));
      double* wl = (double*)xalloc(sizeof(double) * (size_t)(rows * nch));
      double* wo = (double*)xalloc(sizeof(double) * (size_t)(rows * nch * d));
      if (oracle_weighted_chunk_states(s16, v, wdt, rows, cols, d, rpg, &mk[k], ch, 0, rows, wm, wl, wo) != 0)
        abort();
      if (nch >= 2) {
        double om[3], mo, lo;
        oracle_weighted_merge(wm[0], wl[0], wo, wm[1], wl[1], wo + d, d, &mo, &lo, om);
      }
      free(v);
      free(out);
      free(st2);
      free(s16);
      free(wm);
      free(wl);
      free(wo);
      if (rpg == rows) break;
    }
  }
  /* the backward on p, g in the element format */
  {
    void* g = make_x(dt, rows, cols);
    double* dx = (double*)xalloc(sizeof(double) * (size_t)n);
    if (oracle_softmax_backward_rows(x, g, dt, rows, cols, 0, rows, dx) != 0) abort();
    free(g);
    free(dx);
  }
  for (int64_t i = 0; i < n; ++i) (void)oracle_decode(x, dt, i);
  for (int64_t r = 0; r < rows; ++r) (void)oracle_valid_prefix(&mk[1], r, cols);
  free(x);
  free(vl);
  free(keep);
  free(tgt);
}

int main(void) {
  const int64_t shapes[][2] = {{0, 0}, {0, 5}, {3, 0}, {1, 1}, {2, 7}, {5, 64}, {4, 513}, {7, 33}};
  for (int dt = 0; dt < 3; ++dt)
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) shape(dt, shapes[i][0], shapes[i][1]);
  /* the online recurrences and the merge on edge values */
  const double row[8] = {1, 2, -3, 12, 11, 4, -INFINITY, 1000};
  double mt[8], dtr[8];
  oracle_online_elementwise(row, 8, mt, dtr);
  oracle_online_tiled(row, 8, 3, mt, dtr);
  oracle_online_no_rescale(row, 8, mt, dtr);
  double mo, lo;
  oracle_merge(-INFINITY, 0, -INFINITY, 0, &mo, &lo);
  oracle_merge(NAN, NAN, 1, 1, &mo, &lo);
  oracle_merge(5, 2, -INFINITY, 0, &mo, &lo);
  /* rounding at the formats' edges */
  const double edges[] = {0.0, -0.0, 5e-324, 1e-45, 1.4e-45, 6e-8, 5.96e-8, 1e-40, 65504.0, 65520.0, 65519.99,
                          3.4e38, 3.5e38, INFINITY, -INFINITY, NAN, 1.0, -1.0, 0.5, 2.0 / 3.0};
  for (size_t i = 0; i < sizeof edges / sizeof edges[0]; ++i) {
    (void)oracle_round_f32_bits(edges[i]);
    (void)oracle_round_f16_bits(edges[i]);
    (void)oracle_round_bf16_bits(edges[i]);
  }
  puts("sanitize run complete");
  return 0;
}
