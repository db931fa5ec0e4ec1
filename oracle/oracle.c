/*
 * oracle.c — plain, slow, double-precision CPU reference for batched
 * row-wise softmax, chunk summaries and their merge.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library; the product path never calls
 * it, and nothing here comes from the product path.
 *
 * The page titles cited below are the sources of each definition; section
 * names refer to headings on those pages.
 */
#define _POSIX_C_SOURCE 200809L
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Decoding: the three element formats, exactly.                             */
/* ------------------------------------------------------------------------ */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits;
 * exponent 0 encodes zero and subnormals (fraction * 2^-24), exponent 31
 * encodes infinities and NaNs. */
static double decode_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);
  } else if (e == 31) {
    v = (f == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)(1024 + f), e - 25);
  }
  return sign ? -v : v;
}

/* bfloat16 is the upper half of a binary32 word. */
static double decode_bf16(uint16_t b) {
  uint32_t w = (uint32_t)b << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

double oracle_decode(const void* x, int dtype, int64_t i) {
  if (dtype == ORACLE_F32) {
    float f;
    memcpy(&f, (const char*)x + 4 * i, sizeof f);
    return (double)f;
  }
  uint16_t h;
  memcpy(&h, (const char*)x + 2 * i, sizeof h);
  return dtype == ORACLE_F16 ? decode_f16(h) : decode_bf16(h);
}

/* ------------------------------------------------------------------------ */
/* The mask contract.                                                        */
/* "Stable softmax: keep the normalizer consistent as tiles arrive", masks   */
/* paragraph: invalid tail lanes are excluded from the max and the sum.      */
/* "Online stable softmax", section "Masks, empty rows, and precision": a    */
/* masked score behaves as negative infinity, and a partially masked tile    */
/* forces its masked lanes to negative infinity.                             */
/* ------------------------------------------------------------------------ */

static int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

int64_t oracle_valid_prefix(const oracle_mask* mk, int64_t r, int64_t cols) {
  if (mk == NULL || mk->kind == ORACLE_MASK_NONE) return cols;
  if (mk->kind == ORACLE_MASK_VALID_LEN)
    return clamp64((int64_t)mk->valid_len[r], 0, cols);
  if (mk->kind == ORACLE_MASK_CAUSAL)
    return clamp64((r % mk->causal_period) + 1 + mk->causal_offset, 0, cols);
  return -1;
}

static int lane_valid(const oracle_mask* mk, int64_t r, int64_t j,
                      int64_t cols, int64_t prefix) {
  if (prefix >= 0) return j < prefix;
  return mk->keep[r * cols + j] != 0;
}

static int mask_ok(const oracle_mask* mk) {
  if (mk == NULL) return 1;
  switch (mk->kind) {
    case ORACLE_MASK_NONE: return 1;
    case ORACLE_MASK_VALID_LEN: return mk->valid_len != NULL;
    case ORACLE_MASK_CAUSAL: return mk->causal_period > 0;
    case ORACLE_MASK_KEEP: return mk->keep != NULL;
    default: return 0;
  }
}

/* A value that poisons its row under the declared policy: +inf or NaN in a
 * valid lane ("Stable softmax: keep the normalizer consistent as tiles
 * arrive", masks paragraph: +inf and NaN need an explicit policy; the policy
 * taken is a NaN row). */
static int poisons(double v) { return isnan(v) || (isinf(v) && v > 0); }

/* Neumaier's compensated sum, accumulated in ascending index order. */
typedef struct {
  double s, c;
} nsum;

static void nsum_add(nsum* a, double t) {
  double u = a->s + t;
  if (fabs(a->s) >= fabs(t))
    a->c += (a->s - u) + t;
  else
    a->c += (t - u) + a->s;
  a->s = u;
}

static double nsum_value(const nsum* a) { return a->s + a->c; }

/* ------------------------------------------------------------------------ */
/* Three-pass stable softmax of one row ("Kernel visualization: online       */
/* softmax", section "Overview of safe softmax"; "Softmax numerics           */
/* architecture", section "The max-subtraction identity").                   */
/* ------------------------------------------------------------------------ */

static void set_policy_row(double* p, uint8_t* cls, int64_t cols, double v,
                           uint8_t c) {
  for (int64_t j = 0; j < cols; ++j) {
    p[j] = v;
    cls[j] = c;
  }
}

static int32_t softmax_one_row(const void* x, int dtype, int64_t cols,
                               const oracle_mask* mk, int64_t r, double* p,
                               uint8_t* cls) {
  const int64_t base = r * cols;
  const int64_t prefix = oracle_valid_prefix(mk, r, cols);

  /* Policy check over the valid lanes only. */
  for (int64_t j = 0; j < cols; ++j) {
    if (!lane_valid(mk, r, j, cols, prefix)) continue;
    if (poisons(oracle_decode(x, dtype, base + j))) {
      set_policy_row(p, cls, cols, NAN, ORACLE_LANE_NAN);
      return ORACLE_ROW_POISON;
    }
  }

  /* Pass 1: the maximum over valid lanes that are not -inf. */
  double m = -INFINITY;
  int64_t count = 0;
  for (int64_t j = 0; j < cols; ++j) {
    if (!lane_valid(mk, r, j, cols, prefix)) continue;
    double v = oracle_decode(x, dtype, base + j);
    if (v == -INFINITY) continue;
    if (count == 0 || v > m) m = v;
    ++count;
  }
  if (count == 0) {
    /* Empty or fully masked row: the declared result is all +0.0, and no
     * -inf - (-inf) is ever formed. */
    set_policy_row(p, cls, cols, 0.0, ORACLE_LANE_ZERO);
    return ORACLE_ROW_EMPTY;
  }

  /* Pass 2: l = sum of exp(x_j - m). */
  nsum acc = {0.0, 0.0};
  for (int64_t j = 0; j < cols; ++j) {
    if (!lane_valid(mk, r, j, cols, prefix)) continue;
    double v = oracle_decode(x, dtype, base + j);
    if (v == -INFINITY) continue;
    nsum_add(&acc, exp(v - m));
  }
  const double l = nsum_value(&acc);

  /* Pass 3: divide. */
  for (int64_t j = 0; j < cols; ++j) {
    double v = lane_valid(mk, r, j, cols, prefix)
                   ? oracle_decode(x, dtype, base + j)
                   : -INFINITY;
    if (v == -INFINITY) {
      p[j] = 0.0;
      cls[j] = ORACLE_LANE_ZERO;
    } else {
      p[j] = exp(v - m) / l;
      cls[j] = ORACLE_LANE_NUMERIC;
    }
  }
  return ORACLE_ROW_OK;
}

int oracle_softmax_rows(const void* x, int dtype, int64_t rows, int64_t cols,
                        const oracle_mask* mk, int64_t r0, int64_t r1,
                        double* p, uint8_t* lane_class, int32_t* row_status) {
  if (dtype < 0 || dtype > 2 || rows < 0 || cols < 0 || r0 < 0 || r1 > rows ||
      r0 > r1 || !mask_ok(mk))
    return -1;
  for (int64_t r = r0; r < r1; ++r) {
    int32_t st = softmax_one_row(x, dtype, cols, mk, r, p + (r - r0) * cols,
                                 lane_class + (r - r0) * cols);
    if (row_status) row_status[r - r0] = st;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Chunk summaries ("Stable softmax: keep the normalizer consistent as       */
/* tiles arrive", block-merge paragraph: a block is summarized by its        */
/* maximum and the sum of exponentials shifted by that maximum).             */
/* ------------------------------------------------------------------------ */

int oracle_chunk_stats(const void* x, int dtype, int64_t rows, int64_t cols,
                       const oracle_mask* mk, int64_t chunk_cols, int64_t r0,
                       int64_t r1, double* m, double* l) {
  if (dtype < 0 || dtype > 2 || rows < 0 || cols < 0 || chunk_cols <= 0 ||
      r0 < 0 || r1 > rows || r0 > r1 || !mask_ok(mk))
    return -1;
  const int64_t n_chunks = (cols + chunk_cols - 1) / chunk_cols;
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t prefix = oracle_valid_prefix(mk, r, cols);
    for (int64_t c = 0; c < n_chunks; ++c) {
      const int64_t lo = c * chunk_cols;
      const int64_t hi = lo + chunk_cols < cols ? lo + chunk_cols : cols;
      double cm = -INFINITY;
      int64_t count = 0;
      int poisoned = 0;
      for (int64_t j = lo; j < hi; ++j) {
        if (!lane_valid(mk, r, j, cols, prefix)) continue;
        double v = oracle_decode(x, dtype, r * cols + j);
        if (poisons(v)) {
          poisoned = 1;
          break;
        }
        if (v == -INFINITY) continue;
        if (count == 0 || v > cm) cm = v;
        ++count;
      }
      double* mo = m + (r - r0) * n_chunks + c;
      double* lo_ = l + (r - r0) * n_chunks + c;
      if (poisoned) {
        *mo = NAN;
        *lo_ = NAN;
        continue;
      }
      if (count == 0) {
        *mo = -INFINITY;
        *lo_ = 0.0;
        continue;
      }
      nsum acc = {0.0, 0.0};
      for (int64_t j = lo; j < hi; ++j) {
        if (!lane_valid(mk, r, j, cols, prefix)) continue;
        double v = oracle_decode(x, dtype, r * cols + j);
        if (v == -INFINITY) continue;
        nsum_add(&acc, exp(v - cm));
      }
      *mo = cm;
      *lo_ = nsum_value(&acc);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Softmax-weighted value sums ("Online stable softmax", section on the      */
/* weighted-value numerator: attention also needs the sum of                 */
/* exp(score_j - m) V_j; "Softmax numerics architecture", tiled attention:   */
/* the output is O / d at the end). The plain definition: the three-pass     */
/* probabilities of the row, then each output component as a compensated    */
/* sum of p_j V_jk in ascending j.                                           */
/* ------------------------------------------------------------------------ */

int oracle_softmax_weighted_rows(const void* s, const void* v, int dtype,
                                 int64_t rows, int64_t cols, int64_t d,
                                 int64_t rows_per_group, const oracle_mask* mk,
                                 int64_t r0, int64_t r1, double* out,
                                 int32_t* row_status) {
  if (dtype < 0 || dtype > 2 || rows < 0 || cols < 0 || d < 0 ||
      rows_per_group <= 0 || rows % rows_per_group != 0 || r0 < 0 ||
      r1 > rows || r0 > r1 || !mask_ok(mk))
    return -1;
  double* p = (double*)malloc(sizeof(double) * (size_t)(cols > 0 ? cols : 1));
  uint8_t* cls = (uint8_t*)malloc((size_t)(cols > 0 ? cols : 1));
  if (!p || !cls) {
    free(p);
    free(cls);
    return -1;
  }
  for (int64_t r = r0; r < r1; ++r) {
    double* o = out + (r - r0) * d;
    const int32_t st = softmax_one_row(s, dtype, cols, mk, r, p, cls);
    if (row_status) row_status[r - r0] = st;
    if (st != ORACLE_ROW_OK) {
      for (int64_t k = 0; k < d; ++k) o[k] = st == ORACLE_ROW_POISON ? NAN : 0.0;
      continue;
    }
    const int64_t vbase = (r / rows_per_group) * cols * d;
    for (int64_t k = 0; k < d; ++k) {
      nsum acc = {0.0, 0.0};
      for (int64_t j = 0; j < cols; ++j) {
        if (cls[j] != ORACLE_LANE_NUMERIC) continue;
        nsum_add(&acc, p[j] * oracle_decode(v, dtype, vbase + j * d + k));
      }
      o[k] = nsum_value(&acc);
    }
  }
  free(p);
  free(cls);
  return 0;
}

int oracle_weighted_chunk_states(const void* s, const void* v, int dtype,
                                 int64_t rows, int64_t cols, int64_t d,
                                 int64_t rows_per_group, const oracle_mask* mk,
                                 int64_t chunk_cols, int64_t r0, int64_t r1,
                                 double* m, double* l, double* o) {
  if (d < 0 || rows_per_group <= 0 || rows % rows_per_group != 0) return -1;
  if (oracle_chunk_stats(s, dtype, rows, cols, mk, chunk_cols, r0, r1, m, l))
    return -1;
  const int64_t n_chunks = (cols + chunk_cols - 1) / chunk_cols;
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t prefix = oracle_valid_prefix(mk, r, cols);
    const int64_t vbase = (r / rows_per_group) * cols * d;
    for (int64_t c = 0; c < n_chunks; ++c) {
      const int64_t idx = (r - r0) * n_chunks + c;
      double* oc = o + idx * d;
      if (isnan(m[idx]) || m[idx] == -INFINITY) {
        for (int64_t k = 0; k < d; ++k) oc[k] = isnan(m[idx]) ? NAN : 0.0;
        continue;
      }
      const int64_t lo = c * chunk_cols;
      const int64_t hi = lo + chunk_cols < cols ? lo + chunk_cols : cols;
      for (int64_t k = 0; k < d; ++k) {
        nsum acc = {0.0, 0.0};
        for (int64_t j = lo; j < hi; ++j) {
          if (!lane_valid(mk, r, j, cols, prefix)) continue;
          const double x = oracle_decode(s, dtype, r * cols + j);
          if (x == -INFINITY) continue;
          nsum_add(&acc, exp(x - m[idx]) * oracle_decode(v, dtype, vbase + j * d + k));
        }
        oc[k] = nsum_value(&acc);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* The merge ("Online stable softmax", section "Derive the update for two    */
/* blocks" and "Reference summary"): m' = max(m, m2),                        */
/* l' = exp(m - m') l + exp(m2 - m') l2. The side holding the maximum has    */
/* the factor exactly 1 (the worked example's special case m2 < m keeps the  */
/* old sum unchanged), so an empty side (-inf, 0) is an exact identity and   */
/* -inf - (-inf) is never formed.                                            */
/* ------------------------------------------------------------------------ */

void oracle_merge(double m_a, double l_a, double m_b, double l_b,
                  double* m_out, double* l_out) {
  if (isnan(m_a) || isnan(m_b) || isnan(l_a) || isnan(l_b)) {
    *m_out = NAN;
    *l_out = NAN;
    return;
  }
  const double mm = m_a > m_b ? m_a : m_b;
  if (mm == -INFINITY) {
    *m_out = -INFINITY;
    *l_out = 0.0;
    return;
  }
  const double fa = (m_a == mm) ? 1.0 : exp(m_a - mm);
  const double fb = (m_b == mm) ? 1.0 : exp(m_b - mm);
  *m_out = mm;
  *l_out = fa * l_a + fb * l_b;
}

/* The weighted numerator takes the same two factors as the sum ("Online
 * stable softmax", reference summary: o' = exp(m - m') o + exp(m2 - m') o2). */
void oracle_weighted_merge(double m_a, double l_a, const double* o_a,
                           double m_b, double l_b, const double* o_b,
                           int64_t d, double* m_out, double* l_out,
                           double* o_out) {
  if (isnan(m_a) || isnan(m_b) || isnan(l_a) || isnan(l_b)) {
    *m_out = NAN;
    *l_out = NAN;
    for (int64_t k = 0; k < d; ++k) o_out[k] = NAN;
    return;
  }
  const double mm = m_a > m_b ? m_a : m_b;
  if (mm == -INFINITY) {
    *m_out = -INFINITY;
    *l_out = 0.0;
    for (int64_t k = 0; k < d; ++k) o_out[k] = 0.0;
    return;
  }
  const double fa = (m_a == mm) ? 1.0 : exp(m_a - mm);
  const double fb = (m_b == mm) ? 1.0 : exp(m_b - mm);
  *m_out = mm;
  *l_out = fa * l_a + fb * l_b;
  for (int64_t k = 0; k < d; ++k) o_out[k] = fa * o_a[k] + fb * o_b[k];
}

void oracle_merge_all(const double* m, const double* l, int64_t n,
                      double* m_out, double* l_out) {
  double am = -INFINITY, al = 0.0;
  for (int64_t i = 0; i < n; ++i) oracle_merge(am, al, m[i], l[i], &am, &al);
  *m_out = am;
  *l_out = al;
}

int oracle_merge_normalize(const void* x, int dtype, int64_t rows,
                           int64_t cols, const oracle_mask* mk,
                           const double* m, const double* l, int64_t n_chunks,
                           int64_t r0, int64_t r1, double* p,
                           uint8_t* lane_class, int32_t* row_status) {
  if (dtype < 0 || dtype > 2 || rows < 0 || cols < 0 || n_chunks < 0 ||
      r0 < 0 || r1 > rows || r0 > r1 || !mask_ok(mk))
    return -1;
  for (int64_t r = r0; r < r1; ++r) {
    double* pr = p + (r - r0) * cols;
    uint8_t* cr = lane_class + (r - r0) * cols;
    double M, L;
    oracle_merge_all(m + (r - r0) * n_chunks, l + (r - r0) * n_chunks,
                     n_chunks, &M, &L);
    int32_t st;
    if (isnan(M)) {
      set_policy_row(pr, cr, cols, NAN, ORACLE_LANE_NAN);
      st = ORACLE_ROW_POISON;
    } else if (M == -INFINITY) {
      set_policy_row(pr, cr, cols, 0.0, ORACLE_LANE_ZERO);
      st = ORACLE_ROW_EMPTY;
    } else {
      const int64_t prefix = oracle_valid_prefix(mk, r, cols);
      for (int64_t j = 0; j < cols; ++j) {
        double v = lane_valid(mk, r, j, cols, prefix)
                       ? oracle_decode(x, dtype, r * cols + j)
                       : -INFINITY;
        if (v == -INFINITY) {
          pr[j] = 0.0;
          cr[j] = ORACLE_LANE_ZERO;
        } else {
          pr[j] = exp(v - M) / L;
          cr[j] = ORACLE_LANE_NUMERIC;
        }
      }
      st = ORACLE_ROW_OK;
    }
    if (row_status) row_status[r - r0] = st;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Online recurrences, used only to check the definitions against each       */
/* other.                                                                    */
/* "Kernel visualization: online softmax", section "Online softmax":         */
/*   m_i = max(m_{i-1}, x_i), d_i = d_{i-1} e^{m_{i-1}-m_i} + e^{x_i-m_i},    */
/*   with m_0 = -inf, d_0 = 0.                                               */
/* Same page, section "Tiled version": the tile-at-a-time form.              */
/* ------------------------------------------------------------------------ */

/* e^{a - b} for a <= b, taking the factor 1 when a == b (covers -inf == -inf,
 * where the empty prefix contributes nothing). */
static double rescale(double a, double b) { return a == b ? 1.0 : exp(a - b); }

void oracle_online_elementwise(const double* x, int64_t n, double* m_trace,
                               double* d_trace) {
  double m = -INFINITY, d = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double m_new = x[i] > m ? x[i] : m;
    const double term = (x[i] == -INFINITY) ? 0.0 : rescale(x[i], m_new);
    d = d * rescale(m, m_new) + term;
    m = m_new;
    m_trace[i] = m;
    d_trace[i] = d;
  }
}

void oracle_online_tiled(const double* x, int64_t n, int64_t tile,
                         double* m_trace, double* d_trace) {
  double m = -INFINITY, d = 0.0;
  int64_t t_index = 0;
  for (int64_t t = 0; t < n; t += tile) {
    const int64_t hi = t + tile < n ? t + tile : n;
    double tile_max = -INFINITY;
    for (int64_t j = t; j < hi; ++j)
      if (x[j] > tile_max) tile_max = x[j];
    const double m_new = tile_max > m ? tile_max : m;
    /* correct the running sum, then add the new tile against m_new */
    double corrected = d * rescale(m, m_new);
    double add = 0.0;
    for (int64_t j = t; j < hi; ++j)
      if (x[j] != -INFINITY) add += rescale(x[j], m_new);
    d = corrected + add;
    m = m_new;
    m_trace[t_index] = m;
    d_trace[t_index] = d;
    ++t_index;
  }
}

/* "Online stable softmax", section "Trace an online softmax maximum change":
 * a version that forgets the rescale when the maximum moves. It is WRONG on
 * purpose and exists only so a test can show the check catches it. */
void oracle_online_no_rescale(const double* x, int64_t n, double* m_trace,
                              double* d_trace) {
  double m = -INFINITY, d = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double m_new = x[i] > m ? x[i] : m;
    const double term = (x[i] == -INFINITY) ? 0.0 : rescale(x[i], m_new);
    d = d + term;
    m = m_new;
    m_trace[i] = m;
    d_trace[i] = d;
  }
}

/* ------------------------------------------------------------------------ */
/* Log-sum-exp and log-softmax ("Softmax numerics architecture", section     */
/* "Log-sum-exp: log-probabilities without probabilities"):                  */
/* LSE = m + log(sum exp(x - m)), log_softmax_i = x_i - LSE.                  */
/* ------------------------------------------------------------------------ */

int oracle_log_softmax_rows(const void* x, int dtype, int64_t rows,
                            int64_t cols, const oracle_mask* mk, int64_t r0,
                            int64_t r1, double* lse, double* logp) {
  if (dtype < 0 || dtype > 2 || rows < 0 || cols < 0 || r0 < 0 || r1 > rows ||
      r0 > r1 || !mask_ok(mk))
    return -1;
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t prefix = oracle_valid_prefix(mk, r, cols);
    double* out = logp + (r - r0) * cols;
    int poisoned = 0;
    double m = -INFINITY;
    int64_t count = 0;
    for (int64_t j = 0; j < cols; ++j) {
      if (!lane_valid(mk, r, j, cols, prefix)) continue;
      double v = oracle_decode(x, dtype, r * cols + j);
      if (poisons(v)) poisoned = 1;
      if (v == -INFINITY || isnan(v)) continue;
      if (count == 0 || v > m) m = v;
      ++count;
    }
    if (poisoned) {
      lse[r - r0] = NAN;
      for (int64_t j = 0; j < cols; ++j) out[j] = NAN;
      continue;
    }
    if (count == 0) {
      lse[r - r0] = -INFINITY;
      for (int64_t j = 0; j < cols; ++j) out[j] = -INFINITY;
      continue;
    }
    nsum acc = {0.0, 0.0};
    for (int64_t j = 0; j < cols; ++j) {
      if (!lane_valid(mk, r, j, cols, prefix)) continue;
      double v = oracle_decode(x, dtype, r * cols + j);
      if (v == -INFINITY) continue;
      nsum_add(&acc, exp(v - m));
    }
    const double L = m + log(nsum_value(&acc));
    lse[r - r0] = L;
    for (int64_t j = 0; j < cols; ++j) {
      double v = lane_valid(mk, r, j, cols, prefix)
                     ? oracle_decode(x, dtype, r * cols + j)
                     : -INFINITY;
      out[j] = (v == -INFINITY) ? -INFINITY : v - L;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Softmax backward ("Softmax numerics architecture", section "The Jacobian, */
/* and the backward pass that never divides"): dL/dx = p * (g - g.p).        */
/* ------------------------------------------------------------------------ */

int oracle_softmax_backward_rows(const void* p, const void* g, int dtype,
                                 int64_t rows, int64_t cols, int64_t r0,
                                 int64_t r1, double* dx) {
  if (dtype < 0 || dtype > 2 || rows < 0 || cols < 0 || r0 < 0 || r1 > rows ||
      r0 > r1)
    return -1;
  for (int64_t r = r0; r < r1; ++r) {
    nsum dot = {0.0, 0.0};
    for (int64_t j = 0; j < cols; ++j)
      nsum_add(&dot, oracle_decode(g, dtype, r * cols + j) *
                         oracle_decode(p, dtype, r * cols + j));
    const double gp = nsum_value(&dot);
    for (int64_t j = 0; j < cols; ++j) {
      const double pj = oracle_decode(p, dtype, r * cols + j);
      const double gj = oracle_decode(g, dtype, r * cols + j);
      dx[(r - r0) * cols + j] = pj * (gj - gp);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Cross-entropy with logits ("Softmax numerics architecture", log-sum-exp   */
/* section: CE = LSE - x_t; Jacobian section: the fused gradient p - y with  */
/* y the one-hot target).                                                    */
/* ------------------------------------------------------------------------ */

int oracle_cross_entropy_rows(const void* x, int dtype, int64_t rows,
                              int64_t cols, const oracle_mask* mk,
                              const int32_t* target, int64_t r0, int64_t r1,
                              double* loss, double* dx) {
  if (dtype < 0 || dtype > 2 || rows < 0 || cols < 0 || r0 < 0 || r1 > rows ||
      r0 > r1 || !mask_ok(mk) || target == NULL)
    return -1;
  double* p = (double*)malloc(sizeof(double) * (size_t)(cols ? cols : 1));
  uint8_t* cls = (uint8_t*)malloc((size_t)(cols ? cols : 1));
  if (!p || !cls) {
    free(p);
    free(cls);
    return -1;
  }
  for (int64_t r = r0; r < r1; ++r) {
    double* d = dx ? dx + (r - r0) * cols : NULL;
    const int64_t t = target[r];
    if (t < 0 || t >= cols) { /* ignored row */
      loss[r - r0] = 0.0;
      if (d)
        for (int64_t j = 0; j < cols; ++j) d[j] = 0.0;
      continue;
    }
    const int32_t st = softmax_one_row(x, dtype, cols, mk, r, p, cls);
    if (st == ORACLE_ROW_POISON) {
      loss[r - r0] = NAN;
      if (d)
        for (int64_t j = 0; j < cols; ++j) d[j] = NAN;
      continue;
    }
    double at_t = -1.0; /* dx at the target lane: p_t - 1 */
    if (st == ORACLE_ROW_EMPTY || cls[t] != ORACLE_LANE_NUMERIC) {
      loss[r - r0] = INFINITY; /* the target has probability 0 */
    } else {
      /* LSE - x_t = (m - x_t) + log(l). When the target holds the maximum
       * the loss is log(1 + sum over the other lanes of exp(x_j - m)),
       * written with log1p so a confident prediction's tiny loss keeps its
       * relative precision; otherwise both terms are positive. */
      const int64_t prefix = oracle_valid_prefix(mk, r, cols);
      const double xt = oracle_decode(x, dtype, r * cols + t);
      double m = -INFINITY;
      for (int64_t j = 0; j < cols; ++j) {
        if (!lane_valid(mk, r, j, cols, prefix)) continue;
        double v = oracle_decode(x, dtype, r * cols + j);
        if (v > m) m = v;
      }
      nsum all = {0.0, 0.0}, others = {0.0, 0.0};
      for (int64_t j = 0; j < cols; ++j) {
        if (!lane_valid(mk, r, j, cols, prefix)) continue;
        double v = oracle_decode(x, dtype, r * cols + j);
        if (v == -INFINITY) continue;
        const double e = exp(v - m);
        nsum_add(&all, e);
        if (j != t) nsum_add(&others, e);
      }
      loss[r - r0] = (xt == m) ? log1p(nsum_value(&others))
                               : (m - xt) + log(nsum_value(&all));
      /* p_t - 1 = -(sum of the other lanes' p): the same number, without the
       * cancellation of 1 - p_t when the target holds almost all the mass */
      at_t = -(nsum_value(&others) / nsum_value(&all));
    }
    if (d) {
      for (int64_t j = 0; j < cols; ++j) d[j] = (j == t) ? at_t : p[j];
    }
  }
  free(p);
  free(cls);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Output rounding: nearest-even with gradual underflow.                     */
/* ------------------------------------------------------------------------ */

uint32_t oracle_round_f32_bits(double v) {
  if (isnan(v)) return 0x7FC00000u;
  float f = (float)v; /* C conversion: current rounding mode, nearest-even */
  uint32_t w;
  memcpy(&w, &f, sizeof w);
  return w;
}

/* Round |v| to a format with `mant` stored fraction bits, minimum normal
 * exponent emin, and exponent bias, returning the magnitude bits. Values at
 * or above `overflow` round to infinity. */
static uint32_t round_small_format(double a, int mant, int emin, int bias,
                                   double overflow, uint32_t inf_bits) {
  if (a >= overflow) return inf_bits;
  if (a < ldexp(1.0, emin)) {
    /* subnormal range: quantum 2^(emin - mant) */
    double q = nearbyint(ldexp(a, mant - emin));
    return (uint32_t)q; /* q == 2^mant becomes the smallest normal */
  }
  int E;
  frexp(a, &E); /* a = f * 2^E, f in [0.5, 1): unbiased exponent E - 1 */
  double q = nearbyint(ldexp(a, mant + 1 - E)); /* in [2^mant, 2^(mant+1)] */
  uint32_t biased = (uint32_t)(E - 1 + bias);
  return (biased << mant) + ((uint32_t)q - (1u << mant));
}

uint16_t oracle_round_f16_bits(double v) {
  if (isnan(v)) return 0x7E00;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  /* largest finite 65504; the midpoint to 2^16 is 65520 */
  return sign | (uint16_t)round_small_format(a, 10, -14, 15, 65520.0, 0x7C00);
}

uint16_t oracle_round_bf16_bits(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  /* largest finite (2 - 2^-7) 2^127; the midpoint to 2^128 is (2 - 2^-8) 2^127 */
  double overflow = ldexp(2.0 - ldexp(1.0, -8), 127);
  return sign | (uint16_t)round_small_format(a, 7, -126, 127, overflow, 0x7F80);
}

void oracle_encode(const double* p, int64_t n, int dtype, void* out) {
  for (int64_t i = 0; i < n; ++i) {
    if (dtype == ORACLE_F32) {
      uint32_t w = oracle_round_f32_bits(p[i]);
      memcpy((char*)out + 4 * i, &w, 4);
    } else {
      uint16_t h = dtype == ORACLE_F16 ? oracle_round_f16_bits(p[i])
                                       : oracle_round_bf16_bits(p[i]);
      memcpy((char*)out + 2 * i, &h, 2);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* The CPU baseline: the same three-pass rows, encoded, over host threads.   */
/* ------------------------------------------------------------------------ */

typedef struct {
  const void* x;
  void* y;
  int dtype;
  int64_t rows, cols, r0, r1;
  const oracle_mask* mk;
  int rc;
} mt_job;

static void* mt_worker(void* arg) {
  mt_job* jb = (mt_job*)arg;
  const int64_t cols = jb->cols;
  double* p = (double*)malloc(sizeof(double) * (size_t)(cols ? cols : 1));
  uint8_t* c = (uint8_t*)malloc((size_t)(cols ? cols : 1));
  if (!p || !c) {
    jb->rc = -1;
    free(p);
    free(c);
    return NULL;
  }
  const size_t esz = jb->dtype == ORACLE_F32 ? 4 : 2;
  for (int64_t r = jb->r0; r < jb->r1; ++r) {
    softmax_one_row(jb->x, jb->dtype, cols, jb->mk, r, p, c);
    oracle_encode(p, cols, jb->dtype, (char*)jb->y + (size_t)r * cols * esz);
  }
  free(p);
  free(c);
  jb->rc = 0;
  return NULL;
}

int oracle_softmax_rows_encode_mt(const void* x, void* y, int dtype,
                                  int64_t rows, int64_t cols,
                                  const oracle_mask* mk, int threads) {
  if (dtype < 0 || dtype > 2 || rows < 0 || cols < 0 || !mask_ok(mk) ||
      threads < 1)
    return -1;
  if (threads > rows) threads = rows > 0 ? (int)rows : 1;
  mt_job* jobs = (mt_job*)calloc((size_t)threads, sizeof(mt_job));
  pthread_t* tid = (pthread_t*)calloc((size_t)threads, sizeof(pthread_t));
  if (!jobs || !tid) {
    free(jobs);
    free(tid);
    return -1;
  }
  int rc = 0;
  for (int t = 0; t < threads; ++t) {
    jobs[t] = (mt_job){x, y, dtype, rows, cols, rows * t / threads,
                       rows * (t + 1) / threads, mk, -1};
    if (pthread_create(&tid[t], NULL, mt_worker, &jobs[t]) != 0) {
      jobs[t].rc = -1;
      tid[t] = 0;
      rc = -1;
    }
  }
  for (int t = 0; t < threads; ++t) {
    if (tid[t]) pthread_join(tid[t], NULL);
    if (jobs[t].rc != 0) rc = -1;
  }
  free(jobs);
  free(tid);
  return rc;
}
