/*
 * oracle.h — plain, slow, double-precision CPU reference for batched
 * row-wise softmax, chunk summaries and their merge, and for the entry
 * points built on them (log-softmax, softmax backward, cross-entropy,
 * softmax-weighted value sums).
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library. The product path (the HIP
 * library and its Python binding) never includes, links or calls it, and
 * this code includes nothing from the product path.
 *
 * Every routine follows a definition stated on the source pages:
 *  - "Softmax numerics architecture", section "The max-subtraction identity":
 *    softmax(x - c) = softmax(x); with c = max(x) every exponential is in
 *    (0, 1] and the sum is in [1, N].
 *  - "Kernel visualization: online softmax", section "Overview of safe
 *    softmax" and "The naive version: three passes": max, then the sum of
 *    shifted exponentials, then divide.
 *  - "Online stable softmax", section "Derive the update for two blocks" and
 *    "Reference summary": the (m, l) merge rule.
 *  - "Stable softmax: keep the normalizer consistent as tiles arrive", the
 *    paragraph on masks, and "Online stable softmax", section "Masks, empty
 *    rows, and precision": the mask / empty-row / inf / NaN contract.
 *  - "Softmax numerics architecture", sections on log-sum-exp and on the
 *    Jacobian: log-softmax, cross-entropy with logits and its gradient, the
 *    softmax vector-Jacobian product.
 *  - "Online stable softmax", section on the weighted-value numerator and
 *    "Reference summary", and "Softmax numerics architecture", tiled
 *    attention: the softmax-weighted value sums and their (m, l, o) states.
 *
 * All arithmetic is IEEE double, in the order written, compiled without
 * floating-point contraction. Inputs are decoded exactly; outputs are rounded
 * once, to nearest-even with gradual underflow.
 */
#ifndef NSO_ORACLE_H
#define NSO_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats (x and y share one). */
#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2

/* Mask kinds. A lane j of row r is "valid" when:
 *   NONE      : always
 *   VALID_LEN : j < clamp(valid_len[r], 0, cols)
 *   CAUSAL    : j < clamp((r mod period) + 1 + offset, 0, cols)
 *   KEEP      : keep[r*cols + j] != 0                                       */
#define ORACLE_MASK_NONE 0
#define ORACLE_MASK_VALID_LEN 1
#define ORACLE_MASK_CAUSAL 2
#define ORACLE_MASK_KEEP 3

/* Lane classes written beside every reference value. */
#define ORACLE_LANE_NUMERIC 0 /* a probability; may underflow numerically     */
#define ORACLE_LANE_ZERO 1    /* policy +0.0: masked, -inf, or an empty row   */
#define ORACLE_LANE_NAN 2     /* policy NaN: the row holds +inf or NaN        */

/* Row status codes. */
#define ORACLE_ROW_OK 0
#define ORACLE_ROW_EMPTY 1
#define ORACLE_ROW_POISON 2

typedef struct {
  int kind;
  const int32_t* valid_len; /* [rows], indexed by the global row */
  int64_t causal_period;
  int64_t causal_offset;
  const uint8_t* keep; /* [rows * cols] */
} oracle_mask;

/* Exact decode of element i of x into double. */
double oracle_decode(const void* x, int dtype, int64_t i);

/* Number of valid lanes of row r, or -1 for the KEEP kind (arbitrary lanes). */
int64_t oracle_valid_prefix(const oracle_mask* mk, int64_t r, int64_t cols);

/* Three-pass stable softmax of rows [r0, r1) of x ([rows, cols], row-major).
 * p and lane_class have (r1 - r0) * cols entries; row_status (may be NULL)
 * has r1 - r0. p holds the double reference value (NaN on a poisoned row).
 * Returns 0, or -1 on bad arguments.                                        */
int oracle_softmax_rows(const void* x, int dtype, int64_t rows, int64_t cols,
                        const oracle_mask* mk, int64_t r0, int64_t r1,
                        double* p, uint8_t* lane_class, int32_t* row_status);

/* Per-chunk summaries of rows [r0, r1): chunk c covers columns
 * [c*chunk_cols, min((c+1)*chunk_cols, cols)). m and l have
 * (r1 - r0) * n_chunks entries. Poisoned chunk: (NaN, NaN).
 * Chunk with no finite valid lane: (-inf, 0).                               */
int oracle_chunk_stats(const void* x, int dtype, int64_t rows, int64_t cols,
                       const oracle_mask* mk, int64_t chunk_cols, int64_t r0,
                       int64_t r1, double* m, double* l);

/* The two-summary merge: (m_a, l_a) (+) (m_b, l_b). */
void oracle_merge(double m_a, double l_a, double m_b, double l_b,
                  double* m_out, double* l_out);

/* Fold a row's n summaries left to right with oracle_merge. */
void oracle_merge_all(const double* m, const double* l, int64_t n,
                      double* m_out, double* l_out);

/* Merge each row's chunk summaries, then write p = exp(x - M) / L for valid
 * finite lanes. Policy: any poisoned summary -> NaN row; every summary empty
 * -> zero row. m and l are [(r1 - r0) * n_chunks].                          */
int oracle_merge_normalize(const void* x, int dtype, int64_t rows,
                           int64_t cols, const oracle_mask* mk,
                           const double* m, const double* l, int64_t n_chunks,
                           int64_t r0, int64_t r1, double* p,
                           uint8_t* lane_class, int32_t* row_status);

/* Online recurrences over a double vector, for self-checks. The traces hold
 * the state after each element (elementwise) or after each tile (tiled).    */
void oracle_online_elementwise(const double* x, int64_t n, double* m_trace,
                               double* d_trace);
void oracle_online_tiled(const double* x, int64_t n, int64_t tile,
                         double* m_trace, double* d_trace);
/* Deliberately wrong: never rescales the running sum (a negative control). */
void oracle_online_no_rescale(const double* x, int64_t n, double* m_trace,
                              double* d_trace);

/* Log-sum-exp and log-softmax of rows [r0, r1): lse has r1 - r0 entries,
 * logp has (r1 - r0) * cols (masked lanes -inf; empty row: lse -inf, lanes
 * -inf; poisoned row: NaN).                                                 */
int oracle_log_softmax_rows(const void* x, int dtype, int64_t rows,
                            int64_t cols, const oracle_mask* mk, int64_t r0,
                            int64_t r1, double* lse, double* logp);

/* Softmax vector-Jacobian product for rows [r0, r1):
 * dx_j = p_j * (g_j - sum_k g_k p_k), p and g given in the element format.  */
int oracle_softmax_backward_rows(const void* p, const void* g, int dtype,
                                 int64_t rows, int64_t cols, int64_t r0,
                                 int64_t r1, double* dx);

/* Cross-entropy with logits and its gradient for rows [r0, r1):
 *   loss_r = LSE_r - x[r, t_r],   dx[r, j] = p[r, j] - [j == t_r].
 * Policy: t_r outside [0, cols) ignores the row (loss 0, dx 0); a poisoned
 * row gives NaN loss and dx; an empty row, or a target lane that is masked
 * or -inf, gives loss +inf (p_t = 0) with dx = p - onehot(t). dx may be
 * NULL; loss has r1 - r0 entries, dx (r1 - r0) * cols.                      */
int oracle_cross_entropy_rows(const void* x, int dtype, int64_t rows,
                              int64_t cols, const oracle_mask* mk,
                              const int32_t* target, int64_t r0, int64_t r1,
                              double* loss, double* dx);

/* Softmax-weighted sum of value vectors ("Online stable softmax", section
 * on the weighted-value numerator; "Softmax numerics architecture", section
 * on tiled attention): for rows [r0, r1),
 *   out[r, k] = sum_j p[r, j] * v[g, j, k],   g = r / rows_per_group,
 * p the three-pass softmax of row r under the mask. s is [rows, cols], v is
 * [rows / rows_per_group, cols, d] and shares s's element format; out has
 * (r1 - r0) * d entries. Policy: a poisoned row gives NaN, an empty row 0.
 * row_status (may be NULL) has r1 - r0 entries. rows must be a multiple of
 * rows_per_group.                                                           */
int oracle_softmax_weighted_rows(const void* s, const void* v, int dtype,
                                 int64_t rows, int64_t cols, int64_t d,
                                 int64_t rows_per_group, const oracle_mask* mk,
                                 int64_t r0, int64_t r1, double* out,
                                 int32_t* row_status);

/* Per-chunk online states (m, l, o) of rows [r0, r1): chunk c covers
 * columns [c*chunk_cols, min((c+1)*chunk_cols, cols)); m and l as in
 * oracle_chunk_stats, o[k] = sum over the chunk's finite valid lanes of
 * exp(s_j - m) v[g, j, k]. m, l have (r1 - r0) * n_chunks entries, o has
 * (r1 - r0) * n_chunks * d. Poisoned chunk: (NaN, NaN, NaN...); chunk with
 * no finite valid lane: (-inf, 0, 0...).                                    */
int oracle_weighted_chunk_states(const void* s, const void* v, int dtype,
                                 int64_t rows, int64_t cols, int64_t d,
                                 int64_t rows_per_group, const oracle_mask* mk,
                                 int64_t chunk_cols, int64_t r0, int64_t r1,
                                 double* m, double* l, double* o);

/* The state merge (m_a, l_a, o_a) (+) (m_b, l_b, o_b): the (m, l) rule of
 * oracle_merge, and o' = f_a o_a + f_b o_b with the same factors.          */
void oracle_weighted_merge(double m_a, double l_a, const double* o_a,
                           double m_b, double l_b, const double* o_b,
                           int64_t d, double* m_out, double* l_out,
                           double* o_out);

/* Rounding of a double to an element format, to nearest-even with gradual
 * underflow. NaN becomes the canonical quiet NaN (f32 0x7FC00000, f16 0x7E00,
 * bf16 0x7FC0).                                                             */
uint32_t oracle_round_f32_bits(double v);
uint16_t oracle_round_f16_bits(double v);
uint16_t oracle_round_bf16_bits(double v);
/* Round n doubles into out (element format dtype). */
void oracle_encode(const double* p, int64_t n, int dtype, void* out);

/* Multi-threaded three-pass softmax writing the element format directly: the
 * CPU baseline. Rows are split into contiguous blocks over `threads` threads.
 * Returns 0 on success.                                                     */
int oracle_softmax_rows_encode_mt(const void* x, void* y, int dtype,
                                  int64_t rows, int64_t cols,
                                  const oracle_mask* mk, int threads);

#ifdef __cplusplus
}
#endif
#endif
