/*
 * smx.h — C ABI of the MI355X (gfx950) row-softmax library.
 *
 * Batched row-wise stable softmax computed by online normalization:
 *   p_j = exp(x_j - m) / l,  m = max_j x_j,  l = sum_j exp(x_j - m)
 * over the valid lanes of each row of a row-major [rows, cols] tensor.
 *
 * Sources (web pages; section names as on the pages):
 *  - "Softmax numerics architecture", section "The max-subtraction identity,
 *    and why it is exact": shifting by the row maximum keeps every
 *    exponential in (0, 1] and the sum in [1, N].
 *  - Same page, section "Why the accumulator is fp32 even when the inputs are
 *    not": bf16/fp16 inputs keep an fp32 running max and accumulator.
 *  - "Online stable softmax", sections "Derive the update for two blocks" and
 *    "Reference summary": a block is summarized by (m, l); two summaries
 *    merge as m' = max(m, m2), l' = exp(m - m') l + exp(m2 - m') l2.
 *  - "Stable softmax: keep the normalizer consistent as tiles arrive", the
 *    paragraphs on masks and on fused rows: the mask contract, and a row is
 *    read once when it fits on chip, otherwise with a counted reread.
 *
 * Contract for every call
 *  - All pointers except `mask` and the mask descriptor itself are DEVICE
 *    pointers on the current HIP device, allocated and owned by the caller.
 *    The mask descriptor struct is read on the host during the call.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *    the default stream). Results are valid once the stream has synchronized.
 *    The library never synchronizes the host and keeps no device memory
 *    between calls, except the fixed scratch of softmax_rows_noalloc.
 *  - Return value: SMX_OK (0) or an SMX_E* code; smx_last_error() then
 *    returns a message (thread-local, valid until the next call on the same
 *    thread). Invalid arguments are rejected before anything is enqueued.
 *  - rows == 0 or cols == 0 is a successful no-op.
 *  - x == y (exact aliasing) is allowed; partial overlap is SMX_EINVAL.
 *  - Any pointer alignment is accepted; 16-byte aligned x and y with
 *    cols * element_size a multiple of 16 take the 128-bit vector path.
 *  - Results are deterministic: the same inputs give bitwise the same output.
 *
 * Data policy (values are never errors)
 *  - Masked lanes contribute nothing and are written as +0.0. A valid lane
 *    holding -inf behaves like a masked lane.
 *  - A row with no valid finite lane (cols == 0, valid length 0, every lane
 *    masked, or every valid lane -inf) is written as all +0.0; no
 *    -inf - (-inf) is ever formed.
 *  - A row with +inf or NaN (any sign, quiet or signalling) in a VALID lane is
 *    written as the canonical quiet NaN in every lane: f32 0x7FC00000,
 *    f16 0x7E00, bf16 0x7FC0. +inf or NaN in a masked lane is ignored.
 *  - Accumulation is fp32 for every element type; outputs are rounded to
 *    nearest-even with gradual underflow (subnormals are kept).
 */
#ifndef SMX_H
#define SMX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library exports exactly the functions declared here. */
#if defined(__GNUC__) || defined(__clang__)
#define SMX_API __attribute__((visibility("default")))
#else
#define SMX_API
#endif

/* Status codes. */
#define SMX_OK 0
#define SMX_EINVAL 1 /* a bad argument; nothing was enqueued            */
#define SMX_EHIP 2   /* the HIP runtime reported an error               */

/* Element type of x and y (they share one); accumulation is always fp32. */
typedef enum { SMX_F32 = 0, SMX_F16 = 1, SMX_BF16 = 2 } smx_dtype;

/* Mask kinds. Lane j of row r is valid when:
 *   SMX_MASK_NONE      : always;
 *   SMX_MASK_VALID_LEN : j < clamp(valid_len[r], 0, cols);
 *   SMX_MASK_CAUSAL    : j < clamp((r mod causal_period) + 1 + causal_offset,
 *                                  0, cols)  (row i of each period keeps
 *                                  columns 0..i+causal_offset);
 *   SMX_MASK_KEEP_BYTES: keep[r * cols + j] != 0.
 * An out-of-range valid length is clamped, not an error. */
typedef enum {
  SMX_MASK_NONE = 0,
  SMX_MASK_VALID_LEN = 1,
  SMX_MASK_CAUSAL = 2,
  SMX_MASK_KEEP_BYTES = 3
} smx_mask_kind;

typedef struct {
  smx_mask_kind kind;
  const int32_t* valid_len; /* VALID_LEN: device [rows]                      */
  int64_t causal_period;    /* CAUSAL: > 0                                   */
  int64_t causal_offset;    /* CAUSAL: any value                             */
  const uint8_t* keep;      /* KEEP_BYTES: device [rows, cols], row-major    */
} smx_mask;                 /* a NULL descriptor pointer means SMX_MASK_NONE */

/* A chunk summary: m is the chunk's maximum over valid finite lanes and
 * l = sum exp(x_j - m) over them (l in [1, lanes]). An empty chunk is
 * (-inf, 0); a chunk holding +inf or NaN in a valid lane is (NaN, NaN). */
typedef struct {
  float m;
  float l;
} smx_stat;

/* Kernel paths. */
typedef enum {
  SMX_PATH_AUTO = 0,  /* chosen from the row size and the row count        */
  SMX_PATH_WAVE = 1,  /* one wave64 per row, the row held in registers     */
  SMX_PATH_LDS = 2,   /* one workgroup per row, the row staged in LDS and
                         read from HBM once: up to 32 KiB held in registers,
                         up to 152 KiB kept in LDS for all three passes    */
  SMX_PATH_SPLIT = 3  /* chunk summaries, then merge + normalize (2 reads) */
} smx_path;

/* softmax_rows — y[r, :] = softmax of the valid lanes of x[r, :].
 *   x, y  : device [rows, cols] row-major, element type dtype.
 *   valid_len_or_mask : host pointer to a mask descriptor, or NULL.
 *   stream: hipStream_t.
 * Rows of at most 4 KiB take one wave each. Rows up to 152 KiB with 16-byte
 * aligned x and y and cols * element size a multiple of 16 are read once on
 * the LDS path ("Stable softmax: keep the normalizer consistent as tiles
 * arrive", paragraph on fused rows: a row that fits on chip is read once).
 * Longer rows, and unaligned ones the wave path cannot hold, go through the
 * split path (the row read twice), which takes its summary workspace
 * (rows * ceil(cols / chunk) * 8 bytes, plus 8 bytes per row when a row has
 * more than 1024 chunks and its summaries are merged once per row first)
 * with a stream-ordered allocation and frees it on the same stream. That
 * allocation and its release cost the host some 15 to 20 us per call, which
 * dominates small split-path calls; softmax_rows_noalloc has no such cost. */
SMX_API int softmax_rows(const void* x, void* y, int64_t rows, int64_t cols,
                 smx_dtype dtype, const smx_mask* valid_len_or_mask,
                 void* stream);

/* Bytes of device scratch softmax_rows_noalloc holds per device. */
#define SMX_NOALLOC_SCRATCH_BYTES (4 * 1024 * 1024)

/* softmax_rows_noalloc — softmax_rows_path for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation. It calls no allocator (no hipMalloc,
 * hipMallocAsync or hipFree, and none through another library).
 *  - The split path keeps its chunk summaries in a static device array of
 *    SMX_NOALLOC_SCRATCH_BYTES bytes that the library holds on each device
 *    it runs on until the process ends. A split-path call whose summaries
 *    need more (rows * ceil(cols / chunk) * 8 bytes, plus rows * 8 when a
 *    row has more than 1024 chunks) is SMX_EINVAL before anything is
 *    enqueued: pass a larger chunk_cols, or use softmax_rows_path.
 *  - The wave and LDS paths use no scratch.
 *  - Every call on one device shares that device's array, which keeps the
 *    last call's contents (nothing in it needs clearing: each call writes
 *    every summary before reading it). Calls that overlap in time on one
 *    device (on two streams, or from two host threads) race on it and must
 *    be ordered by the caller.
 *  - The device address of the array is looked up on the first call made
 *    with that device current; later calls reuse it.
 * Arguments, paths, results (bitwise those of softmax_rows_path) and errors
 * otherwise as softmax_rows_path. */
SMX_API int softmax_rows_noalloc(const void* x, void* y, int64_t rows, int64_t cols,
                                 smx_dtype dtype, const smx_mask* valid_len_or_mask,
                                 smx_path path, int64_t chunk_cols, void* stream);

/* softmax_rows_path — softmax_rows with the kernel path forced (AUTO picks
 * as softmax_rows does). chunk_cols applies to SMX_PATH_SPLIT (0 = the
 * default). A path that cannot hold the row (WAVE above its register budget,
 * LDS above its LDS budget) is SMX_EINVAL. */
SMX_API int softmax_rows_path(const void* x, void* y, int64_t rows, int64_t cols,
                      smx_dtype dtype, const smx_mask* valid_len_or_mask,
                      smx_path path, int64_t chunk_cols, void* stream);

/* The path softmax_rows takes for a shape (no device access). */
SMX_API smx_path softmax_select_path(int64_t rows, int64_t cols, smx_dtype dtype);

/* softmax_row_stats — per-chunk summaries ("Stable softmax: keep the
 * normalizer consistent as tiles arrive", block-merge paragraph).
 *   chunk_cols: > 0; chunk c covers columns [c*chunk_cols,
 *               min((c+1)*chunk_cols, cols)).
 *   stats: device [rows][n_chunks], n_chunks = ceil(cols / chunk_cols). */
SMX_API int softmax_row_stats(const void* x, int64_t rows, int64_t cols,
                      smx_dtype dtype, const smx_mask* valid_len_or_mask,
                      int64_t chunk_cols, smx_stat* stats, void* stream);

/* softmax_merge_normalize — merges each row's n_chunks summaries with the
 * (m, l) rule ("Online stable softmax", "Reference summary"; the side holding
 * the maximum keeps factor 1, so (-inf, 0) is an exact identity), then
 * rereads x and writes y = exp(x - M) / L over valid finite lanes.
 * Any (NaN, NaN) summary makes a NaN row; all-empty summaries a zero row.
 *   stats: device [rows][n_chunks], as written by softmax_row_stats or by the
 *          caller (e.g. summaries exchanged between devices);
 *   n_chunks must equal ceil(cols / chunk_cols).
 * Up to 1024 chunks per row, every chunk's workgroup merges its row's
 * summaries itself (no workspace). Beyond that each row's summaries are first
 * merged once, bitwise as the workgroups would merge them, into a
 * stream-ordered workspace of rows * 8 bytes, so the summary reads grow
 * linearly with n_chunks. */
SMX_API int softmax_merge_normalize(const void* x, void* y, int64_t rows, int64_t cols,
                            smx_dtype dtype, const smx_mask* valid_len_or_mask,
                            int64_t chunk_cols, const smx_stat* stats,
                            int64_t n_chunks, void* stream);

/* log_softmax_rows — log-probabilities and the per-row log-sum-exp
 * ("Softmax numerics architecture", section on log-sum-exp: LSE = m +
 * log(sum exp(x - m)), log_softmax = x - LSE; going to log space directly
 * avoids log(0) of an underflowed probability).
 *   y  : device [rows, cols] in dtype, y[r, j] = x[r, j] - LSE_r over valid
 *        finite lanes, -inf on masked and -inf lanes; may be NULL when only
 *        the LSE is wanted.
 *   lse: device float [rows], LSE_r in fp32; may be NULL (not both NULL).
 * Policy: an empty or fully masked row gives LSE = -inf and y = -inf in
 * every lane; a poisoned row (+inf/NaN in a valid lane) gives the canonical
 * NaN in lse and in every lane of y. Same paths, alignment rules, errors and
 * stream semantics as softmax_rows; lse must not overlap x or y. */
SMX_API int log_softmax_rows(const void* x, void* y, float* lse, int64_t rows, int64_t cols, smx_dtype dtype,
                     const smx_mask* valid_len_or_mask, void* stream);

/* log_softmax_rows with the kernel path forced, as softmax_rows_path. */
SMX_API int log_softmax_rows_path(const void* x, void* y, float* lse, int64_t rows, int64_t cols, smx_dtype dtype,
                          const smx_mask* valid_len_or_mask, smx_path path, int64_t chunk_cols, void* stream);

/* softmax_cross_entropy_rows — cross-entropy with logits and its fused
 * gradient ("Softmax numerics architecture": log-sum-exp section, CE =
 * LSE - x_t; Jacobian section, the gradient p - y with y the one-hot target,
 * which never divides by a probability).
 *   x     : device [rows, cols] logits;
 *   target: device int32 [rows]; a target outside [0, cols) ignores its row;
 *   loss  : device float [rows], loss_r = LSE_r - x[r, t_r];
 *   dx    : device [rows, cols] in dtype, dx = softmax(x) - onehot(t), or
 *           NULL for the loss alone; dx may equal x (in place).
 * Policy: an ignored row has loss 0 and dx 0; a poisoned row (+inf/NaN in a
 * valid lane) has loss NaN and a NaN dx row; an empty row, or a target lane
 * that is masked or -inf, has loss +inf with dx = p - onehot(t) (p = 0 on an
 * empty row). When the target holds the row maximum the loss is computed as
 * log1p of the other lanes' shifted sum, and dx_t as -(others / sum), so a
 * confident prediction keeps full relative precision. Paths, masks, errors
 * and streams as softmax_rows; the split path's workspace adds 4 bytes per
 * row. loss must not overlap x or dx. */
SMX_API int softmax_cross_entropy_rows(const void* x, const int32_t* target, float* loss, void* dx, int64_t rows,
                                       int64_t cols, smx_dtype dtype, const smx_mask* valid_len_or_mask,
                                       void* stream);

/* softmax_cross_entropy_rows with the kernel path forced. */
SMX_API int softmax_cross_entropy_rows_path(const void* x, const int32_t* target, float* loss, void* dx,
                                            int64_t rows, int64_t cols, smx_dtype dtype,
                                            const smx_mask* valid_len_or_mask, smx_path path, int64_t chunk_cols,
                                            void* stream);

/* softmax_weighted_rows — softmax-weighted sums of value vectors, the
 * attention output for given scores ("Online stable softmax", section on the
 * weighted-value numerator: besides m and l each row carries the numerator
 * o = sum_j exp(s_j - m) V_j, rescaled by the same factor as l when the
 * maximum moves; "Softmax numerics architecture", tiled attention: the
 * output is o / l):
 *   out[r, k] = sum_j softmax(s[r])_j * v[r / rows_per_group, j, k].
 *   s  : device [rows, cols] scores in dtype (SMX_F16 or SMX_BF16), under
 *        the mask exactly as softmax_rows; 16-byte aligned, cols % 8 == 0,
 *        cols <= 2^30;
 *   v  : device [rows / rows_per_group, cols, d] values in dtype, one matrix
 *        per group of rows_per_group consecutive rows; 16-byte aligned;
 *        expected finite (a non-finite value can reach any row of its group
 *        whose block of columns covers it);
 *   out: device [rows, d] in dtype, 8-byte aligned, overlapping neither s
 *        nor v;
 *   d  : 32, 64 or 128; rows must be a multiple of rows_per_group.
 * The running state is fp32. The weights p enter the matrix cores as a
 * high and a low 16-bit part (about 16 significant bits); the values enter
 * exactly; products accumulate in fp32. Groups of at most 4 rows (or of at
 * most 8 when there are fewer than 256 groups) take the key split of
 * softmax_weighted_states and softmax_weighted_merge instead (fp32 on the
 * vector ALUs), with a stream-ordered workspace; its key chunk grows (up to
 * 2048 keys) until a row has at most 16384 chunk states, and rows of more
 * than 2^25 keys stay on the matrix cores.
 * Policy: a poisoned row (+inf/NaN in a valid lane) gives the canonical NaN
 * in every component; an empty or fully masked row gives zeros. SMX_F32,
 * other widths, misalignment and overlap are SMX_EINVAL; rows = 0 is a
 * no-op. Asynchronous on stream. */
SMX_API int softmax_weighted_rows(const void* s, const void* v, void* out, int64_t rows, int64_t cols, int64_t d,
                                  int64_t rows_per_group, smx_dtype dtype, const smx_mask* valid_len_or_mask,
                                  void* stream);

/* softmax_weighted_states — the weighted sums split along the keys: one
 * online state per (row, chunk of keys) ("Online stable softmax", section on
 * the weighted numerator: a block carries (m, l, o) with
 * o = sum_j exp(s_j - m) V_j; "Softmax numerics architecture", tiled
 * attention, where blocks of keys are visited in turn).
 *   s, v, rows, cols, d, rows_per_group, dtype, mask: as softmax_weighted_rows;
 *   chunk_cols: in [1, 2048]; chunk c covers keys [c*chunk_cols,
 *               min((c+1)*chunk_cols, cols)), n_chunks = ceil(cols / chunk_cols);
 *   ml: device float [rows][n_chunks][2]: m, the chunk's maximum over valid
 *       finite scores (exact), and l = sum exp(s_j - m) over them;
 *   o:  device float [rows][n_chunks][d]: sum exp(s_j - m) v[r / rows_per_group, j, k].
 * An empty chunk is m = -inf, l = 0, o = 0; a chunk with +inf or NaN in a
 * valid lane is NaN in m, l and o. The state is fp32 and computed on the
 * vector ALUs (this split serves groups of few rows and many keys). ml and o
 * must overlap neither each other nor s or v. Asynchronous on stream. */
SMX_API int softmax_weighted_states(const void* s, const void* v, int64_t rows, int64_t cols, int64_t d,
                                    int64_t rows_per_group, smx_dtype dtype, const smx_mask* valid_len_or_mask,
                                    int64_t chunk_cols, float* ml, float* o, void* stream);

/* softmax_weighted_merge — folds each row's n_chunks states by the merge
 * rule ("Online stable softmax", derive the update for two blocks and the
 * weighted numerator: M = max m_c; l and o take the same factor
 * exp(m_c - M), exactly 1 on the side holding the maximum, so an empty state
 * is an identity) and writes out[r, k] = O_k / L in dtype (SMX_F16 or
 * SMX_BF16), rounded to nearest even.
 *   ml, o: as softmax_weighted_states wrote them (or any states of that
 *          layout, e.g. gathered from several devices);
 *   out:   device [rows, d]; n_chunks <= 16384.
 * A NaN state (or m = +inf) makes the row the canonical NaN; a row whose
 * states are all empty is +0.0. Chunks are folded in order, so results are
 * deterministic. softmax_weighted_rows takes this split (states in a
 * stream-ordered workspace of rows * n_chunks * (d + 2) * 4 bytes, then this
 * merge) for groups of few rows. */
SMX_API int softmax_weighted_merge(const float* ml, const float* o, int64_t rows, int64_t n_chunks, int64_t d,
                                   smx_dtype dtype, void* out, void* stream);

/* softmax_backward_rows — the vector-Jacobian product of the softmax
 * ("Softmax numerics architecture", section on the Jacobian and the backward
 * pass: J = diag(p) - p p^T is never formed; dx = p * (g - g.p)).
 *   p  : device [rows, cols], a softmax output (masked lanes 0);
 *   g  : device [rows, cols], the gradient with respect to p;
 *   dx : device [rows, cols], dx[r, j] = p[r, j] * (g[r, j] - sum_k g[r, k] p[r, k]).
 * All three share dtype; the dot product accumulates in compensated fp32. dx
 * may equal p or g exactly (in place); partial overlap is SMX_EINVAL. A NaN
 * in a row's p or g makes that row's dx the canonical NaN. Long rows take two
 * passes (per-chunk partial dot products in a stream-ordered workspace of
 * rows * ceil(cols / chunk) * 8 bytes, plus 8 bytes per row when a row has
 * more than 1024 chunks and its partials are summed once per row first). */
SMX_API int softmax_backward_rows(const void* p, const void* g, void* dx, int64_t rows, int64_t cols,
                                  smx_dtype dtype, void* stream);

/* softmax_backward_rows with the path forced: SMX_PATH_WAVE (one wave per
 * row), SMX_PATH_LDS (one workgroup per row), SMX_PATH_SPLIT (two passes). */
SMX_API int softmax_backward_rows_path(const void* p, const void* g, void* dx, int64_t rows, int64_t cols,
                                       smx_dtype dtype, smx_path path, int64_t chunk_cols, void* stream);

/* The chunk width softmax_rows uses on the split path (a tuning hint). */
SMX_API int64_t softmax_default_chunk_cols(int64_t rows, int64_t cols,
                                   smx_dtype dtype);

/* A plain streaming copy of `bytes` bytes from x to y (device pointers, both
 * 16-byte aligned, bytes a multiple of 16, the two ranges disjoint), with
 * nontemporal 16-byte accesses. It is no step of the softmax: it measures the
 * HBM rate a bare copy reaches on a footprint, the reference against which
 * the row kernels' effective bandwidth is read. SMX_EINVAL on a bad size,
 * alignment, NULL pointer or overlap; bytes = 0 is a no-op. */
SMX_API int smx_stream_copy(const void* x, void* y, int64_t bytes, void* stream);

/* Message for the last nonzero status on this thread ("" if none). */
SMX_API const char* smx_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SMX_H */
