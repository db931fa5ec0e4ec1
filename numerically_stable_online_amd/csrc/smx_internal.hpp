// smx_internal.hpp — what the host dispatcher and the kernel files share:
// argument bundles, constants and the launchers each kernel file defines.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smx.h"

namespace smx {

constexpr int kF32 = SMX_F32;
constexpr int kF16 = SMX_F16;
constexpr int kBF16 = SMX_BF16;

constexpr int kMaskNone = SMX_MASK_NONE;
constexpr int kMaskValidLen = SMX_MASK_VALID_LEN;
constexpr int kMaskCausal = SMX_MASK_CAUSAL;
constexpr int kMaskKeep = SMX_MASK_KEEP_BYTES;

// Workgroup size of every kernel: four wave64s.
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

struct MaskArgs {
  int kind;
  const int32_t* valid_len;
  int64_t period;
  int64_t offset;
  const uint8_t* keep;
};

struct RowArgs {
  const char* x;
  char* y;                // may be null (log-sum-exp only, loss only)
  float* lse;             // per-row log-sum-exp, or null
  const int32_t* target;  // cross-entropy: per-row target lane
  float* loss;            // cross-entropy: per-row loss
  float* xt;              // cross-entropy on the split path: per-row target logit
  int64_t rows;
  int64_t cols;
  MaskArgs mask;
};

// What the kernels write once a row's (m, l) is known.
constexpr int kEpiSoftmax = 0;     // y = exp(x - m) / l
constexpr int kEpiLogSoftmax = 1;  // y = x - (m + log l), and/or lse = m + log l
constexpr int kEpiXent = 2;        // loss = LSE - x_t, y = p - onehot(t)

inline int elem_size(int dtype) { return dtype == kF32 ? 4 : 2; }
// elements per 128-bit access
inline int vec_elems(int dtype) { return 16 / elem_size(dtype); }

// --- wave-per-row kernel (k_wave.hip) ---
// Largest cols the wave path holds in registers.
int64_t wave_max_cols(int dtype, bool vec);
hipError_t launch_wave(const RowArgs& a, int dtype, bool vec, int epi, hipStream_t stream);

// --- workgroup-per-row, LDS-staged kernels ---
// The LDS path: rows up to 32 KiB staged in LDS and held in registers
// (k_lds.hip), longer ones up to lds_max_cols resident in LDS (k_lds_res.hip).
int64_t lds_max_cols(int dtype);
hipError_t launch_lds(const RowArgs& a, int dtype, int epi, hipStream_t stream);
// rows too long for the registers: three passes over the row in LDS
int64_t lds_res_max_cols(int dtype);
hipError_t launch_lds_res(const RowArgs& a, int dtype, int epi, hipStream_t stream);

// --- split path (k_split.hip) ---
// Elements one workgroup holds per round of a chunk.
int64_t split_round_cols(int dtype, bool vec);
// xent: the target lane is left out of the summaries and its logit is
// written to a.xt
hipError_t launch_stats(const RowArgs& a, int dtype, bool vec, bool xent, int64_t chunk_cols, int64_t n_chunks,
                        smx_stat* stats, hipStream_t stream);
// stats holds n_summaries summaries per row: every chunk's (n_chunks), or the
// single one launch_row_merge left
hipError_t launch_merge_normalize(const RowArgs& a, int dtype, bool vec, int epi, int64_t chunk_cols,
                                  int64_t n_chunks, const smx_stat* stats, int64_t n_summaries, hipStream_t stream);
// each row's n_chunks summaries merged into merged[row], bitwise as the
// normalize pass would merge them
hipError_t launch_row_merge(const smx_stat* stats, int64_t rows, int64_t n_chunks, smx_stat* merged,
                            hipStream_t stream);
// more chunks per row than this: the summaries are merged once per row first
constexpr int64_t kRowMergeMinChunks = 1024;

// --- softmax backward (k_backward.hip) ---
int64_t bwd_wave_max_cols(int dtype, bool vec);
int64_t bwd_block_max_cols(int dtype, bool vec);
hipError_t launch_bwd_rows(const char* p, const char* g, char* dx, int64_t rows, int64_t cols, int dtype,
                           bool vec, bool wave, hipStream_t stream);
// partials holds rows * n_chunks partial dot products, then (when n_chunks
// exceeds kRowMergeMinChunks) room for one merged pair per row
hipError_t launch_bwd_split(const char* p, const char* g, char* dx, int64_t rows, int64_t cols, int dtype, bool vec,
                            int64_t chunk, int64_t n_chunks, float2* partials, hipStream_t stream);

// --- softmax-weighted value sums split along the keys (k_wsplit.hip) ---
// the longest key chunk of one state (its weights sit in LDS)
constexpr int kMaxWChunk = 2048;
// the most chunk states one row's merge takes (their factors sit in LDS)
constexpr int64_t kMaxWMergeChunks = 16384;
// per (row, chunk): ml = (m, l), o[d]; v 16-byte aligned
hipError_t launch_wstates(const char* s, const char* v, int64_t rows, int64_t cols, int64_t d, int64_t rows_per_group,
                          int dtype, const MaskArgs& mask, int64_t chunk, int64_t n_chunks, float* ml, float* o,
                          hipStream_t stream);
hipError_t launch_wmerge(const float* ml, const float* o, int64_t rows, int64_t n_chunks, int64_t d, int dtype,
                         char* out, hipStream_t stream);

// --- softmax-weighted value sums on the matrix cores (k_pv.hip) ---
bool pv_supported_d(int64_t d);
hipError_t launch_pv(const char* s, const char* v, char* out, int64_t rows, int64_t cols, int64_t d,
                     int64_t rows_per_group, int dtype, const MaskArgs& mask, hipStream_t stream);

// --- the streaming copy used as a bandwidth reference (k_copy.hip) ---
// n16 16-byte packs from x to y; both 16-byte aligned, not overlapping
hipError_t launch_stream_copy(const void* x, void* y, int64_t n16, hipStream_t stream);

}  // namespace smx
