// smx_api.hip — the C ABI: argument checks, path choice and launches.
//
// Nothing here touches the device before every argument has been checked;
// an invalid call returns SMX_EINVAL with a message and enqueues nothing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "smx_internal.hpp"

namespace smx {
namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SMX_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SMX_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Row geometry and mask, checked.
struct Call {
  RowArgs a{};
  int dtype = 0;
  bool vec = false;  // 128-bit accesses allowed
};

int check_common(const void* x, const void* y, int64_t rows, int64_t cols, int dtype, const smx_mask* mk,
                 bool need_y, Call& c) {
  if (dtype != SMX_F32 && dtype != SMX_F16 && dtype != SMX_BF16)
    return fail(SMX_EINVAL, "dtype %d is not SMX_F32, SMX_F16 or SMX_BF16", dtype);
  if (rows < 0 || cols < 0) return fail(SMX_EINVAL, "rows (%lld) and cols (%lld) must be >= 0", (long long)rows,
                                        (long long)cols);
  const int64_t s = elem_size(dtype);
  if (cols > 0 && rows > INT64_MAX / cols / s) return fail(SMX_EINVAL, "rows * cols * element size overflows int64");
  const int64_t n = rows * cols;
  if (n > 0 && x == nullptr) return fail(SMX_EINVAL, "x is NULL");
  if (need_y && n > 0 && y == nullptr) return fail(SMX_EINVAL, "y is NULL");
  if (need_y && n > 0 && x != y) {
    const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y, bytes = (uintptr_t)(n * s);
    if (xa < ya + bytes && ya < xa + bytes) return fail(SMX_EINVAL, "x and y overlap without being equal");
  }
  MaskArgs m{};
  m.kind = mk ? (int)mk->kind : SMX_MASK_NONE;
  switch (m.kind) {
    case SMX_MASK_NONE:
      break;
    case SMX_MASK_VALID_LEN:
      if (rows > 0 && mk->valid_len == nullptr) return fail(SMX_EINVAL, "SMX_MASK_VALID_LEN needs valid_len");
      m.valid_len = mk->valid_len;
      break;
    case SMX_MASK_CAUSAL:
      if (mk->causal_period <= 0) return fail(SMX_EINVAL, "SMX_MASK_CAUSAL needs causal_period > 0");
      if (mk->causal_offset > ((int64_t)1 << 62) || mk->causal_offset < -((int64_t)1 << 62))
        return fail(SMX_EINVAL, "causal_offset out of range (|offset| <= 2^62)");
      m.period = mk->causal_period;
      m.offset = mk->causal_offset;
      break;
    case SMX_MASK_KEEP_BYTES:
      if (n > 0 && mk->keep == nullptr) return fail(SMX_EINVAL, "SMX_MASK_KEEP_BYTES needs keep");
      m.keep = mk->keep;
      break;
    default:
      return fail(SMX_EINVAL, "mask kind %d is not a smx_mask_kind", m.kind);
  }
  c.dtype = dtype;
  c.a.x = (const char*)x;
  c.a.y = (char*)y;
  c.a.rows = rows;
  c.a.cols = cols;
  c.a.mask = m;
  const int e = vec_elems(dtype);
  c.vec = ((uintptr_t)x % 16 == 0) && (!need_y || (uintptr_t)y % 16 == 0) && ((cols * s) % 16 == 0) &&
          (m.kind != SMX_MASK_KEEP_BYTES || (uintptr_t)m.keep % e == 0);
  return SMX_OK;
}

// Rows of at most 4 KiB take a wave each; aligned rows up to the LDS budget
// (152 KiB) are read once on the LDS path whatever their number (measured
// faster than the split path from 64 rows up, and the split path's two
// launches and stream-ordered workspace cost some 24 us on small inputs);
// unaligned rows the wave path still holds, when there are enough of them to
// fill the chip, stay there; everything else is split.
constexpr int64_t kWaveMinRows = 1024;

smx_path choose(int64_t rows, int64_t cols, int dtype, bool vec) {
  const int64_t bytes = cols * elem_size(dtype);
  if (cols <= wave_max_cols(dtype, vec) && bytes <= 4096) return SMX_PATH_WAVE;
  if (vec && cols <= lds_max_cols(dtype)) return SMX_PATH_LDS;
  if (cols <= wave_max_cols(dtype, vec) && rows >= kWaveMinRows) return SMX_PATH_WAVE;
  return SMX_PATH_SPLIT;
}

int64_t default_chunk(int64_t rows, int64_t cols, int dtype, bool vec) {
  // 32 KiB chunks (two register rounds per thread of the stats pass, both in
  // flight from the start), halved while the grid has fewer than 1024
  // workgroups (4 per CU), never below 64 packs. Measured on the split path
  // against 64 KiB chunks and a floor of 2048 workgroups: 1 to 4 % faster on
  // every large fp32 and 16-bit shape, 5 % on a few long fp32 rows.
  const int64_t e = vec ? vec_elems(dtype) : 1;
  int64_t chunk = 32768 / elem_size(dtype);
  const int64_t floor_chunk = 64 * e;
  while (chunk > floor_chunk && rows * ((cols + chunk - 1) / chunk) < 1024) chunk /= 2;
  return chunk;
}

// The split path's workspace: the chunk summaries, then (many chunks per row)
// one merged summary per row, then (cross-entropy) one target logit per row.
// Every byte of it is written before it is read within one call, so nothing
// in it has to start at zero.
struct SplitWs {
  size_t stat_bytes, merged_bytes, bytes;
  bool row_merge;
};
SplitWs split_ws(int64_t rows, int64_t nch, int epi) {
  SplitWs w;
  w.row_merge = nch > kRowMergeMinChunks;
  w.stat_bytes = (size_t)(rows * nch) * sizeof(smx_stat);
  w.merged_bytes = w.row_merge ? (size_t)rows * sizeof(smx_stat) : 0;
  w.bytes = w.stat_bytes + w.merged_bytes + (epi == kEpiXent ? (size_t)rows * sizeof(float) : 0);
  return w;
}

// fixed_ws: a caller-provided workspace of at least split_ws(...).bytes (the
// no-allocation entry point's scratch), or null for a stream-ordered
// allocation freed on the same stream
int run_split(const Call& c0, int64_t chunk, int epi, hipStream_t stream, void* fixed_ws) {
  Call c = c0;
  const int64_t e = vec_elems(c.dtype);
  const bool vec = c.vec && chunk % e == 0;
  const int64_t nch = (c.a.cols + chunk - 1) / chunk;
  const SplitWs w = split_ws(c.a.rows, nch, epi);
  const bool row_merge = w.row_merge;
  const size_t stat_bytes = w.stat_bytes, merged_bytes = w.merged_bytes;
  void* ws = fixed_ws;
  hipError_t err = hipSuccess;
  if (ws == nullptr) {
    err = hipMallocAsync(&ws, w.bytes, stream);
    if (err != hipSuccess) return hip_fail(err, "hipMallocAsync of the summary workspace");
  }
  smx_stat* const stats = (smx_stat*)ws;
  smx_stat* const merged = (smx_stat*)((char*)ws + stat_bytes);
  if (epi == kEpiXent) c.a.xt = (float*)((char*)ws + stat_bytes + merged_bytes);
  err = launch_stats(c.a, c.dtype, vec, epi == kEpiXent, chunk, nch, stats, stream);
  if (err == hipSuccess && row_merge) err = launch_row_merge(stats, c.a.rows, nch, merged, stream);
  if (err == hipSuccess) {
    err = row_merge ? launch_merge_normalize(c.a, c.dtype, vec, epi, chunk, nch, merged, 1, stream)
                    : launch_merge_normalize(c.a, c.dtype, vec, epi, chunk, nch, stats, nch, stream);
  }
  const hipError_t ferr = fixed_ws == nullptr ? hipFreeAsync(ws, stream) : hipSuccess;
  if (err != hipSuccess) return hip_fail(err, "split-path launch");
  if (ferr != hipSuccess) return hip_fail(ferr, "hipFreeAsync of the summary workspace");
  return ok();
}

int run_rows(const Call& c, smx_path path, int64_t chunk_cols, int epi, hipStream_t stream,
             void* fixed_ws = nullptr) {
  const int64_t rows = c.a.rows, cols = c.a.cols;
  if (path == SMX_PATH_AUTO) path = choose(rows, cols, c.dtype, c.vec);
  hipError_t err = hipSuccess;
  switch (path) {
    case SMX_PATH_WAVE:
      if (cols > wave_max_cols(c.dtype, c.vec))
        return fail(SMX_EINVAL, "the wave path holds at most %lld cols for this dtype/alignment",
                    (long long)wave_max_cols(c.dtype, c.vec));
      err = launch_wave(c.a, c.dtype, c.vec, epi, stream);
      break;
    case SMX_PATH_LDS:
      if (!c.vec)
        return fail(SMX_EINVAL, "the LDS path needs 16-byte aligned x, y and rows of a multiple of 16 bytes");
      if (cols > lds_max_cols(c.dtype))
        return fail(SMX_EINVAL, "the LDS path holds at most %lld cols for this dtype",
                    (long long)lds_max_cols(c.dtype));
      err = launch_lds(c.a, c.dtype, epi, stream);
      break;
    case SMX_PATH_SPLIT: {
      if (chunk_cols < 0) return fail(SMX_EINVAL, "chunk_cols must be >= 0");
      const int64_t chunk = chunk_cols > 0 ? chunk_cols : default_chunk(rows, cols, c.dtype, c.vec);
      return run_split(c, chunk, epi, stream, fixed_ws);
    }
    default:
      return fail(SMX_EINVAL, "path %d is not a smx_path", (int)path);
  }
  if (err != hipSuccess) return hip_fail(err, "kernel launch");
  return ok();
}

// whether [a, a + na) and [b, b + nb) share a byte
bool overlaps(const void* a, uintptr_t na, const void* b, uintptr_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

// The checks shared by the weighted-sum calls: scores s [rows, cols] under
// the mask, values v [rows / rows_per_group, cols, d], 16-bit, aligned.
int check_weighted(const char* name, const void* s, const void* v, int64_t rows, int64_t cols, int64_t d,
                   int64_t rows_per_group, smx_dtype dtype, const smx_mask* mask, Call& c) {
  if (int rc = check_common(s, nullptr, rows, cols, (int)dtype, mask, false, c)) return rc;
  if (dtype == SMX_F32) return fail(SMX_EINVAL, "%s takes SMX_F16 or SMX_BF16", name);
  if (!pv_supported_d(d)) return fail(SMX_EINVAL, "d = %lld: the value width must be 32, 64 or 128", (long long)d);
  if (rows_per_group <= 0 || rows % rows_per_group != 0)
    return fail(SMX_EINVAL, "rows (%lld) must be a positive multiple of rows_per_group (%lld)", (long long)rows,
                (long long)rows_per_group);
  if (cols % 8 != 0) return fail(SMX_EINVAL, "cols (%lld) must be a multiple of 8", (long long)cols);
  if (cols > ((int64_t)1 << 30))
    return fail(SMX_EINVAL, "cols (%lld) exceeds 2^30, the longest row the weighted sums take", (long long)cols);
  const int64_t groups = rows / rows_per_group;
  if (cols > 0 && groups > INT64_MAX / cols / d / 2) return fail(SMX_EINVAL, "the size of v overflows int64");
  if (rows > INT64_MAX / d / 2) return fail(SMX_EINVAL, "the size of out overflows int64");
  if (rows > 0 && cols > 0 && v == nullptr) return fail(SMX_EINVAL, "v must not be NULL");
  if ((uintptr_t)s % 16 != 0 || (uintptr_t)v % 16 != 0) return fail(SMX_EINVAL, "s and v must be 16-byte aligned");
  if (c.a.mask.kind == SMX_MASK_KEEP_BYTES && (uintptr_t)c.a.mask.keep % 8 != 0)
    return fail(SMX_EINVAL, "keep must be 8-byte aligned");
  return SMX_OK;
}

// softmax_weighted_rows takes the key-split path for groups of at most 4
// score rows, and of at most 8 when there are too few groups (under 256) for
// the matrix-core kernel's one workgroup per 128-row tile to fill the chip;
// larger groups keep the matrix cores, whose products the vector ALUs cannot
// match (measured: 256 groups of 8 rows, 8192 keys: 163 us there, 300 us split)
bool weighted_split(int64_t rows_per_group, int64_t groups) {
  return rows_per_group <= 4 || (rows_per_group <= 8 && groups < 256);
}

// the key chunk of that path: 512, halved (down to 128) while the grid has
// fewer than 2048 workgroups, doubled (up to kMaxWChunk) while a row would
// leave more chunk states than one merge folds (kMaxWMergeChunks: their
// factors sit in LDS); 0 when even the longest chunk leaves too many, and
// those rows (more than kMaxWChunk * kMaxWMergeChunks = 2^25 keys) take the
// matrix-core kernel instead
int64_t weighted_split_chunk(int64_t groups, int64_t cols) {
  int64_t chunk = 512;
  while (chunk > 128 && groups * ((cols + chunk - 1) / chunk) < 2048) chunk /= 2;
  while (chunk < kMaxWChunk && (cols + chunk - 1) / chunk > kMaxWMergeChunks) chunk *= 2;
  return (cols + chunk - 1) / chunk > kMaxWMergeChunks ? 0 : chunk;
}

}  // namespace

// The scratch of softmax_rows_noalloc: the split path's summaries for callers
// that cannot allocate. Each device holds its own copy for the life of the
// process. In host code the array's name is only a stand-in; the device
// address comes from hipGetSymbolAddress on that device.
static __device__ __align__(256) char scratch[SMX_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// The current device's copy of scratch: looked up once per device, on the
// first call made with that device current, and kept.
int scratch_on_current_device(void** ptr) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SMX_EHIP, "device %d: softmax_rows_noalloc tracks devices 0 to %d", dev, kMaxDevices - 1);
  ScratchSlot& s = g_scratch[dev];
  std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  if (s.err != hipSuccess) return hip_fail(s.err, "hipGetSymbolAddress of the scratch buffer");
  *ptr = s.ptr;
  return SMX_OK;
}

}  // namespace
}  // namespace smx

using namespace smx;

extern "C" {

int softmax_rows_path(const void* x, void* y, int64_t rows, int64_t cols, smx_dtype dtype, const smx_mask* mask,
                      smx_path path, int64_t chunk_cols, void* stream) {
  Call c;
  if (int rc = check_common(x, y, rows, cols, (int)dtype, mask, true, c)) return rc;
  if ((int)path < SMX_PATH_AUTO || (int)path > SMX_PATH_SPLIT) return fail(SMX_EINVAL, "path %d is not a smx_path", (int)path);
  if (chunk_cols < 0) return fail(SMX_EINVAL, "chunk_cols must be >= 0");
  if (rows == 0 || cols == 0) return ok();
  return run_rows(c, path, chunk_cols, kEpiSoftmax, (hipStream_t)stream);
}

int softmax_rows(const void* x, void* y, int64_t rows, int64_t cols, smx_dtype dtype, const smx_mask* mask,
                 void* stream) {
  return softmax_rows_path(x, y, rows, cols, dtype, mask, SMX_PATH_AUTO, 0, stream);
}

int softmax_rows_noalloc(const void* x, void* y, int64_t rows, int64_t cols, smx_dtype dtype, const smx_mask* mask,
                         smx_path path, int64_t chunk_cols, void* stream) {
  Call c;
  if (int rc = check_common(x, y, rows, cols, (int)dtype, mask, true, c)) return rc;
  if ((int)path < SMX_PATH_AUTO || (int)path > SMX_PATH_SPLIT) return fail(SMX_EINVAL, "path %d is not a smx_path", (int)path);
  if (chunk_cols < 0) return fail(SMX_EINVAL, "chunk_cols must be >= 0");
  if (rows == 0 || cols == 0) return ok();
  const smx_path p = path == SMX_PATH_AUTO ? choose(rows, cols, c.dtype, c.vec) : path;
  void* ws = nullptr;
  if (p == SMX_PATH_SPLIT) {
    // only the split path uses scratch; its size is checked before anything
    // is enqueued (rows * n_chunks is bounded first so the product cannot
    // overflow)
    const int64_t chunk = chunk_cols > 0 ? chunk_cols : default_chunk(rows, cols, c.dtype, c.vec);
    const int64_t nch = (cols + chunk - 1) / chunk;
    const int64_t max_summaries = SMX_NOALLOC_SCRATCH_BYTES / (int64_t)sizeof(smx_stat);
    if (rows > max_summaries / nch || split_ws(rows, nch, kEpiSoftmax).bytes > (size_t)SMX_NOALLOC_SCRATCH_BYTES)
      return fail(SMX_EINVAL,
                  "the split path needs %lld x %lld chunk summaries here, more than the %lld bytes of scratch "
                  "softmax_rows_noalloc holds (use larger chunk_cols, or softmax_rows_path)",
                  (long long)rows, (long long)nch, (long long)SMX_NOALLOC_SCRATCH_BYTES);
    if (int rc = scratch_on_current_device(&ws)) return rc;
  }
  return run_rows(c, p, chunk_cols, kEpiSoftmax, (hipStream_t)stream, ws);
}

smx_path softmax_select_path(int64_t rows, int64_t cols, smx_dtype dtype) {
  if ((int)dtype < 0 || (int)dtype > 2 || rows < 0 || cols < 0) return SMX_PATH_AUTO;
  // the path for 16-byte aligned buffers
  return choose(rows, cols, (int)dtype, (cols * elem_size((int)dtype)) % 16 == 0);
}

int64_t softmax_default_chunk_cols(int64_t rows, int64_t cols, smx_dtype dtype) {
  if ((int)dtype < 0 || (int)dtype > 2 || rows < 0 || cols < 0) return 0;
  return default_chunk(rows, cols, (int)dtype, (cols * elem_size((int)dtype)) % 16 == 0);
}

int softmax_row_stats(const void* x, int64_t rows, int64_t cols, smx_dtype dtype, const smx_mask* mask,
                      int64_t chunk_cols, smx_stat* stats, void* stream) {
  Call c;
  if (int rc = check_common(x, nullptr, rows, cols, (int)dtype, mask, false, c)) return rc;
  if (chunk_cols <= 0) return fail(SMX_EINVAL, "chunk_cols must be > 0");
  const int64_t nch = (cols + chunk_cols - 1) / chunk_cols;
  if (rows > 0 && nch > 0 && stats == nullptr) return fail(SMX_EINVAL, "stats is NULL");
  if (rows == 0 || cols == 0) return ok();
  const bool vec = c.vec && chunk_cols % vec_elems(c.dtype) == 0;
  hipError_t err = launch_stats(c.a, c.dtype, vec, false, chunk_cols, nch, stats, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "stats launch");
  return ok();
}

int softmax_merge_normalize(const void* x, void* y, int64_t rows, int64_t cols, smx_dtype dtype,
                            const smx_mask* mask, int64_t chunk_cols, const smx_stat* stats, int64_t n_chunks,
                            void* stream) {
  Call c;
  if (int rc = check_common(x, y, rows, cols, (int)dtype, mask, true, c)) return rc;
  if (chunk_cols <= 0) return fail(SMX_EINVAL, "chunk_cols must be > 0");
  const int64_t nch = (cols + chunk_cols - 1) / chunk_cols;
  if (n_chunks != nch)
    return fail(SMX_EINVAL, "n_chunks is %lld but ceil(cols / chunk_cols) is %lld", (long long)n_chunks,
                (long long)nch);
  if (rows > 0 && nch > 0 && stats == nullptr) return fail(SMX_EINVAL, "stats is NULL");
  if (rows == 0 || cols == 0) return ok();
  const bool vec = c.vec && chunk_cols % vec_elems(c.dtype) == 0;
  const hipStream_t st = (hipStream_t)stream;
  if (nch <= kRowMergeMinChunks) {
    const hipError_t err = launch_merge_normalize(c.a, c.dtype, vec, kEpiSoftmax, chunk_cols, nch, stats, nch, st);
    if (err != hipSuccess) return hip_fail(err, "merge/normalize launch");
    return ok();
  }
  // many chunks per row: each row's summaries are merged once (8 bytes per
  // row in a stream-ordered workspace), bitwise as every chunk's workgroup
  // would merge them, so the summary reads grow linearly with n_chunks
  void* ws = nullptr;
  hipError_t err = hipMallocAsync(&ws, (size_t)rows * sizeof(smx_stat), st);
  if (err != hipSuccess) return hip_fail(err, "hipMallocAsync of the merged summaries");
  smx_stat* const merged = (smx_stat*)ws;
  err = launch_row_merge(stats, rows, nch, merged, st);
  if (err == hipSuccess) err = launch_merge_normalize(c.a, c.dtype, vec, kEpiSoftmax, chunk_cols, nch, merged, 1, st);
  const hipError_t ferr = hipFreeAsync(ws, st);
  if (err != hipSuccess) return hip_fail(err, "merge/normalize launch");
  if (ferr != hipSuccess) return hip_fail(ferr, "hipFreeAsync of the merged summaries");
  return ok();
}

int log_softmax_rows_path(const void* x, void* y, float* lse, int64_t rows, int64_t cols, smx_dtype dtype,
                          const smx_mask* mask, smx_path path, int64_t chunk_cols, void* stream) {
  Call c;
  if (int rc = check_common(x, y, rows, cols, (int)dtype, mask, y != nullptr, c)) return rc;
  if ((int)path < SMX_PATH_AUTO || (int)path > SMX_PATH_SPLIT) return fail(SMX_EINVAL, "path %d is not a smx_path", (int)path);
  if (chunk_cols < 0) return fail(SMX_EINVAL, "chunk_cols must be >= 0");
  if (y == nullptr && lse == nullptr && rows > 0 && cols > 0) return fail(SMX_EINVAL, "y and lse are both NULL");
  if (lse != nullptr && rows > 0) {
    const uintptr_t la = (uintptr_t)lse, lb = (uintptr_t)(rows * 4);
    const uintptr_t xb = (uintptr_t)(rows * cols * elem_size((int)dtype));
    const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y;
    if (xb > 0 && ((la < xa + xb && xa < la + lb) || (y != nullptr && la < ya + xb && ya < la + lb)))
      return fail(SMX_EINVAL, "lse overlaps x or y");
  }
  c.a.lse = lse;
  if (rows == 0) return ok();
  if (cols == 0) {
    // every row is empty: lse = -inf (nothing else to write)
    if (lse == nullptr) return ok();
    c.a.cols = 0;
    hipError_t err = launch_wave(c.a, c.dtype, false, kEpiLogSoftmax, (hipStream_t)stream);
    if (err != hipSuccess) return hip_fail(err, "kernel launch");
    return ok();
  }
  return run_rows(c, path, chunk_cols, kEpiLogSoftmax, (hipStream_t)stream);
}

int log_softmax_rows(const void* x, void* y, float* lse, int64_t rows, int64_t cols, smx_dtype dtype,
                     const smx_mask* mask, void* stream) {
  return log_softmax_rows_path(x, y, lse, rows, cols, dtype, mask, SMX_PATH_AUTO, 0, stream);
}

int softmax_cross_entropy_rows_path(const void* x, const int32_t* target, float* loss, void* dx, int64_t rows,
                                    int64_t cols, smx_dtype dtype, const smx_mask* mask, smx_path path,
                                    int64_t chunk_cols, void* stream) {
  Call c;
  if (int rc = check_common(x, dx, rows, cols, (int)dtype, mask, dx != nullptr, c)) return rc;
  if ((int)path < SMX_PATH_AUTO || (int)path > SMX_PATH_SPLIT) return fail(SMX_EINVAL, "path %d is not a smx_path", (int)path);
  if (chunk_cols < 0) return fail(SMX_EINVAL, "chunk_cols must be >= 0");
  if (rows > 0 && (target == nullptr || loss == nullptr)) return fail(SMX_EINVAL, "target and loss must not be NULL");
  if (rows > 0) {
    const uintptr_t la = (uintptr_t)loss, lb = (uintptr_t)(rows * 4);
    const uintptr_t xb = (uintptr_t)(rows * cols * elem_size((int)dtype));
    const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)dx;
    if (xb > 0 && ((la < xa + xb && xa < la + lb) || (dx != nullptr && la < ya + xb && ya < la + lb)))
      return fail(SMX_EINVAL, "loss overlaps x or dx");
  }
  c.a.target = target;
  c.a.loss = loss;
  if (rows == 0) return ok();
  if (cols == 0) {
    // every target is out of range: every row is ignored (loss 0)
    hipError_t err = launch_wave(c.a, c.dtype, false, kEpiXent, (hipStream_t)stream);
    if (err != hipSuccess) return hip_fail(err, "kernel launch");
    return ok();
  }
  return run_rows(c, path, chunk_cols, kEpiXent, (hipStream_t)stream);
}

int softmax_cross_entropy_rows(const void* x, const int32_t* target, float* loss, void* dx, int64_t rows,
                               int64_t cols, smx_dtype dtype, const smx_mask* mask, void* stream) {
  return softmax_cross_entropy_rows_path(x, target, loss, dx, rows, cols, dtype, mask, SMX_PATH_AUTO, 0, stream);
}

int softmax_backward_rows_path(const void* p, const void* g, void* dx, int64_t rows, int64_t cols, smx_dtype dtype,
                               smx_path path, int64_t chunk_cols, void* stream) {
  const int dt = (int)dtype;
  if (dt != SMX_F32 && dt != SMX_F16 && dt != SMX_BF16)
    return fail(SMX_EINVAL, "dtype %d is not SMX_F32, SMX_F16 or SMX_BF16", dt);
  if (rows < 0 || cols < 0) return fail(SMX_EINVAL, "rows and cols must be >= 0");
  const int64_t s = elem_size(dt);
  if (cols > 0 && rows > INT64_MAX / cols / s) return fail(SMX_EINVAL, "rows * cols * element size overflows int64");
  if ((int)path < SMX_PATH_AUTO || (int)path > SMX_PATH_SPLIT) return fail(SMX_EINVAL, "path %d is not a smx_path", (int)path);
  if (chunk_cols < 0) return fail(SMX_EINVAL, "chunk_cols must be >= 0");
  const int64_t n = rows * cols;
  if (n == 0) return ok();
  if (p == nullptr || g == nullptr || dx == nullptr) return fail(SMX_EINVAL, "p, g and dx must not be NULL");
  const uintptr_t bytes = (uintptr_t)(n * s), da = (uintptr_t)dx;
  for (const void* in : {p, g}) {
    const uintptr_t ia = (uintptr_t)in;
    if (ia != da && ia < da + bytes && da < ia + bytes) return fail(SMX_EINVAL, "dx overlaps p or g without being equal");
  }
  const bool vec = (uintptr_t)p % 16 == 0 && (uintptr_t)g % 16 == 0 && da % 16 == 0 && (cols * s) % 16 == 0;
  if (path == SMX_PATH_AUTO) {
    if (cols <= bwd_wave_max_cols(dt, vec) && cols * s <= 4096)
      path = SMX_PATH_WAVE;
    else if (cols <= bwd_block_max_cols(dt, vec) && rows >= 1024)
      path = SMX_PATH_LDS;
    else
      path = SMX_PATH_SPLIT;
  }
  hipError_t err = hipSuccess;
  const hipStream_t st = (hipStream_t)stream;
  if (path == SMX_PATH_WAVE || path == SMX_PATH_LDS) {
    const bool wave = path == SMX_PATH_WAVE;
    const int64_t cap = wave ? bwd_wave_max_cols(dt, vec) : bwd_block_max_cols(dt, vec);
    if (cols > cap) return fail(SMX_EINVAL, "this path holds at most %lld cols for this dtype/alignment", (long long)cap);
    err = launch_bwd_rows((const char*)p, (const char*)g, (char*)dx, rows, cols, dt, vec, wave, st);
    if (err != hipSuccess) return hip_fail(err, "kernel launch");
    return ok();
  }
  const int64_t e = vec_elems(dt);
  const int64_t chunk = chunk_cols > 0 ? chunk_cols : default_chunk(rows, cols, dt, vec);
  const bool cvec = vec && chunk % e == 0;
  const int64_t nch = (cols + chunk - 1) / chunk;
  void* ws = nullptr;
  const size_t part_count = (size_t)(rows * nch) + (nch > kRowMergeMinChunks ? (size_t)rows : 0);
  err = hipMallocAsync(&ws, part_count * sizeof(float2), st);
  if (err != hipSuccess) return hip_fail(err, "hipMallocAsync of the partial-dot workspace");
  err = launch_bwd_split((const char*)p, (const char*)g, (char*)dx, rows, cols, dt, cvec, chunk, nch, (float2*)ws, st);
  const hipError_t ferr = hipFreeAsync(ws, st);
  if (err != hipSuccess) return hip_fail(err, "kernel launch");
  if (ferr != hipSuccess) return hip_fail(ferr, "hipFreeAsync of the partial-dot workspace");
  return ok();
}

int softmax_backward_rows(const void* p, const void* g, void* dx, int64_t rows, int64_t cols, smx_dtype dtype,
                          void* stream) {
  return softmax_backward_rows_path(p, g, dx, rows, cols, dtype, SMX_PATH_AUTO, 0, stream);
}

int softmax_weighted_rows(const void* s, const void* v, void* out, int64_t rows, int64_t cols, int64_t d,
                          int64_t rows_per_group, smx_dtype dtype, const smx_mask* mask, void* stream) {
  Call c;
  if (int rc = check_weighted("softmax_weighted_rows", s, v, rows, cols, d, rows_per_group, dtype, mask, c)) return rc;
  if (rows == 0) return ok();
  if (out == nullptr) return fail(SMX_EINVAL, "out must not be NULL");
  if ((uintptr_t)out % 8 != 0) return fail(SMX_EINVAL, "out must be 8-byte aligned");
  const int64_t groups = rows / rows_per_group;
  const uintptr_t ob = (uintptr_t)(rows * d * 2);
  if (overlaps(out, ob, s, (uintptr_t)(rows * cols * 2)) || overlaps(out, ob, v, (uintptr_t)(groups * cols * d * 2)))
    return fail(SMX_EINVAL, "out overlaps s or v");
  const hipStream_t st = (hipStream_t)stream;
  const int64_t chunk = weighted_split(rows_per_group, groups) ? weighted_split_chunk(groups, cols) : 0;
  if (chunk == 0 || cols == 0) {
    const hipError_t err = launch_pv((const char*)s, (const char*)v, (char*)out, rows, cols, d, rows_per_group,
                                     c.dtype, c.a.mask, st);
    if (err != hipSuccess) return hip_fail(err, "kernel launch");
    return ok();
  }
  // few rows per group: per-chunk states in a stream-ordered workspace, merged
  const int64_t nch = (cols + chunk - 1) / chunk;
  const size_t ml_bytes = (size_t)(rows * nch) * 2 * sizeof(float);
  const size_t bytes = ml_bytes + (size_t)(rows * nch * d) * sizeof(float);
  void* ws = nullptr;
  hipError_t err = hipMallocAsync(&ws, bytes, st);
  if (err != hipSuccess) return hip_fail(err, "hipMallocAsync of the state workspace");
  float* const ml = (float*)ws;
  float* const o = (float*)((char*)ws + ml_bytes);
  err = launch_wstates((const char*)s, (const char*)v, rows, cols, d, rows_per_group, c.dtype, c.a.mask, chunk, nch,
                       ml, o, st);
  if (err == hipSuccess) err = launch_wmerge(ml, o, rows, nch, d, c.dtype, (char*)out, st);
  const hipError_t ferr = hipFreeAsync(ws, st);
  if (err != hipSuccess) return hip_fail(err, "kernel launch");
  if (ferr != hipSuccess) return hip_fail(ferr, "hipFreeAsync of the state workspace");
  return ok();
}

int softmax_weighted_states(const void* s, const void* v, int64_t rows, int64_t cols, int64_t d,
                            int64_t rows_per_group, smx_dtype dtype, const smx_mask* mask, int64_t chunk_cols,
                            float* ml, float* o, void* stream) {
  Call c;
  if (int rc = check_weighted("softmax_weighted_states", s, v, rows, cols, d, rows_per_group, dtype, mask, c))
    return rc;
  if (chunk_cols <= 0 || chunk_cols > kMaxWChunk)
    return fail(SMX_EINVAL, "chunk_cols (%lld) must be in [1, %d]", (long long)chunk_cols, kMaxWChunk);
  const int64_t nch = (cols + chunk_cols - 1) / chunk_cols;
  if (rows == 0 || nch == 0) return ok();
  if (ml == nullptr || o == nullptr) return fail(SMX_EINVAL, "ml and o must not be NULL");
  if ((uintptr_t)ml % 4 != 0 || (uintptr_t)o % 4 != 0) return fail(SMX_EINVAL, "ml and o must be 4-byte aligned");
  if (rows * nch > INT64_MAX / d / 4) return fail(SMX_EINVAL, "the size of o overflows int64");
  const int64_t groups = rows / rows_per_group;
  const uintptr_t mlb = (uintptr_t)(rows * nch * 8), obb = (uintptr_t)(rows * nch * d * 4);
  const uintptr_t sb = (uintptr_t)(rows * cols * 2), vb = (uintptr_t)(groups * cols * d * 2);
  if (overlaps(ml, mlb, o, obb) || overlaps(ml, mlb, s, sb) || overlaps(ml, mlb, v, vb) || overlaps(o, obb, s, sb) ||
      overlaps(o, obb, v, vb))
    return fail(SMX_EINVAL, "ml and o must overlap neither each other nor s or v");
  const hipError_t err = launch_wstates((const char*)s, (const char*)v, rows, cols, d, rows_per_group, c.dtype,
                                        c.a.mask, chunk_cols, nch, ml, o, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "kernel launch");
  return ok();
}

int softmax_weighted_merge(const float* ml, const float* o, int64_t rows, int64_t n_chunks, int64_t d,
                           smx_dtype dtype, void* out, void* stream) {
  if (dtype != SMX_F16 && dtype != SMX_BF16)
    return fail(SMX_EINVAL, "softmax_weighted_merge writes SMX_F16 or SMX_BF16");
  if (!pv_supported_d(d)) return fail(SMX_EINVAL, "d = %lld: the value width must be 32, 64 or 128", (long long)d);
  if (rows < 0 || n_chunks < 0) return fail(SMX_EINVAL, "rows and n_chunks must be >= 0");
  if (n_chunks > kMaxWMergeChunks)
    return fail(SMX_EINVAL, "n_chunks (%lld) exceeds %lld", (long long)n_chunks, (long long)kMaxWMergeChunks);
  if (rows == 0) return ok();
  if (rows > INT64_MAX / (n_chunks + 1) / d / 4) return fail(SMX_EINVAL, "the size of o overflows int64");
  if (out == nullptr || (n_chunks > 0 && (ml == nullptr || o == nullptr)))
    return fail(SMX_EINVAL, "ml, o and out must not be NULL");
  if ((uintptr_t)out % 2 != 0 || (uintptr_t)ml % 4 != 0 || (uintptr_t)o % 4 != 0)
    return fail(SMX_EINVAL, "out must be 2-byte aligned, ml and o 4-byte aligned");
  const uintptr_t ob = (uintptr_t)(rows * d * 2);
  if (overlaps(out, ob, ml, (uintptr_t)(rows * n_chunks * 8)) || overlaps(out, ob, o, (uintptr_t)(rows * n_chunks * d * 4)))
    return fail(SMX_EINVAL, "out overlaps ml or o");
  const hipError_t err = launch_wmerge(ml, o, rows, n_chunks, d, (int)dtype, (char*)out, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "kernel launch");
  return ok();
}

int smx_stream_copy(const void* x, void* y, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return fail(SMX_EINVAL, "bytes (%lld) must be a non-negative multiple of 16", (long long)bytes);
  if (bytes == 0) return ok();
  if (x == nullptr || y == nullptr) return fail(SMX_EINVAL, "x and y must not be NULL");
  if ((uintptr_t)x % 16 != 0 || (uintptr_t)y % 16 != 0) return fail(SMX_EINVAL, "x and y must be 16-byte aligned");
  if (overlaps(x, (uintptr_t)bytes, y, (uintptr_t)bytes)) return fail(SMX_EINVAL, "x and y overlap");
  const hipError_t err = launch_stream_copy(x, y, bytes / 16, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail(err, "kernel launch");
  return ok();
}

const char* smx_last_error(void) { return g_err; }

}  // extern "C"
