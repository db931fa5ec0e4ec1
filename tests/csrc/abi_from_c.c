/*
 * abi_from_c.c — drives the library through include/smx.h from plain C, the
 * way a caller with no Python would: device buffers from hipMalloc, one
 * non-default stream, every entry point, results copied back.
 *
 * usage: abi_from_c <inputs.bin> <outputs.bin>
 *
 * inputs.bin (little-endian):
 *   int64 rows, cols, wrows, wcols, d, rows_per_group, chunk_cols
 *   float  x[rows*cols]          logits (f32)
 *   int32  valid_len[rows]
 *   uint16 xb[rows*cols]         logits (bf16 bits)
 *   int32  target[rows]
 *   float  g[rows*cols]          upstream gradient (f32)
 *   uint16 s[wrows*wcols]        scores (bf16 bits)
 *   uint16 v[wrows/rows_per_group * wcols * d]   values (bf16 bits)
 * outputs.bin, in this order:
 *   float  y[rows*cols]          softmax_rows(x, valid_len)
 *   float  y2[rows*cols]         softmax_row_stats + softmax_merge_normalize
 *   uint16 logp[rows*cols]       log_softmax_rows(xb, valid_len)
 *   float  lse[rows]
 *   float  loss[rows]            softmax_cross_entropy_rows(xb, target)
 *   uint16 dxb[rows*cols]
 *   float  dx[rows*cols]         softmax_backward_rows(y, g)
 *   uint16 o[wrows*d]            softmax_weighted_rows(s, v), causal per group
 *   uint16 o2[wrows*d]           softmax_weighted_states (chunks of 64 keys) +
 *                                softmax_weighted_merge, the same sums
 * The _path variants (with SMX_PATH_AUTO) are checked here to equal their
 * plain calls bit for bit, smx_stream_copy to reproduce its input exactly,
 * and the two host helpers to return a path and a chunk width.
 * Exit status 0 only if every call returned SMX_OK, every check held and an
 * invalid call was rejected with SMX_EINVAL and a message.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "smx.h"

static void die(const char* what) {
  fprintf(stderr, "abi_from_c: %s\n", what);
  exit(1);
}

static void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "abi_from_c: %s: %s\n", what, hipGetErrorString(e));
    exit(1);
  }
}

static void smx_check(int rc, const char* what) {
  if (rc != SMX_OK) {
    fprintf(stderr, "abi_from_c: %s returned %d: %s\n", what, rc, smx_last_error());
    exit(1);
  }
}

static void* read_block(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p == NULL) die("out of host memory");
  if (bytes && fread(p, 1, bytes, f) != bytes) die("short input file");
  return p;
}

static void* to_device(const void* h, size_t bytes) {
  void* d = NULL;
  hip_check(hipMalloc(&d, bytes ? bytes : 16), "hipMalloc");
  if (bytes) hip_check(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice), "hipMemcpy to device");
  return d;
}

static void* device_buffer(size_t bytes) {
  void* d = NULL;
  hip_check(hipMalloc(&d, bytes ? bytes : 16), "hipMalloc");
  return d;
}

/* the device buffers a and b hold the same bytes */
static void same_bytes(const void* a, const void* b, size_t bytes, const char* what) {
  unsigned char* ha = (unsigned char*)malloc(bytes ? bytes : 1);
  unsigned char* hb = (unsigned char*)malloc(bytes ? bytes : 1);
  if (ha == NULL || hb == NULL) die("out of host memory");
  if (bytes) {
    hip_check(hipMemcpy(ha, a, bytes, hipMemcpyDeviceToHost), "hipMemcpy to host");
    hip_check(hipMemcpy(hb, b, bytes, hipMemcpyDeviceToHost), "hipMemcpy to host");
  }
  if (memcmp(ha, hb, bytes) != 0) {
    fprintf(stderr, "abi_from_c: %s differ\n", what);
    exit(1);
  }
  free(ha);
  free(hb);
}

static void write_back(FILE* f, const void* d, size_t bytes) {
  void* h = malloc(bytes ? bytes : 1);
  if (h == NULL) die("out of host memory");
  if (bytes) hip_check(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost), "hipMemcpy to host");
  if (bytes && fwrite(h, 1, bytes, f) != bytes) die("short write");
  free(h);
}

int main(int argc, char** argv) {
  if (argc != 3) die("usage: abi_from_c <inputs.bin> <outputs.bin>");
  FILE* in = fopen(argv[1], "rb");
  if (in == NULL) die("cannot open the input file");
  int64_t hdr[7];
  if (fread(hdr, sizeof hdr, 1, in) != 1) die("short header");
  const int64_t rows = hdr[0], cols = hdr[1], wrows = hdr[2], wcols = hdr[3], d = hdr[4], rpg = hdr[5],
                chunk = hdr[6];
  if (rows <= 0 || cols <= 0 || wrows <= 0 || wcols <= 0 || d <= 0 || rpg <= 0 || chunk <= 0 || wrows % rpg)
    die("bad header");
  const size_t n = (size_t)(rows * cols), wn = (size_t)(wrows * wcols), vn = (size_t)(wrows / rpg * wcols * d);
  const int64_t nch = (cols + chunk - 1) / chunk;

  void* h_x = read_block(in, n * 4);
  void* h_vl = read_block(in, (size_t)rows * 4);
  void* h_xb = read_block(in, n * 2);
  void* h_tgt = read_block(in, (size_t)rows * 4);
  void* h_g = read_block(in, n * 4);
  void* h_s = read_block(in, wn * 2);
  void* h_v = read_block(in, vn * 2);
  fclose(in);

  void* x = to_device(h_x, n * 4);
  int32_t* vl = (int32_t*)to_device(h_vl, (size_t)rows * 4);
  void* xb = to_device(h_xb, n * 2);
  int32_t* tgt = (int32_t*)to_device(h_tgt, (size_t)rows * 4);
  void* g = to_device(h_g, n * 4);
  void* s = to_device(h_s, wn * 2);
  void* v = to_device(h_v, vn * 2);
  void* y = device_buffer(n * 4);
  void* y2 = device_buffer(n * 4);
  smx_stat* stats = (smx_stat*)device_buffer((size_t)(rows * nch) * sizeof(smx_stat));
  void* logp = device_buffer(n * 2);
  float* lse = (float*)device_buffer((size_t)rows * 4);
  float* loss = (float*)device_buffer((size_t)rows * 4);
  void* dxb = device_buffer(n * 2);
  void* dx = device_buffer(n * 4);
  void* o = device_buffer((size_t)(wrows * d) * 2);
  const int64_t wchunk = 64, wnch = (wcols + wchunk - 1) / wchunk;
  float* wml = (float*)device_buffer((size_t)(wrows * wnch) * 2 * sizeof(float));
  float* wo = (float*)device_buffer((size_t)(wrows * wnch * d) * sizeof(float));
  void* o2 = device_buffer((size_t)(wrows * d) * 2);

  hipStream_t st;
  hip_check(hipStreamCreate(&st), "hipStreamCreate");
  smx_mask by_len;
  memset(&by_len, 0, sizeof by_len);
  by_len.kind = SMX_MASK_VALID_LEN;
  by_len.valid_len = vl;
  smx_mask causal;
  memset(&causal, 0, sizeof causal);
  causal.kind = SMX_MASK_CAUSAL;
  causal.causal_period = rpg;

  smx_check(softmax_rows(x, y, rows, cols, SMX_F32, &by_len, st), "softmax_rows");
  smx_check(softmax_row_stats(x, rows, cols, SMX_F32, &by_len, chunk, stats, st), "softmax_row_stats");
  smx_check(softmax_merge_normalize(x, y2, rows, cols, SMX_F32, &by_len, chunk, stats, nch, st),
            "softmax_merge_normalize");
  smx_check(log_softmax_rows(xb, logp, lse, rows, cols, SMX_BF16, &by_len, st), "log_softmax_rows");
  smx_check(softmax_cross_entropy_rows(xb, tgt, loss, dxb, rows, cols, SMX_BF16, NULL, st),
            "softmax_cross_entropy_rows");
  smx_check(softmax_backward_rows(y, g, dx, rows, cols, SMX_F32, st), "softmax_backward_rows");
  smx_check(softmax_weighted_rows(s, v, o, wrows, wcols, d, rpg, SMX_BF16, &causal, st), "softmax_weighted_rows");
  smx_check(softmax_weighted_states(s, v, wrows, wcols, d, rpg, SMX_BF16, &causal, wchunk, wml, wo, st),
            "softmax_weighted_states");
  smx_check(softmax_weighted_merge(wml, wo, wrows, wnch, d, SMX_BF16, o2, st), "softmax_weighted_merge");

  /* the _path variants with the automatic path: the same dispatch, bit for bit */
  void* ya = device_buffer(n * 4);
  void* logpa = device_buffer(n * 2);
  float* lsea = (float*)device_buffer((size_t)rows * 4);
  float* lossa = (float*)device_buffer((size_t)rows * 4);
  void* dxba = device_buffer(n * 2);
  void* dxa = device_buffer(n * 4);
  smx_check(softmax_rows_path(x, ya, rows, cols, SMX_F32, &by_len, SMX_PATH_AUTO, 0, st), "softmax_rows_path");
  smx_check(log_softmax_rows_path(xb, logpa, lsea, rows, cols, SMX_BF16, &by_len, SMX_PATH_AUTO, 0, st),
            "log_softmax_rows_path");
  smx_check(softmax_cross_entropy_rows_path(xb, tgt, lossa, dxba, rows, cols, SMX_BF16, NULL, SMX_PATH_AUTO, 0, st),
            "softmax_cross_entropy_rows_path");
  smx_check(softmax_backward_rows_path(y, g, dxa, rows, cols, SMX_F32, SMX_PATH_AUTO, 0, st),
            "softmax_backward_rows_path");
  /* the streaming copy (the bandwidth reference) of the bf16 logits' whole 16-byte packs */
  const size_t cbytes = (n * 2) / 16 * 16;
  void* xc = device_buffer(n * 2);
  smx_check(smx_stream_copy(xb, xc, (int64_t)cbytes, st), "smx_stream_copy");
  const smx_path pth = softmax_select_path(rows, cols, SMX_F32);
  if (pth != SMX_PATH_WAVE && pth != SMX_PATH_LDS && pth != SMX_PATH_SPLIT) die("softmax_select_path");
  if (softmax_default_chunk_cols(rows, cols, SMX_F32) <= 0) die("softmax_default_chunk_cols");
  hip_check(hipStreamSynchronize(st), "hipStreamSynchronize");
  same_bytes(y, ya, n * 4, "softmax_rows and softmax_rows_path");
  same_bytes(logp, logpa, n * 2, "log_softmax_rows and log_softmax_rows_path (y)");
  same_bytes(lse, lsea, (size_t)rows * 4, "log_softmax_rows and log_softmax_rows_path (lse)");
  same_bytes(loss, lossa, (size_t)rows * 4, "the cross-entropy losses");
  same_bytes(dxb, dxba, n * 2, "the cross-entropy gradients");
  same_bytes(dx, dxa, n * 4, "softmax_backward_rows and softmax_backward_rows_path");
  same_bytes(xb, xc, cbytes, "smx_stream_copy's input and output");

  /* an invalid element type is rejected before anything is enqueued */
  const int bad = softmax_rows(x, y, rows, cols, (smx_dtype)7, NULL, st);
  if (bad != SMX_EINVAL || smx_last_error()[0] == '\0') die("an invalid dtype was not rejected");
  printf("rejected: %s\n", smx_last_error());

  hip_check(hipStreamSynchronize(st), "hipStreamSynchronize");
  FILE* out = fopen(argv[2], "wb");
  if (out == NULL) die("cannot open the output file");
  write_back(out, y, n * 4);
  write_back(out, y2, n * 4);
  write_back(out, logp, n * 2);
  write_back(out, lse, (size_t)rows * 4);
  write_back(out, loss, (size_t)rows * 4);
  write_back(out, dxb, n * 2);
  write_back(out, dx, n * 4);
  write_back(out, o, (size_t)(wrows * d) * 2);
  write_back(out, o2, (size_t)(wrows * d) * 2);
  fclose(out);
  hip_check(hipStreamDestroy(st), "hipStreamDestroy");
  void* bufs[] = {x, vl, xb, tgt, g, s, v, y, y2, stats, logp, lse, loss, dxb, dx, o, wml, wo, o2,
                  ya, logpa, lsea, lossa, dxba, dxa, xc};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) hip_check(hipFree(bufs[i]), "hipFree");
  free(h_x);
  free(h_vl);
  free(h_xb);
  free(h_tgt);
  free(h_g);
  free(h_s);
  free(h_v);
  printf("ok\n");
  return 0;
}
