// k_copy.hip — a plain streaming copy, the reference for the HBM rate this
// GPU reaches on a given footprint. It is no step of the softmax: bench.py
// times it on the same bytes and buffer rotation as the row kernels, so the
// row kernels' bandwidth can be read against what a bare copy achieves.
//
// Two shapes, both with nontemporal 16-byte loads and stores. Below 1 GiB a
// grid-stride loop over 1024 workgroups of 256 threads: a sweep of grid
// sizes (1024 to 16384 workgroups), of several packs in flight per thread,
// of one workgroup per row, and of ordinary instead of nontemporal accesses
// found none faster on 67 MB in + 67 MB out. From 1 GiB, one workgroup per
// 16 KiB with the XCDs' contiguous order: the XCDs take workgroups
// round-robin (workgroup i runs on XCD i mod 8), and workgroup i copies the
// chunk of logical workgroup (i mod 8) G/8 + i / 8, so each XCD streams
// through its own eighth of the buffer. Measured on 1 / 2 / 4 GiB copies:
// 5519 / 5410 / 5312 GB/s for the grid-stride loop, 5798 / 5839 / 5828 GB/s
// for this shape.
#include "smx_device.hpp"

namespace smx {
namespace {

constexpr int64_t kCopyGrid = 1024;
constexpr int64_t kChunkPacks = 1024;                // 16 KiB per workgroup
constexpr int64_t kChunkedMinBytes = (int64_t)1 << 30;

__global__ __launch_bounds__(kThreads) void k_stream_copy(const u32x4* __restrict__ x, u32x4* __restrict__ y,
                                                           int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
    __builtin_nontemporal_store(__builtin_nontemporal_load(x + i), y + i);
  }
}

// the grid is a multiple of 8 (padded: chunks past the buffer copy nothing)
__global__ __launch_bounds__(kThreads) void k_stream_copy_xcd(const u32x4* __restrict__ x, u32x4* __restrict__ y,
                                                               int64_t n16) {
  const unsigned nb = gridDim.x;
  const unsigned b = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  const int64_t base = (int64_t)b * kChunkPacks;
#pragma unroll
  for (int k = 0; k < kChunkPacks / kThreads; ++k) {
    const int64_t i = base + k * kThreads + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(x + i), y + i);
  }
}

}  // namespace

hipError_t launch_stream_copy(const void* x, void* y, int64_t n16, hipStream_t stream) {
  if (n16 * 16 >= kChunkedMinBytes) {
    // a launch's work-items must stay below 2^32: at most 2^24 chunks
    // (buffers up to 256 GiB; larger ones take the grid-stride loop)
    const int64_t chunks = (n16 + kChunkPacks - 1) / kChunkPacks;
    const int64_t grid = (chunks + 7) / 8 * 8;
    if (grid < ((int64_t)1 << 24)) {
      hipLaunchKernelGGL(k_stream_copy_xcd, dim3((unsigned)grid), dim3(kThreads), 0, stream, (const u32x4*)x,
                         (u32x4*)y, n16);
      return hipGetLastError();
    }
  }
  const int64_t blocks = (n16 + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(blocks < kCopyGrid ? blocks : kCopyGrid);
  hipLaunchKernelGGL(k_stream_copy, dim3(grid), dim3(kThreads), 0, stream, (const u32x4*)x, (u32x4*)y, n16);
  return hipGetLastError();
}

}  // namespace smx
