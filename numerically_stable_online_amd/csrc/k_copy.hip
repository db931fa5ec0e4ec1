// k_copy.hip — a plain streaming copy, the reference for the HBM rate this
// GPU reaches on a given footprint. It is no step of the softmax: bench.py
// times it on the same bytes and buffer rotation as the row kernels, so the
// row kernels' bandwidth can be read against what a bare copy achieves.
//
// Shape: a grid-stride loop, one nontemporal 16-byte load and store per
// thread per step, 1024 workgroups of 256 threads. A sweep of grid sizes
// (1024 to 16384 workgroups), of several packs in flight per thread, of one
// workgroup per row, and of ordinary instead of nontemporal accesses found
// none faster on 67 MB in + 67 MB out.
#include "smx_device.hpp"

namespace smx {
namespace {

constexpr int64_t kCopyGrid = 1024;

__global__ __launch_bounds__(kThreads) void k_stream_copy(const u32x4* __restrict__ x, u32x4* __restrict__ y,
                                                           int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
    __builtin_nontemporal_store(__builtin_nontemporal_load(x + i), y + i);
  }
}

}  // namespace

hipError_t launch_stream_copy(const void* x, void* y, int64_t n16, hipStream_t stream) {
  const int64_t blocks = (n16 + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(blocks < kCopyGrid ? blocks : kCopyGrid);
  hipLaunchKernelGGL(k_stream_copy, dim3(grid), dim3(kThreads), 0, stream, (const u32x4*)x, (u32x4*)y, n16);
  return hipGetLastError();
}

}  // namespace smx
