// k_backward.hip — the softmax vector-Jacobian product, row by row:
//   dx_j = p_j * (g_j - s),   s = sum_k g_k p_k
// ("Softmax numerics architecture", section on the Jacobian: the dense
// Jacobian diag(p) - p p^T is never formed; the product reduces to one dot
// product per row and one elementwise pass).
//
// p is a forward output (masked lanes are 0 there, so their dx is 0) and g
// the incoming gradient, both in the element format. The dot product is
// accumulated in fp32 with Kahan compensation over rounded products, then
// summed across lanes as compensated pairs. A NaN anywhere in a row's p or g
// makes the row's dx the canonical NaN.
//
// Paths: one wave per row (registers), one workgroup per row (registers),
// and for rows beyond that two passes: per-chunk partial dot products, then
// each chunk merges its row's partials and writes dx (p and g read twice).
#include "smx_device.hpp"

namespace smx {
namespace {

struct BwdArgs {
  const char* p;
  const char* g;
  char* dx;
  int64_t rows;
  int64_t cols;
};

// a NaN result becomes the canonical quiet NaN before rounding (0x7FC00000
// rounds to the canonical fp16 / bf16 NaN)
__device__ __forceinline__ float canon(float v) { return v != v ? u2f(0x7FC00000u) : v; }

// one workgroup of NT threads per row (NT = 64: one wave per row)
template <int DT, int E, int NT, int VPT>
__global__ __launch_bounds__(NT) void k_bwd_rows(BwdArgs a) {
  constexpr int S = Fmt<DT>::S;
  constexpr int NW = NT / 64;
  __shared__ RedScratch red;
  const int tid = threadIdx.x;
  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const int64_t base = row * a.cols;
    float pv[VPT][E], gv[VPT][E];
    KahanSum dot;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int64_t j0 = ((int64_t)k * NT + tid) * E;
      Pack<DT, E> pp, gg;
      pp.fill(0);
      gg.fill(0);
      if (j0 < a.cols) {
        pp.template load<true>(a.p + (base + j0) * S);
        gg.template load<true>(a.g + (base + j0) * S);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        pv[k][e] = pp.get(e);
        gv[k][e] = gg.get(e);
        dot.add(pv[k][e] * gv[k][e]);
      }
    }
    float s;
    if constexpr (NW == 1) {
      s = wave_sum_pair(dot.hi(), dot.lo());
    } else {
      s = block_sum_pair<NW>(dot.hi(), dot.lo(), red);
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int64_t j0 = ((int64_t)k * NT + tid) * E;
      if (j0 < a.cols) {
        float o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = canon(pv[k][e] * (gv[k][e] - s));
        Pack<DT, E> out;
        out.put_values(o);
        out.template store<true>(a.dx + (base + j0) * S);
      }
    }
  }
}

// pass 1 of the long-row path: the partial dot product of each (row, chunk)
// as a compensated pair
template <int DT, int E, int VPT>
__global__ __launch_bounds__(kThreads) void k_bwd_dot(BwdArgs a, int64_t chunk, int64_t nch, float2* part) {
  constexpr int S = Fmt<DT>::S;
  constexpr int64_t kRound = (int64_t)kThreads * VPT * E;
  __shared__ RedScratch red;
  const int tid = threadIdx.x;
  for (int64_t b = blockIdx.x; b < a.rows * nch; b += gridDim.x) {
    const int64_t row = b / nch;
    const int64_t c = b - row * nch;
    const int64_t j_lo = c * chunk;
    const int64_t j_hi = j_lo + chunk < a.cols ? j_lo + chunk : a.cols;
    const int64_t base = row * a.cols;
    KahanSum dot;
    for (int64_t r0 = j_lo; r0 < j_hi; r0 += kRound) {
      Pack<DT, E> pp[VPT], gg[VPT];
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int64_t j0 = r0 + ((int64_t)k * kThreads + tid) * E;
        pp[k].fill(0);
        gg[k].fill(0);
        if (j0 < j_hi) {
          pp[k].load(a.p + (base + j0) * S);
          gg[k].load(a.g + (base + j0) * S);
        }
      }
#pragma unroll
      for (int k = 0; k < VPT; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) dot.add(pp[k].get(e) * gg[k].get(e));
    }
    // pairs across the workgroup, kept as (hi, lo)
    float hi = dot.hi(), lo = dot.lo();
    pair_step<kDppXor1>(hi, lo);
    pair_step<kDppXor2>(hi, lo);
    pair_step<kDppHalfMirror>(hi, lo);
    pair_step<kDppMirror>(hi, lo);
    float h0 = lane_read(hi, 0), l0 = lane_read(lo, 0);
    float h1 = lane_read(hi, 16), l1 = lane_read(lo, 16);
    float h2 = lane_read(hi, 32), l2 = lane_read(lo, 32);
    float h3 = lane_read(hi, 48), l3 = lane_read(lo, 48);
    pair_add(h0, l0, h1, l1);
    pair_add(h2, l2, h3, l3);
    pair_add(h0, l0, h2, l2);
    if ((tid & 63) == 0) {
      red.a[tid >> 6] = h0;
      red.b[tid >> 6] = l0;
    }
    __syncthreads();
    if (tid == 0) {
      float rh = red.a[0], rl = red.b[0];
#pragma unroll
      for (int i = 1; i < kWaves; ++i) pair_add(rh, rl, red.a[i], red.b[i]);
      part[b] = make_float2(rh, rl);
    }
    __syncthreads();
  }
}

// pass 2: merge the row's nsum partials (compensated, fixed order; every
// chunk's, or the one pair k_bwd_row_sum left), write dx
template <int DT, int E, int VPT>
__global__ __launch_bounds__(kThreads) void k_bwd_apply(BwdArgs a, int64_t chunk, int64_t nch, const float2* part,
                                                        int64_t nsum) {
  constexpr int S = Fmt<DT>::S;
  constexpr int64_t kRound = (int64_t)kThreads * VPT * E;
  __shared__ RedScratch red;
  const int tid = threadIdx.x;
  for (int64_t b = blockIdx.x; b < a.rows * nch; b += gridDim.x) {
    const int64_t row = b / nch;
    const int64_t c = b - row * nch;
    const int64_t j_lo = c * chunk;
    const int64_t j_hi = j_lo + chunk < a.cols ? j_lo + chunk : a.cols;
    const int64_t base = row * a.cols;
    float hi = 0.0f, lo = 0.0f;
    for (int64_t i = tid; i < nsum; i += kThreads) {
      const float2 q = part[row * nsum + i];
      pair_add(hi, lo, q.x, q.y);
    }
    const float s = block_sum_pair<kWaves>(hi, lo, red);
    for (int64_t r0 = j_lo; r0 < j_hi; r0 += kRound) {
      Pack<DT, E> pp[VPT], gg[VPT];
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int64_t j0 = r0 + ((int64_t)k * kThreads + tid) * E;
        pp[k].fill(0);
        gg[k].fill(0);
        if (j0 < j_hi) {
          pp[k].template load<true>(a.p + (base + j0) * S);
          gg[k].template load<true>(a.g + (base + j0) * S);
        }
      }
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int64_t j0 = r0 + ((int64_t)k * kThreads + tid) * E;
        if (j0 < j_hi) {
          float o[E];
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = canon(pp[k].get(e) * (gg[k].get(e) - s));
          Pack<DT, E> out;
          out.put_values(o);
          out.template store<true>(a.dx + (base + j0) * S);
        }
      }
    }
  }
}

// Rows with many chunks sum their partials once, here, instead of once in
// every chunk's workgroup of pass 2: the same per-thread order and the same
// tree as k_bwd_apply, left as the (hi, lo) pair, which pass 2 then adds to
// zeros exactly, so dx is bitwise the same. A thread's loads are issued
// eight at a time, ahead of the dependent additions.
__global__ __launch_bounds__(kThreads) void k_bwd_row_sum(const float2* part, int64_t rows, int64_t nch,
                                                          float2* merged) {
  constexpr int kBatch = 8;
  __shared__ RedScratch red;
  const int tid = threadIdx.x;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const float2* rp = part + row * nch;
    float hi = 0.0f, lo = 0.0f;
    for (int64_t i0 = tid; i0 < nch; i0 += (int64_t)kBatch * kThreads) {
      float2 q[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int64_t i = i0 + (int64_t)k * kThreads;
        q[k] = i < nch ? rp[i] : make_float2(0.0f, 0.0f);
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        if (i0 + (int64_t)k * kThreads >= nch) break;
        pair_add(hi, lo, q[k].x, q[k].y);
      }
    }
    block_pair_reduce<kWaves>(hi, lo, red);
    if (tid == 0) merged[row] = make_float2(hi, lo);
  }
}

constexpr int64_t kMaxGrid = 1 << 20;

template <int DT, int E>
hipError_t launch_rows_t(const BwdArgs& a, bool wave, hipStream_t s) {
  const unsigned grid = (unsigned)(a.rows < kMaxGrid ? a.rows : kMaxGrid);
  if (wave) {
    const int64_t need = (a.cols + 64 * E - 1) / (64 * E);
    if (need <= 2) {
      hipLaunchKernelGGL((k_bwd_rows<DT, E, 64, 2>), dim3(grid), dim3(64), 0, s, a);
    } else if (need <= 4) {
      hipLaunchKernelGGL((k_bwd_rows<DT, E, 64, 4>), dim3(grid), dim3(64), 0, s, a);
    } else {
      hipLaunchKernelGGL((k_bwd_rows<DT, E, 64, 8>), dim3(grid), dim3(64), 0, s, a);
    }
  } else {
    const int64_t need = (a.cols + kThreads * E - 1) / (kThreads * E);
    if (need <= 2) {
      hipLaunchKernelGGL((k_bwd_rows<DT, E, kThreads, 2>), dim3(grid), dim3(kThreads), 0, s, a);
    } else if (need <= 4) {
      hipLaunchKernelGGL((k_bwd_rows<DT, E, kThreads, 4>), dim3(grid), dim3(kThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL((k_bwd_rows<DT, E, kThreads, 8>), dim3(grid), dim3(kThreads), 0, s, a);
    }
  }
  return hipGetLastError();
}

template <int DT, int E>
hipError_t launch_split_t(const BwdArgs& a, int64_t chunk, int64_t nch, float2* part, hipStream_t s) {
  constexpr int VPT = E == 1 ? 8 : 4;
  const int64_t total = a.rows * nch;
  const unsigned grid = (unsigned)(total < kMaxGrid ? total : kMaxGrid);
  hipLaunchKernelGGL((k_bwd_dot<DT, E, VPT>), dim3(grid), dim3(kThreads), 0, s, a, chunk, nch, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nch > kRowMergeMinChunks) {
    float2* const merged = part + a.rows * nch;
    const unsigned rgrid = (unsigned)(a.rows < kMaxGrid ? a.rows : kMaxGrid);
    hipLaunchKernelGGL(k_bwd_row_sum, dim3(rgrid), dim3(kThreads), 0, s, (const float2*)part, a.rows, nch, merged);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_bwd_apply<DT, E, VPT>), dim3(grid), dim3(kThreads), 0, s, a, chunk, nch,
                       (const float2*)merged, (int64_t)1);
  } else {
    hipLaunchKernelGGL((k_bwd_apply<DT, E, VPT>), dim3(grid), dim3(kThreads), 0, s, a, chunk, nch,
                       (const float2*)part, nch);
  }
  return hipGetLastError();
}

}  // namespace

int64_t bwd_wave_max_cols(int dtype, bool vec) { return 64 * 8 * (vec ? vec_elems(dtype) : 1); }
int64_t bwd_block_max_cols(int dtype, bool vec) { return (int64_t)kThreads * 8 * (vec ? vec_elems(dtype) : 1); }

hipError_t launch_bwd_rows(const char* p, const char* g, char* dx, int64_t rows, int64_t cols, int dtype,
                           bool vec, bool wave, hipStream_t s) {
  const BwdArgs a{p, g, dx, rows, cols};
  switch (dtype) {
    case kF32:
      return vec ? launch_rows_t<kF32, 4>(a, wave, s) : launch_rows_t<kF32, 1>(a, wave, s);
    case kF16:
      return vec ? launch_rows_t<kF16, 8>(a, wave, s) : launch_rows_t<kF16, 1>(a, wave, s);
    default:
      return vec ? launch_rows_t<kBF16, 8>(a, wave, s) : launch_rows_t<kBF16, 1>(a, wave, s);
  }
}

hipError_t launch_bwd_split(const char* p, const char* g, char* dx, int64_t rows, int64_t cols, int dtype, bool vec,
                            int64_t chunk, int64_t nch, float2* part, hipStream_t s) {
  const BwdArgs a{p, g, dx, rows, cols};
  switch (dtype) {
    case kF32:
      return vec ? launch_split_t<kF32, 4>(a, chunk, nch, part, s) : launch_split_t<kF32, 1>(a, chunk, nch, part, s);
    case kF16:
      return vec ? launch_split_t<kF16, 8>(a, chunk, nch, part, s) : launch_split_t<kF16, 1>(a, chunk, nch, part, s);
    default:
      return vec ? launch_split_t<kBF16, 8>(a, chunk, nch, part, s) : launch_split_t<kBF16, 1>(a, chunk, nch, part, s);
  }
}

}  // namespace smx
