// k_wsplit.hip — softmax-weighted value sums split along the keys: per-chunk
// online states, then their merge.
//
// Each (row, chunk) is summarized by its state (m, l, o): m the chunk's
// maximum over valid finite scores, l = sum exp(s_j - m), o = sum exp(s_j - m)
// V_j; two states merge by rescaling l and o alike to the larger maximum, and
// the row's output is o / l ("Online stable softmax", sections on the
// weighted numerator and the reference summary; "Softmax numerics
// architecture", tiled attention). This is the shape of work where a group has
// few score rows and many keys (one query per head, a long context): the
// matrix-core kernel's 128-row tiles would stay mostly empty, while here the
// chunks of every group run in parallel and V streams from HBM once per
// group. The products are an HBM-bound matrix-vector product, so they run on
// the vector ALUs.
//
// k_wstates: one workgroup per (group, chunk). Rows of the group are taken
// four (or eight) at a time: their scores for the chunk become weights in LDS
// (the chunk maximum found first, so m is exact), then each thread streams
// 16-byte slices of V rows (8 value components), four loads ahead, and
// accumulates those components for each of the rows. The threads sharing components are reduced with shuffles
// inside a wave and through LDS across waves.
//
// k_wmerge: one workgroup per row; the states are folded by the merge rule
// (the side holding the maximum keeps factor 1, so an empty state (-inf, 0,
// 0) is an identity and a NaN state poisons the row) and o / l is written.
#include "smx_device.hpp"

namespace smx {
namespace {

// RP: score rows whose weights sit in LDS at once (4, or 8 for larger groups)
template <int DT, int D, int RP, bool KEEP>
__global__ __launch_bounds__(kThreads) void k_wstates(const char* __restrict__ s, const char* __restrict__ v,
                                                      int64_t rows, int64_t cols, int64_t rpg, MaskArgs mask,
                                                      int64_t chunk, int64_t nch, float* __restrict__ ml,
                                                      float* __restrict__ o) {
  constexpr int S = 2;
  constexpr int kRowsPerPass = RP;
  constexpr int KL = D / 8;             // threads covering one V row (8 components each)
  constexpr int JR = kThreads / KL;     // V rows in flight per step across the workgroup
  constexpr int kUnroll = 4;            // V loads of a thread issued ahead of their products
  extern __shared__ float wbuf[];       // RP x chunk weights
  __shared__ float part[kWaves][kRowsPerPass][D];
  __shared__ RedScratch red;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int kq = tid % KL;
  const int jr = tid / KL;
  const int64_t groups = rows / rpg;
  const int64_t total = groups * nch;

  for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
    const int64_t g = b / nch;
    const int64_t c = b - g * nch;
    const int64_t j0 = c * chunk;
    const int64_t j1 = j0 + chunk < cols ? j0 + chunk : cols;
    const int n = (int)(j1 - j0);
    const char* vg = v + (g * cols + j0) * D * S;

    for (int64_t r0 = g * rpg; r0 < (g + 1) * rpg; r0 += kRowsPerPass) {
      const int nr = (int)((g + 1) * rpg - r0 < kRowsPerPass ? (g + 1) * rpg - r0 : kRowsPerPass);
      // weights of the pass's rows: the chunk maximum over valid lanes (NaN
      // and +inf propagate and poison the state), then exp(s - m)
      float mrow[kRowsPerPass], lrow[kRowsPerPass];
      bool live[kRowsPerPass];
#pragma unroll
      for (int q = 0; q < kRowsPerPass; ++q) {
        mrow[q] = -kInf;
        lrow[q] = 0.0f;
        live[q] = false;
        if (q >= nr) continue;  // uniform across the workgroup
        const int64_t r = r0 + q;
        const int64_t prefix = valid_prefix(mask, r, cols);
        const int lim = (int)(prefix - j0 < 0 ? 0 : (prefix - j0 > n ? n : prefix - j0));
        const char* sr = s + (r * cols + j0) * S;
        float mx = -kInf;
        for (int j = tid; j < n; j += kThreads) {
          float x = -kInf;
          if (j < lim && (!KEEP || mask.keep[r * cols + j0 + j] != 0)) {
            x = dec<DT>(*reinterpret_cast<const uint16_t*>(sr + j * S));
          }
          wbuf[q * chunk + j] = x;
          mx = vmax(mx, x);
        }
        mx = block_max<kWaves>(mx, red);
        mrow[q] = mx;
        const bool poisoned = !(mx < kInf);
        live[q] = !poisoned && mx != -kInf;
        float sum = 0.0f;
        if (live[q]) {
          for (int j = tid; j < n; j += kThreads) {
            const float e = __builtin_amdgcn_exp2f((wbuf[q * chunk + j] - mx) * kLog2e);  // -inf lanes give 0
            wbuf[q * chunk + j] = e;
            sum += e;
          }
          sum = block_sum<kWaves>(sum, red);
        }
        lrow[q] = poisoned ? __builtin_nanf("") : sum;
      }
      __syncthreads();  // the weights are complete

      // o[q][k] = sum_j w[q][j] V[j][k]: this thread's 8 components kq*8 ..
      // kq*8+7 over the V rows jr, jr + JR, ...
      float acc[kRowsPerPass][8];
#pragma unroll
      for (int q = 0; q < kRowsPerPass; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[q][e] = 0.0f;
      for (int j0u = jr; j0u < n; j0u += kUnroll * JR) {
        u32x4 raw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int j = j0u + u * JR;
          raw[u] = j < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vg + ((int64_t)j * D + kq * 8) * S))
                         : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int j = j0u + u * JR;
          if (j >= n) break;
          const uint32_t ws[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
          float vv[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vv[2 * e] = dec<DT>(ws[e] & 0xFFFFu);
            vv[2 * e + 1] = dec<DT>(ws[e] >> 16);
          }
#pragma unroll
          for (int q = 0; q < kRowsPerPass; ++q) {
            if (!live[q]) continue;  // uniform
            const float wj = wbuf[q * chunk + j];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][e] = __builtin_fmaf(wj, vv[e], acc[q][e]);
          }
        }
      }
      // the wave's V rows sharing a component: lanes kq, kq + KL, ...
#pragma unroll
      for (int off = KL; off < 64; off <<= 1)
#pragma unroll
        for (int q = 0; q < kRowsPerPass; ++q)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[q][e] += __shfl_xor(acc[q][e], off);
      if (lane < KL) {
#pragma unroll
        for (int q = 0; q < kRowsPerPass; ++q)
#pragma unroll
          for (int e = 0; e < 8; ++e) part[wid][q][lane * 8 + e] = acc[q][e];
      }
      __syncthreads();
      // the waves' partials, summed in a fixed order; then the states
      for (int i = tid; i < nr * D; i += kThreads) {
        const int q = i / D, k = i - q * D;
        const int64_t r = r0 + q;
        float sum = part[0][q][k];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) sum += part[ww][q][k];
        const float val = live[q] ? sum : (mrow[q] == -kInf ? 0.0f : __builtin_nanf(""));
        o[(r * nch + c) * D + k] = val;
      }
      if (tid < nr) {
        const int64_t r = r0 + tid;
        float mv = mrow[0], lv = lrow[0];
#pragma unroll
        for (int q = 1; q < kRowsPerPass; ++q) {
          mv = tid == q ? mrow[q] : mv;
          lv = tid == q ? lrow[q] : lv;
        }
        const bool pois = !(mv < kInf);
        ml[(r * nch + c) * 2] = pois ? __builtin_nanf("") : mv;
        ml[(r * nch + c) * 2 + 1] = lv;
      }
      __syncthreads();  // w and part are reused by the next pass
    }
  }
}

// One row per workgroup: M = max m_c, factors f_c = exp(m_c - M) (exactly 1
// where m_c == M), L = sum l_c f_c, O_k = sum_c o_ck f_c in chunk order, out =
// O / L rounded to the element format. A NaN state poisons the row (canonical
// NaN in every component); a row with no valid finite score is all +0.0.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_wmerge(const float* __restrict__ ml, const float* __restrict__ o,
                                                     int64_t rows, int64_t nch, int64_t d, char* __restrict__ out) {
  extern __shared__ float fac[];  // nch factors
  __shared__ RedScratch red;
  const int tid = threadIdx.x;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const float* mr = ml + r * nch * 2;
    float mx = -kInf;
    bool bad = false;
    for (int64_t c = tid; c < nch; c += kThreads) {
      const float m = mr[2 * c], l = mr[2 * c + 1];
      if (m != m || l != l) {
        bad = true;
      } else {
        mx = fmaxf(mx, m);
      }
    }
    mx = block_max<kWaves>(bad ? kInf : mx, red);
    const bool poisoned = mx == kInf;
    char* orow = out + r * d * 2;
    if (poisoned || mx == -kInf) {
      const uint32_t fill = poisoned ? Fmt<DT>::kNaN : 0u;
      for (int64_t k = tid; k < d; k += kThreads) *reinterpret_cast<uint16_t*>(orow + k * 2) = (uint16_t)fill;
      __syncthreads();  // fac and red are reused by the next row
      continue;
    }
    float lsum = 0.0f;
    for (int64_t c = tid; c < nch; c += kThreads) {
      const float f = exp_diff(mr[2 * c], mx);
      fac[c] = f;
      lsum += mr[2 * c + 1] * f;
    }
    const float L = block_sum<kWaves>(lsum, red);  // its barriers also publish fac
    const float inv = 1.0f / L;
    for (int64_t k = tid; k < d; k += kThreads) {
      float acc = 0.0f;
      for (int64_t c = 0; c < nch; ++c) {
        const float f = fac[c];
        if (f != 0.0f) acc = __builtin_fmaf(o[(r * nch + c) * d + k], f, acc);
      }
      *reinterpret_cast<uint16_t*>(orow + k * 2) = (uint16_t)enc<DT>(acc * inv);
    }
    __syncthreads();  // fac is reused by the next row
  }
}

constexpr int64_t kMaxGrid = 1 << 20;

template <int DT, int D, int RP>
hipError_t launch_states_rp(const char* s, const char* v, int64_t rows, int64_t cols, int64_t rpg,
                            const MaskArgs& mask, int64_t chunk, int64_t nch, float* ml, float* o, hipStream_t st) {
  const int64_t total = rows / rpg * nch;
  const unsigned grid = (unsigned)(total < kMaxGrid ? total : kMaxGrid);
  const size_t lds = (size_t)RP * (size_t)chunk * sizeof(float);
  if (mask.kind == kMaskKeep) {
    hipLaunchKernelGGL((k_wstates<DT, D, RP, true>), dim3(grid), dim3(kThreads), lds, st, s, v, rows, cols, rpg,
                       mask, chunk, nch, ml, o);
  } else {
    hipLaunchKernelGGL((k_wstates<DT, D, RP, false>), dim3(grid), dim3(kThreads), lds, st, s, v, rows, cols, rpg,
                       mask, chunk, nch, ml, o);
  }
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_states_d(const char* s, const char* v, int64_t rows, int64_t cols, int64_t rpg,
                           const MaskArgs& mask, int64_t chunk, int64_t nch, float* ml, float* o, hipStream_t st) {
  if (rpg > 4) return launch_states_rp<DT, D, 8>(s, v, rows, cols, rpg, mask, chunk, nch, ml, o, st);
  return launch_states_rp<DT, D, 4>(s, v, rows, cols, rpg, mask, chunk, nch, ml, o, st);
}

template <int DT>
hipError_t launch_states_dt(const char* s, const char* v, int64_t rows, int64_t cols, int64_t d, int64_t rpg,
                            const MaskArgs& mask, int64_t chunk, int64_t nch, float* ml, float* o, hipStream_t st) {
  if (d == 32) return launch_states_d<DT, 32>(s, v, rows, cols, rpg, mask, chunk, nch, ml, o, st);
  if (d == 64) return launch_states_d<DT, 64>(s, v, rows, cols, rpg, mask, chunk, nch, ml, o, st);
  return launch_states_d<DT, 128>(s, v, rows, cols, rpg, mask, chunk, nch, ml, o, st);
}

}  // namespace

hipError_t launch_wstates(const char* s, const char* v, int64_t rows, int64_t cols, int64_t d, int64_t rpg,
                          int dtype, const MaskArgs& mask, int64_t chunk, int64_t nch, float* ml, float* o,
                          hipStream_t stream) {
  return dtype == kF16 ? launch_states_dt<kF16>(s, v, rows, cols, d, rpg, mask, chunk, nch, ml, o, stream)
                       : launch_states_dt<kBF16>(s, v, rows, cols, d, rpg, mask, chunk, nch, ml, o, stream);
}

hipError_t launch_wmerge(const float* ml, const float* o, int64_t rows, int64_t nch, int64_t d, int dtype, char* out,
                         hipStream_t stream) {
  const unsigned grid = (unsigned)(rows < kMaxGrid ? rows : kMaxGrid);
  const size_t lds = (size_t)nch * sizeof(float);
  if (dtype == kF16) {
    hipLaunchKernelGGL(k_wmerge<kF16>, dim3(grid), dim3(kThreads), lds, stream, ml, o, rows, nch, d, out);
  } else {
    hipLaunchKernelGGL(k_wmerge<kBF16>, dim3(grid), dim3(kThreads), lds, stream, ml, o, rows, nch, d, out);
  }
  return hipGetLastError();
}

}  // namespace smx
