// k_split.hip — the split-row path for rows larger than on-chip storage.
//
// Pass 1 (k_stats): one workgroup per (row, chunk) reads its chunk once and
// writes the chunk summary (m, l): m the chunk maximum, l the sum of
// exp(x - m) ("Stable softmax: keep the normalizer consistent as tiles
// arrive", block-merge paragraph). Within the workgroup every thread keeps
// its own running (m, l) over rounds of register-resident packs with the
// tiled recurrence of "Kernel visualization: online softmax", section
// "Tiled version", and the thread summaries are merged with the two-block
// rule of "Online stable softmax" in a fixed DPP/LDS tree.
//
// Pass 2 (k_merge_normalize): every workgroup of a row merges that row's
// summaries (the same rule; (-inf, 0) is an identity and a NaN summary
// poisons the row), then rereads its chunk and writes exp(x - M) / L. The
// reread is the second HBM read that online softmax does not remove
// ("Kernel visualization: online softmax", section "Online softmax: two
// passes").
#include "smx_device.hpp"

namespace smx {
namespace {

constexpr int kVptScalar = 16;  // packs per thread per round for single-element packs

template <int DT, int E>
constexpr int vpt() {
  return E == 1 ? kVptScalar : (DT == kF32 ? 16 : 8);
}

template <int DT, int E, bool KEEP>
__global__ __launch_bounds__(kThreads) void k_stats(RowArgs a, int64_t chunk, int64_t nch, smx_stat* stats) {
  constexpr int S = Fmt<DT>::S;
  constexpr bool ACC = DT == kF32;
  constexpr int VPT = vpt<DT, E>();
  constexpr int64_t kRound = (int64_t)kThreads * VPT * E;
  __shared__ RedScratch red;
  const int tid = threadIdx.x;
  const int64_t total = a.rows * nch;
  for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
    const int64_t row = b / nch;
    const int64_t c = b - row * nch;
    const int64_t j_lo = c * chunk;
    const int64_t j_hi = j_lo + chunk < a.cols ? j_lo + chunk : a.cols;
    const int64_t prefix = valid_prefix(a.mask, row, a.cols);
    const int64_t lim = j_hi < prefix ? j_hi : prefix;
    const char* xr = a.x + row * a.cols * S;

    float m_t = -kInf, l_t = 0.0f;  // l_t scaled by 2^64
    bool bad = false;
    for (int64_t base = j_lo; base < lim; base += kRound) {
      float v[VPT][E];
      float mr = -kInf;
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int64_t j0 = base + (int64_t)(k * kThreads + tid) * E;
        Pack<DT, E> p;
        p.fill(0);
        uint64_t kb = ~0ull;
        const bool ld = j0 < lim;
        if (ld) {
          p.load(xr + j0 * S);
          if constexpr (KEEP) kb = load_keep<E>(a.mask.keep + row * a.cols + j0);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool ok = ld && (j0 + e < lim) && (!KEEP || keep_lane(kb, e));
          const float f = ok ? p.get(e) : -kInf;
          bad |= !(f < kInf);
          mr = fmaxf(mr, f);
          v[k][e] = f;
        }
      }
      const float m_new = fmaxf(m_t, mr);
      if (m_new != -kInf) {
        // correct the running sum, then add this round against m_new
        float add;
        if constexpr (ACC) {
          KahanSum ks;
#pragma unroll
          for (int k = 0; k < VPT; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e) ks.add(exp_acc_b64(v[k][e], m_new));
          add = ks.hi() + ks.lo();
        } else {
          float s = 0.0f;
#pragma unroll
          for (int k = 0; k < VPT; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e) s += exp_hw_b64(v[k][e], m_new);
          add = s;
        }
        l_t = l_t * exp_diff(m_t, m_new) + add;
        m_t = m_new;
      }
    }
    // thread summaries -> chunk summary; NaN/inf poisons the chunk
    const bool poisoned = block_any<kWaves>(bad, red);
    float m = m_t, l = l_t;
    block_merge<kWaves>(m, l, red);
    if (tid == 0) {
      smx_stat s;
      if (poisoned) {
        s.m = __builtin_nanf("");
        s.l = __builtin_nanf("");
      } else if (m == -kInf) {
        s.m = -kInf;
        s.l = 0.0f;
      } else {
        s.m = m;
        s.l = l * 5.42101086242752217e-20f;  // remove the 2^64 scale (exact)
      }
      stats[b] = s;
    }
  }
}

template <int DT, int E, bool KEEP>
__global__ __launch_bounds__(kThreads) void k_merge_normalize(RowArgs a, int64_t chunk, int64_t nch,
                                                              const smx_stat* stats) {
  constexpr int S = Fmt<DT>::S;
  constexpr bool ACC = DT == kF32;
  constexpr int VPT = vpt<DT, E>();
  constexpr int64_t kRound = (int64_t)kThreads * VPT * E;
  __shared__ RedScratch red;
  const int tid = threadIdx.x;
  const int64_t total = a.rows * nch;
  for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
    const int64_t row = b / nch;
    const int64_t c = b - row * nch;
    const int64_t j_lo = c * chunk;
    const int64_t j_hi = j_lo + chunk < a.cols ? j_lo + chunk : a.cols;
    const int64_t prefix = valid_prefix(a.mask, row, a.cols);
    const int64_t lim = j_hi < prefix ? j_hi : prefix;
    const char* xr = a.x + row * a.cols * S;
    char* yr = a.y + row * a.cols * S;

    // merge this row's summaries
    float m = -kInf, l = 0.0f;
    bool bad = false;
    for (int64_t i = tid; i < nch; i += kThreads) {
      const smx_stat s = stats[row * nch + i];
      if (s.m != s.m || s.l != s.l) {
        bad = true;
      } else {
        merge_ml(m, l, s.m, s.l);
      }
    }
    const bool poisoned = block_any<kWaves>(bad, red);
    block_merge<kWaves>(m, l, red);

    if (poisoned || m == -kInf) {
      Pack<DT, E> p;
      p.fill(poisoned ? Fmt<DT>::kNaN : 0u);
      for (int64_t j0 = j_lo + (int64_t)tid * E; j0 < j_hi; j0 += (int64_t)kThreads * E) p.store(yr + j0 * S);
      continue;
    }
    const float inv = 1.0f / (l * 18446744073709551616.0f);  // 2^-64 / L

    for (int64_t base = j_lo; base < j_hi; base += kRound) {
      Pack<DT, E> in[VPT];
      uint64_t kb[VPT];
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int64_t j0 = base + (int64_t)(k * kThreads + tid) * E;
        in[k].fill(0);
        kb[k] = ~0ull;
        if (j0 < lim) {
          in[k].load(xr + j0 * S);
          if constexpr (KEEP) kb[k] = load_keep<E>(a.mask.keep + row * a.cols + j0);
        }
      }
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int64_t j0 = base + (int64_t)(k * kThreads + tid) * E;
        if (j0 < j_hi) {
          uint32_t h[E];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const bool ok = (j0 + e < lim) && (!KEEP || keep_lane(kb[k], e));
            const float f = ok ? in[k].get(e) : -kInf;
            h[e] = enc<DT>(exp_b64<ACC>(f, m) * inv);
          }
          Pack<DT, E> out;
          out.put(h);
          out.store(yr + j0 * S);
        }
      }
    }
  }
}

constexpr int64_t kMaxGrid = 1 << 20;

template <int DT, int E>
hipError_t launch_stats_t(const RowArgs& a, int64_t chunk, int64_t nch, smx_stat* stats, hipStream_t s) {
  const int64_t total = a.rows * nch;
  const unsigned grid = (unsigned)(total < kMaxGrid ? total : kMaxGrid);
  if (a.mask.kind == kMaskKeep) {
    hipLaunchKernelGGL((k_stats<DT, E, true>), dim3(grid), dim3(kThreads), 0, s, a, chunk, nch, stats);
  } else {
    hipLaunchKernelGGL((k_stats<DT, E, false>), dim3(grid), dim3(kThreads), 0, s, a, chunk, nch, stats);
  }
  return hipGetLastError();
}

template <int DT, int E>
hipError_t launch_mn_t(const RowArgs& a, int64_t chunk, int64_t nch, const smx_stat* stats, hipStream_t s) {
  const int64_t total = a.rows * nch;
  const unsigned grid = (unsigned)(total < kMaxGrid ? total : kMaxGrid);
  if (a.mask.kind == kMaskKeep) {
    hipLaunchKernelGGL((k_merge_normalize<DT, E, true>), dim3(grid), dim3(kThreads), 0, s, a, chunk, nch, stats);
  } else {
    hipLaunchKernelGGL((k_merge_normalize<DT, E, false>), dim3(grid), dim3(kThreads), 0, s, a, chunk, nch, stats);
  }
  return hipGetLastError();
}

}  // namespace

int64_t split_round_cols(int dtype, bool vec) {
  if (!vec) return (int64_t)kThreads * kVptScalar;
  return dtype == kF32 ? (int64_t)kThreads * 16 * 4 : (int64_t)kThreads * 8 * 8;
}

hipError_t launch_stats(const RowArgs& a, int dtype, bool vec, int64_t chunk, int64_t nch, smx_stat* stats,
                        hipStream_t s) {
  switch (dtype) {
    case kF32:
      return vec ? launch_stats_t<kF32, 4>(a, chunk, nch, stats, s) : launch_stats_t<kF32, 1>(a, chunk, nch, stats, s);
    case kF16:
      return vec ? launch_stats_t<kF16, 8>(a, chunk, nch, stats, s) : launch_stats_t<kF16, 1>(a, chunk, nch, stats, s);
    default:
      return vec ? launch_stats_t<kBF16, 8>(a, chunk, nch, stats, s)
                 : launch_stats_t<kBF16, 1>(a, chunk, nch, stats, s);
  }
}

hipError_t launch_merge_normalize(const RowArgs& a, int dtype, bool vec, int64_t chunk, int64_t nch,
                                  const smx_stat* stats, hipStream_t s) {
  switch (dtype) {
    case kF32:
      return vec ? launch_mn_t<kF32, 4>(a, chunk, nch, stats, s) : launch_mn_t<kF32, 1>(a, chunk, nch, stats, s);
    case kF16:
      return vec ? launch_mn_t<kF16, 8>(a, chunk, nch, stats, s) : launch_mn_t<kF16, 1>(a, chunk, nch, stats, s);
    default:
      return vec ? launch_mn_t<kBF16, 8>(a, chunk, nch, stats, s) : launch_mn_t<kBF16, 1>(a, chunk, nch, stats, s);
  }
}

}  // namespace smx
