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
// poisons the row), then rereads its chunk and writes exp(x - M) / L. For a
// row that cannot stay on chip this second read of x is inherent to the
// online method: no output can be written before the row's sum is final
// ("Kernel visualization: online softmax", sections "Tiled version" and
// "Online softmax: two passes").
#include "smx_device.hpp"

namespace smx {
namespace {

constexpr int kVptScalar = 16;  // packs per thread per round for single-element packs

template <int DT, int E>
constexpr int vpt() {
  return E == 1 ? kVptScalar : 8;
}

// the stats pass keeps two rounds in registers (the one being reduced and
// the one in flight)
template <int DT, int E>
constexpr int vpt_stats() {
  return E == 1 ? 8 : 4;
}

template <int DT, int E, int VPT, bool KEEP, bool XENT>
__global__ __launch_bounds__(kThreads) void k_stats(RowArgs a, int64_t chunk, int64_t nch, smx_stat* stats) {
  constexpr int S = Fmt<DT>::S;
  constexpr bool ACC = DT == kF32;
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
    const uint8_t* kr = KEEP ? a.mask.keep + row * a.cols : nullptr;
    // cross-entropy: the target lane stays out of the summary and the chunk
    // holding it records its logit; a NaN or +inf there still poisons the
    // chunk
    const int64_t t = XENT ? row_target(a.target, row, a.cols) : -1;
    bool tbad = false;
    if (XENT && t >= j_lo && t < j_hi && tid == 0) {
      float xt = -kInf;
      if (t < prefix && (!KEEP || kr[t] != 0)) {
        Pack<DT, 1> q;
        q.load(xr + t * S);
        xt = q.get(0);
      }
      a.xt[row] = xt;
      tbad = !(xt < kInf);
    }

    // one round's loads into registers. These are ordinary loads, not
    // nontemporal ones: part of x then stays in the Infinity Cache for the
    // normalize pass's reread (nontemporal loads here made the two passes
    // 12-14 % slower end to end)
    // a round wholly inside the valid prefix needs no per-element test
    // (keep masks and the cross-entropy's target lane always do); the test
    // is uniform across the workgroup, so the two forms are scalar branches
    auto full_round = [&](int64_t base) { return !KEEP && !XENT && base + kRound <= lim; };
    auto fetch = [&](int64_t base, Pack<DT, E>(&p)[VPT], uint64_t(&kb)[VPT]) {
      if (full_round(base)) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
          p[k].load(xr + (base + (int64_t)(k * kThreads + tid) * E) * S);
          kb[k] = ~0ull;
        }
        return;
      }
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int64_t j0 = base + (int64_t)(k * kThreads + tid) * E;
        p[k].fill(0);
        kb[k] = ~0ull;
        if (j0 < lim) {
          p[k].load(xr + j0 * S);
          if constexpr (KEEP) kb[k] = load_keep<E>(kr + j0);
        }
      }
    };

    // fold one round into the thread's running (m, l): the tiled recurrence.
    // The maximum propagates NaN, so a thread's m ends NaN or +inf exactly
    // when one of its valid lanes holds NaN or +inf.
    float m_t = -kInf, l_t = 0.0f;
    auto fold = [&](int64_t base, const Pack<DT, E>(&p)[VPT], const uint64_t(&kb)[VPT]) {
      const int slot = XENT ? target_slot<kThreads, E>(t >= base && t - base < kRound ? t - base : -1, tid) : -1;
      float v[VPT * E];
      float mr = -kInf;
      if (full_round(base)) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
#pragma unroll
          for (int e = 0; e < E; ++e) v[k * E + e] = p[k].get(e);
        }
        mr = tree_max<VPT * E>(v);
      } else {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
          const int64_t left = lim - (base + (int64_t)(k * kThreads + tid) * E);
          const int rem = left <= 0 ? 0 : (left >= E ? E : (int)left);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const bool ok = e < rem && (!KEEP || keep_lane(kb[k], e)) && (!XENT || k * E + e != slot);
            v[k * E + e] = ok ? p[k].get(e) : -kInf;
          }
#pragma unroll
          for (int e = 0; e < E; ++e) mr = vmax(mr, v[k * E + e]);
        }
      }
      const float m_new = vmax(m_t, mr);
      if (m_new != -kInf) {
        // correct the running sum, then add this round against m_new; the
        // round's terms are summed as a tree in registers
        const double m64 = (double)m_new;
#pragma unroll
        for (int i = 0; i < VPT * E; ++i) {
          if constexpr (ACC) {
            v[i] = exp_acc_sum(v[i], m64);  // a NaN lane adds 0 here; m_new carries it into the poison flag
          } else {
            // the cross-entropy's sum feeds its fp32 loss: the accurate exponential
            v[i] = XENT ? exp_acc_sum(v[i], m64) : __builtin_amdgcn_exp2f((v[i] - m_new) * kLog2e);
          }
        }
        l_t = l_t * exp_diff(m_t, m_new) + tree_sum<VPT * E>(v);
        m_t = m_new;
      }
    };

    // two register rounds, alternating: while one is folded the other's
    // loads are in flight, and nothing is copied between them
    Pack<DT, E> ra[VPT], rb[VPT];
    uint64_t ka[VPT], kb[VPT];
    if (j_lo < lim) fetch(j_lo, ra, ka);
    for (int64_t base = j_lo; base < lim; base += 2 * kRound) {
      const bool more_b = base + kRound < lim;
      if (more_b) fetch(base + kRound, rb, kb);
      fold(base, ra, ka);
      if (!more_b) break;
      if (base + 2 * kRound < lim) fetch(base + 2 * kRound, ra, ka);
      fold(base + kRound, rb, kb);
    }
    // thread summaries -> chunk summary; NaN/inf poisons the chunk
    float m = m_t, l = l_t;
    const bool poisoned = block_merge_flagged<kWaves>(m, l, tbad || !(m_t < kInf), red);
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
        s.l = l;
      }
      stats[b] = s;
    }
  }
}

template <int DT, int E, bool KEEP, int EPI>
__global__ __launch_bounds__(kThreads) void k_merge_normalize(RowArgs a, int64_t chunk, int64_t nch,
                                                              const smx_stat* stats, int64_t nsum) {
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
    // with no y, only the per-row scalars (log-sum-exp, loss) are wanted:
    // one workgroup per row
    if (a.y == nullptr && c != 0) continue;
    const int64_t j_lo = c * chunk;
    const int64_t j_hi = j_lo + chunk < a.cols ? j_lo + chunk : a.cols;
    const int64_t prefix = valid_prefix(a.mask, row, a.cols);
    const int64_t lim = j_hi < prefix ? j_hi : prefix;
    const char* xr = a.x + row * a.cols * S;
    char* yr = a.y + row * a.cols * S;

    // cross-entropy: the row's target lane (-1: ignored row) and the target's
    // logit as the stats pass left it, loaded together with the summaries
    // (the ignored-row branch waits for the merge, so no load waits on
    // another)
    const int64_t t = EPI == kEpiXent ? row_target(a.target, row, a.cols) : -1;
    const float xt_in = EPI == kEpiXent ? a.xt[row] : -kInf;

    // merge this row's nsum summaries (every chunk's, or the one k_row_merge
    // left)
    float m = -kInf, l = 0.0f;
    bool bad = false;
    for (int64_t i = tid; i < nsum; i += kThreads) {
      const smx_stat s = stats[row * nsum + i];
      if (s.m != s.m || s.l != s.l) {
        bad = true;
      } else {
        merge_ml(m, l, s.m, s.l);
      }
    }
    const bool poisoned = block_merge_flagged<kWaves>(m, l, bad, red);

    // cross-entropy: an ignored row has loss 0 and gradient 0
    if (EPI == kEpiXent && t < 0) {
      if (c == 0 && tid == 0) a.loss[row] = 0.0f;
      if (a.y != nullptr) {
        Pack<DT, E> z;
        z.fill(0u);
        for (int64_t j0 = j_lo + (int64_t)tid * E; j0 < j_hi; j0 += (int64_t)kThreads * E)
          z.template store<true>(yr + j0 * S);
      }
      continue;
    }
    // cross-entropy: the summaries leave out the target lane; fold it back
    // in, in the 2^64 scale (o64, l64), so that the others keep their
    // relative precision when they lie far below the target (the loss of a
    // confident row is made of them); others and l are the same unscaled,
    // each rounded once
    float others = 0.0f, xt = -kInf, o64 = 0.0f, l64 = 1.0f;
    if constexpr (EPI == kEpiXent) {
      if (!poisoned) {
        xt = xt_in;
        const float mm = fmaxf(m, xt);
        o64 = l * exp_diff_b64(m, mm);
        l64 = o64 + exp_diff_b64(xt, mm);
        others = o64 * 5.42101086242752217e-20f;  // * 2^-64
        l = l64 * 5.42101086242752217e-20f;       // >= 1: exact
        m = mm;
      }
      if (c == 0 && tid == 0) {
        a.loss[row] = poisoned ? u2f(0x7FC00000u) : (m == -kInf ? kInf : xent_loss(m, xt, others, l));
      }
      if (a.y == nullptr) continue;
    }
    if constexpr (EPI == kEpiLogSoftmax) {
      if (c == 0 && tid == 0) write_lse(a.lse, row, poisoned, poisoned ? kInf : m, l);
      if (a.y == nullptr) continue;
    }

    if (poisoned || m == -kInf) {
      const uint32_t fill = poisoned ? Fmt<DT>::kNaN : (EPI == kEpiLogSoftmax ? Fmt<DT>::kNegInf : 0u);
      for (int64_t j0 = j_lo + (int64_t)tid * E; j0 < j_hi; j0 += (int64_t)kThreads * E) {
        uint32_t h[E];
#pragma unroll
        for (int e = 0; e < E; ++e) h[e] = (!poisoned && j0 + e == t) ? enc<DT>(-1.0f) : fill;
        Pack<DT, E> p;
        p.put(h);
        p.template store<true>(yr + j0 * S);
      }
      continue;
    }
    // softmax / cross-entropy: the reciprocal 2^-64 / L; log-softmax: M + log L as hi + lo
    const float inv = EPI != kEpiLogSoftmax ? 1.0f / (l * 18446744073709551616.0f) : 0.0f;
    const Lse lse = EPI != kEpiLogSoftmax ? Lse{0.0f, 0.0f} : make_lse(m, l);
    const float at_t = (0.0f - o64) / l64;  // cross-entropy target lane: -(others / L)

    for (int64_t base = j_lo; base < j_hi; base += kRound) {
      // cross-entropy: the target's place in this round's registers (-1: not
      // here). A round may reach past the chunk (chunk < kRound), so the target
      // must also lie inside this chunk: its lane belongs to one workgroup only
      const int slot = EPI == kEpiXent
                           ? target_slot<kThreads, E>(t >= base && t < j_hi && t - base < kRound ? t - base : -1, tid)
                           : -1;
      Pack<DT, E> in[VPT];
      uint64_t kb[VPT];
      // a round wholly inside the valid prefix: every pack is loaded and
      // stored, no lane is masked (uniform across the workgroup)
      if (!KEEP && base + kRound <= lim) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) in[k].template load<true>(xr + (base + (int64_t)(k * kThreads + tid) * E) * S);
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
          const int64_t j0 = base + (int64_t)(k * kThreads + tid) * E;
          float o[E];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            if constexpr (EPI == kEpiLogSoftmax) {
              o[e] = minus_lse(in[k].get(e), lse);
            } else {
              o[e] = exp_b64<ACC>(in[k].get(e), m) * inv;
            }
          }
          Pack<DT, E> out;
          out.put_values(o);
          out.template store<true>(yr + j0 * S);
        }
        if constexpr (EPI == kEpiXent) {
          if (slot >= 0) store_one<DT>(yr + t * S, at_t);
        }
        continue;
      }
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int64_t j0 = base + (int64_t)(k * kThreads + tid) * E;
        in[k].fill(0);
        kb[k] = ~0ull;
        if (j0 < lim) {
          in[k].template load<true>(xr + j0 * S);
          if constexpr (KEEP) kb[k] = load_keep<E>(a.mask.keep + row * a.cols + j0);
        }
      }
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int64_t j0 = base + (int64_t)(k * kThreads + tid) * E;
        if (j0 < j_hi) {
          // the pack's valid lanes: E inside the prefix, 0 past it
          const int64_t left = lim - j0;
          const int rem = left <= 0 ? 0 : (left >= E ? E : (int)left);
          float o[E];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const bool ok = e < rem && (!KEEP || keep_lane(kb[k], e));
            const float f = ok ? in[k].get(e) : -kInf;
            if constexpr (EPI == kEpiLogSoftmax) {
              o[e] = minus_lse(f, lse);
            } else {
              o[e] = exp_b64<ACC>(f, m) * inv;
            }
          }
          Pack<DT, E> out;
          out.put_values(o);
          out.template store<true>(yr + j0 * S);
        }
      }
      // the cross-entropy's gradient at the target, over the value its pack
      // wrote (the same thread, so the two stores land in order)
      if constexpr (EPI == kEpiXent) {
        if (slot >= 0) store_one<DT>(yr + t * S, at_t);
      }
    }
  }
}

// Rows with many chunks merge their summaries once, here, instead of once in
// every chunk's workgroup of the normalize pass (whose merge reads would grow
// as chunks squared). Each thread folds the same summaries in the same order
// and the same tree combines the threads as in k_merge_normalize, so (M, L) is
// bitwise the one the normalize pass would form; folded again there, (M, L)
// merged into the empty (-inf, 0) comes out unchanged. The loads of a thread
// are issued eight at a time, ahead of the dependent folds.
__global__ __launch_bounds__(kThreads) void k_row_merge(const smx_stat* stats, int64_t rows, int64_t nch,
                                                        smx_stat* merged) {
  constexpr int kBatch = 8;
  __shared__ RedScratch red;
  const int tid = threadIdx.x;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const smx_stat* rs = stats + row * nch;
    float m = -kInf, l = 0.0f;
    bool bad = false;
    for (int64_t i0 = tid; i0 < nch; i0 += (int64_t)kBatch * kThreads) {
      smx_stat q[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int64_t i = i0 + (int64_t)k * kThreads;
        q[k] = i < nch ? rs[i] : smx_stat{-kInf, 0.0f};
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        if (i0 + (int64_t)k * kThreads >= nch) break;
        if (q[k].m != q[k].m || q[k].l != q[k].l) {
          bad = true;
        } else {
          merge_ml(m, l, q[k].m, q[k].l);
        }
      }
    }
    const bool poisoned = block_merge_flagged<kWaves>(m, l, bad, red);
    if (tid == 0) {
      const float nan = __builtin_nanf("");
      merged[row] = poisoned ? smx_stat{nan, nan} : smx_stat{m, l};
    }
  }
}

constexpr int64_t kMaxGrid = 1 << 20;

template <int DT, int E>
hipError_t launch_stats_t(const RowArgs& a, bool xent, int64_t chunk, int64_t nch, smx_stat* stats, hipStream_t s) {
  constexpr int VPT = vpt_stats<DT, E>();
  const int64_t total = a.rows * nch;
  const unsigned grid = (unsigned)(total < kMaxGrid ? total : kMaxGrid);
  if (a.mask.kind == kMaskKeep) {
    if (xent) {
      hipLaunchKernelGGL((k_stats<DT, E, VPT, true, true>), dim3(grid), dim3(kThreads), 0, s, a, chunk, nch, stats);
    } else {
      hipLaunchKernelGGL((k_stats<DT, E, VPT, true, false>), dim3(grid), dim3(kThreads), 0, s, a, chunk, nch, stats);
    }
  } else {
    if (xent) {
      hipLaunchKernelGGL((k_stats<DT, E, VPT, false, true>), dim3(grid), dim3(kThreads), 0, s, a, chunk, nch, stats);
    } else {
      hipLaunchKernelGGL((k_stats<DT, E, VPT, false, false>), dim3(grid), dim3(kThreads), 0, s, a, chunk, nch, stats);
    }
  }
  return hipGetLastError();
}

template <int DT, int E, int EPI>
hipError_t launch_mn_t(const RowArgs& a, int64_t chunk, int64_t nch, const smx_stat* stats, int64_t nsum,
                       hipStream_t s) {
  const int64_t total = a.rows * nch;
  const unsigned grid = (unsigned)(total < kMaxGrid ? total : kMaxGrid);
  if (a.mask.kind == kMaskKeep) {
    hipLaunchKernelGGL((k_merge_normalize<DT, E, true, EPI>), dim3(grid), dim3(kThreads), 0, s, a, chunk, nch, stats,
                       nsum);
  } else {
    hipLaunchKernelGGL((k_merge_normalize<DT, E, false, EPI>), dim3(grid), dim3(kThreads), 0, s, a, chunk, nch, stats,
                       nsum);
  }
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_mn_epi(const RowArgs& a, int dtype, bool vec, int64_t chunk, int64_t nch, const smx_stat* stats,
                         int64_t nsum, hipStream_t s) {
  switch (dtype) {
    case kF32:
      return vec ? launch_mn_t<kF32, 4, EPI>(a, chunk, nch, stats, nsum, s)
                 : launch_mn_t<kF32, 1, EPI>(a, chunk, nch, stats, nsum, s);
    case kF16:
      return vec ? launch_mn_t<kF16, 8, EPI>(a, chunk, nch, stats, nsum, s)
                 : launch_mn_t<kF16, 1, EPI>(a, chunk, nch, stats, nsum, s);
    default:
      return vec ? launch_mn_t<kBF16, 8, EPI>(a, chunk, nch, stats, nsum, s)
                 : launch_mn_t<kBF16, 1, EPI>(a, chunk, nch, stats, nsum, s);
  }
}

}  // namespace

int64_t split_round_cols(int dtype, bool vec) {
  if (!vec) return (int64_t)kThreads * kVptScalar;
  return (int64_t)kThreads * 8 * vec_elems(dtype);
}

hipError_t launch_stats(const RowArgs& a, int dtype, bool vec, bool xent, int64_t chunk, int64_t nch, smx_stat* stats,
                        hipStream_t s) {
  switch (dtype) {
    case kF32:
      return vec ? launch_stats_t<kF32, 4>(a, xent, chunk, nch, stats, s)
                 : launch_stats_t<kF32, 1>(a, xent, chunk, nch, stats, s);
    case kF16:
      return vec ? launch_stats_t<kF16, 8>(a, xent, chunk, nch, stats, s)
                 : launch_stats_t<kF16, 1>(a, xent, chunk, nch, stats, s);
    default:
      return vec ? launch_stats_t<kBF16, 8>(a, xent, chunk, nch, stats, s)
                 : launch_stats_t<kBF16, 1>(a, xent, chunk, nch, stats, s);
  }
}

hipError_t launch_merge_normalize(const RowArgs& a, int dtype, bool vec, int epi, int64_t chunk, int64_t nch,
                                  const smx_stat* stats, int64_t nsum, hipStream_t s) {
  if (epi == kEpiSoftmax) return launch_mn_epi<kEpiSoftmax>(a, dtype, vec, chunk, nch, stats, nsum, s);
  if (epi == kEpiLogSoftmax) return launch_mn_epi<kEpiLogSoftmax>(a, dtype, vec, chunk, nch, stats, nsum, s);
  return launch_mn_epi<kEpiXent>(a, dtype, vec, chunk, nch, stats, nsum, s);
}

hipError_t launch_row_merge(const smx_stat* stats, int64_t rows, int64_t nch, smx_stat* merged, hipStream_t s) {
  const unsigned grid = (unsigned)(rows < kMaxGrid ? rows : kMaxGrid);
  hipLaunchKernelGGL(k_row_merge, dim3(grid), dim3(kThreads), 0, s, stats, rows, nch, merged);
  return hipGetLastError();
}

}  // namespace smx
