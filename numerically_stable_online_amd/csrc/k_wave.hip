// k_wave.hip — one wave64 per row, the whole row held in registers.
//
// The row is read from HBM once ("Stable softmax: keep the normalizer
// consistent as tiles arrive", paragraph on fused rows: load the row, find
// its maximum and sum, write the normalized values). Each lane keeps VPT
// packs of E elements: pack k of lane t covers elements (k*64 + t)*E ..
// +E-1, so every load and store of a wave is one contiguous 1 KiB (E*S = 16)
// or 64 contiguous elements (E = 1). Lanes keep a lane-wise running maximum
// and sum and reduce once per row ("Softmax numerics architecture", pitfall
// of reducing horizontally inside the loop).
//
// Short rows leave a wave with little to do between its load and its store,
// so a wave takes RPW rows at once: all their loads are in flight together
// and their reductions interleave.
#include "smx_device.hpp"

namespace smx {
namespace {

// MK: the mask class, fixed at compile time: kMaskNone (the whole row),
// kMaskValidLen (valid lengths), kMaskCausal (computed valid lengths) or
// kMaskKeep, so a wave's prologue is straight-line code.
//
// xcd_order: the XCDs take workgroups round-robin (workgroup i runs on XCD
// i mod 8); with xcd_order set (and the grid a multiple of 8), workgroup i
// takes the rows of logical workgroup (i mod 8) G/8 + i / 8 instead, so each
// XCD streams through a contiguous eighth of the launch's rows.
template <int DT, int E, int VPT, int RPW, int MK, int EPI>
__global__ __launch_bounds__(kThreads) void k_wave(RowArgs a, int64_t rbase, int xcd_order) {
  constexpr bool KEEP = MK == kMaskKeep;
  constexpr int S = Fmt<DT>::S;
  constexpr bool ACC = DT == kF32;
  const int lane = threadIdx.x & 63;
  const unsigned nbk = gridDim.x;
  const unsigned bid = xcd_order && (nbk & 7) == 0 ? (blockIdx.x & 7) * (nbk >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int64_t row0 = rbase + ((int64_t)bid * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * RPW;
  if (row0 >= a.rows) return;  // wave-uniform
  const int64_t cols = a.cols;

  // load, mask and lane-wise max for every row of the wave
  float v[RPW][VPT][E];
  float mx[RPW];
  const int icols = (int)cols;  // rows on this path hold at most 4096 lanes
  int prefix[RPW];
  // cross-entropy: each row's target lane (-1: ignored row), read before the
  // row so its latency overlaps the row's loads, and the target's logit as
  // this lane holds it (-inf in every other lane)
  int64_t tgt[RPW];
  int slot[RPW];
  float xo[RPW];
  valid_prefixes<MK, RPW>(a.mask, row0, a.rows, cols, prefix);
  if constexpr (EPI == kEpiXent) {
    row_targets<RPW>(a.target, row0, a.rows, cols, tgt);
  } else {
#pragma unroll
    for (int r = 0; r < RPW; ++r) tgt[r] = -1;
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    mx[r] = -kInf;
    slot[r] = target_slot<64, E>(tgt[r], lane);
    xo[r] = -kInf;
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const char* xr = a.x + (row0 + r) * cols * S;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      // the pack's valid lanes: E inside the prefix, 0 past it, so each
      // lane's test is a 32-bit compare with a constant
      const int j0 = (k * 64 + lane) * E;
      const int left = prefix[r] - j0;
      const int rem = left <= 0 ? 0 : (left >= E ? E : left);
      Pack<DT, E> p;
      p.fill(0);
      uint64_t kb = ~0ull;
      if (rem > 0) {
        p.template load<true>(xr + j0 * S);
        if constexpr (KEEP) kb = load_keep<E>(a.mask.keep + (row0 + r) * cols + j0);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool ok = e < rem && (!KEEP || keep_lane(kb, e));
        const float val = ok ? p.get(e) : -kInf;
        if constexpr (EPI == kEpiXent) {
          // the target lane: its logit kept apart, -inf in the row (so it
          // stays out of the sum of the others; its gradient is stored apart)
          const bool at = k * E + e == slot[r];
          xo[r] = at ? val : xo[r];
          v[r][k][e] = at ? -kInf : val;
        } else {
          v[r][k][e] = val;
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) mx[r] = vmax(mx[r], v[r][k][e]);
    }
    // the target's logit counts toward the maximum and the policy
    if constexpr (EPI == kEpiXent) mx[r] = vmax(mx[r], xo[r]);
  }

#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int64_t row = row0 + r;
    if (row >= a.rows) break;  // wave-uniform
    char* yr = a.y + row * cols * S;
    // the maximum propagates NaN, so one reduction gives the row's maximum
    // and its policy: NaN or +inf in a valid lane poisons the row
    const float m = wave_max(mx[r]);
    const bool poisoned = !(m < kInf);

    // cross-entropy: the row's target lane (-1: ignored row) and its logit
    int64_t t = -1;
    float xt = -kInf;
    if constexpr (EPI == kEpiXent) {
      t = tgt[r];
      if (t < 0) {  // ignored row: loss 0, gradient 0
        if (lane == 0) a.loss[row] = 0.0f;
        if (a.y != nullptr) {
          Pack<DT, E> z;
          z.fill(0u);
#pragma unroll
          for (int k = 0; k < VPT; ++k) {
            const int j0 = (k * 64 + lane) * E;
            if (j0 < icols) z.template store<true>(yr + j0 * S);
          }
        }
        continue;
      }
      // the lane holding element t: pack t / E of the row, lane (t / E) mod 64
      xt = lane_read(xo[r], (int)((t / E) & 63));
    }

    if (poisoned || m == -kInf) {
      // declared policy rows: canonical NaN, or the empty row (all +0.0; all
      // -inf for log-probabilities; -onehot(t) and an infinite loss for the
      // cross-entropy) with no -inf - -inf
      if constexpr (EPI == kEpiLogSoftmax) {
        if (lane == 0) write_lse(a.lse, row, poisoned, m, 0.0f);
      }
      if constexpr (EPI == kEpiXent) {
        if (lane == 0) a.loss[row] = poisoned ? u2f(0x7FC00000u) : kInf;
      }
      if (a.y != nullptr) {
        const uint32_t fill = poisoned ? Fmt<DT>::kNaN : (EPI == kEpiLogSoftmax ? Fmt<DT>::kNegInf : 0u);
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
          const int j0 = (k * 64 + lane) * E;
          if (j0 < icols) {
            uint32_t h[E];
#pragma unroll
            for (int e = 0; e < E; ++e) h[e] = (!poisoned && k * E + e == slot[r]) ? enc<DT>(-1.0f) : fill;
            Pack<DT, E> p;
            p.put(h);
            p.template store<true>(yr + j0 * S);
          }
        }
      }
      continue;
    }

    // exp(x - m) * 2^64 and its sum; masked lanes give exactly 0. The
    // softmax and the cross-entropy keep the exponentials for their stores.
    // The cross-entropy sums the lanes other than the target ("others") and
    // adds the target's exponential, which every lane recomputes bit for bit,
    // afterwards: one reduction gives both sums.
    float total, others = 0.0f;
    if constexpr (ACC) {
      KahanSum ks;
#pragma unroll
      for (int k = 0; k < VPT; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float te = exp_acc_b64(v[r][k][e], m);
          if constexpr (EPI != kEpiLogSoftmax) v[r][k][e] = te;
          ks.add(te);
        }
      float hi = ks.hi(), lo = ks.lo();
      wave_pair_reduce(hi, lo);
      if constexpr (EPI == kEpiXent) {
        others = hi + lo;
        pair_add(hi, lo, exp_acc_b64(xt, m), 0.0f);
      }
      total = hi + lo;
    } else {
      float s = 0.0f;
      if (EPI == kEpiSoftmax && __builtin_fabsf(m) < kBiasMaxAbs) {
        const float c = row_exp_bias(m);
#pragma unroll
        for (int k = 0; k < VPT; ++k)
#pragma unroll
          for (int e = 0; e < E; ++e) {
            v[r][k][e] = exp_hw_bias(v[r][k][e], c);
            s += v[r][k][e];
          }
      } else {
#pragma unroll
        for (int k = 0; k < VPT; ++k)
#pragma unroll
          for (int e = 0; e < E; ++e) {
            // the sum of the cross-entropy and of the log-softmax feeds an fp32
            // result (the loss, the log-sum-exp): the accurate exponential, unscaled
            // where it feeds the sum alone (log-softmax; the total is scaled after);
            // the softmax's 16-bit outputs (rows with |m| >= 2^15) need only the first
            const float te = EPI == kEpiSoftmax      ? exp_hw_b64(v[r][k][e], m)
                             : EPI == kEpiLogSoftmax ? exp_acc_sum(v[r][k][e], (double)m)
                                                     : exp_acc_b64(v[r][k][e], m);
            if constexpr (EPI != kEpiLogSoftmax) v[r][k][e] = te;
            s += te;
          }
      }
      total = wave_sum(s);
      if constexpr (EPI == kEpiLogSoftmax) total *= 18446744073709551616.0f;  // into the 2^64 scale (exact)
      if constexpr (EPI == kEpiXent) {
        others = total;
        total = others + exp_acc_b64(xt, m);
      }
    }

    if constexpr (EPI == kEpiLogSoftmax) {
      // log-softmax: y = x - (m + log l); masked and -inf lanes stay -inf
      const float lsum = total * 5.42101086242752217e-20f;  // remove 2^64 (exact)
      const Lse lse = make_lse(m, lsum);
      if (lane == 0) write_lse(a.lse, row, false, m, lsum);
      if (a.y != nullptr) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
          const int j0 = (k * 64 + lane) * E;
          if (j0 < icols) {
            float o[E];
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = minus_lse(v[r][k][e], lse);
            Pack<DT, E> p;
            p.put_values(o);
            p.template store<true>(yr + j0 * S);
          }
        }
      }
    } else {
      const float inv = 1.0f / total;  // 2^-64 / l
      // the target lane of the cross-entropy gradient: p_t - 1 = -(others / l)
      // (a correctly rounded divide: exactly -1 when the target lane is masked)
      const float at_t = (0.0f - others) / total;
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int j0 = (k * 64 + lane) * E;
        if (a.y != nullptr && j0 < icols) {
          float o[E];
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = v[r][k][e] * inv;  // 0 at the cross-entropy's target
          Pack<DT, E> p;
          p.put_values(o);
          p.template store<true>(yr + j0 * S);
        }
      }
      // the cross-entropy's gradient at the target, over the 0 its pack wrote
      // (the same lane, so the two stores land in order)
      if constexpr (EPI == kEpiXent) {
        if (slot[r] >= 0 && a.y != nullptr) store_one<DT>(yr + t * S, at_t);
      }
      // the loss last, once the row's values are no longer live
      if constexpr (EPI == kEpiXent) {
        if (lane == 0) {
          a.loss[row] = xent_loss(m, xt, others * 5.42101086242752217e-20f, total * 5.42101086242752217e-20f);
        }
      }
    }
  }
}

// Inputs of at least 1.5 GiB take the XCD-contiguous row order. Measured
// against the round-robin order in one process (outputs bitwise equal):
// causal bf16 rows of 2048 lanes, 1.5 / 2 / 4 GiB: -7.7 / -7.4 / -11.5 %;
// 2 GiB of unmasked bf16 or fp32 rows -0.2 to -1.4 %, of bf16 rows with
// valid lengths -3.2 %; at 1 GiB and below the effect is mixed and mostly a
// loss (256 MiB of causal f16 rows +5.5 %, 1 GiB of fp32 rows +2.5 to 9.8 %).
constexpr int64_t kXcdOrderMinBytes = (int64_t)3 << 29;

template <int DT, int E, int VPT, int RPW, int EPI>
hipError_t launch_vpt(const RowArgs& a, hipStream_t stream) {
  // slices of at most 2^20 workgroups, so a launch's work-items stay below 2^32
  constexpr int64_t kMaxBlocks = (int64_t)1 << 20;
  const int64_t rows_per_block = (int64_t)kWaves * RPW;
  const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  const int xcd = a.rows * a.cols * Fmt<DT>::S >= kXcdOrderMinBytes;
  for (int64_t b0 = 0; b0 < blocks; b0 += kMaxBlocks) {
    const dim3 grid((unsigned)(blocks - b0 < kMaxBlocks ? blocks - b0 : kMaxBlocks));
    const int64_t rbase = b0 * rows_per_block;
    if (a.mask.kind == kMaskKeep) {
      hipLaunchKernelGGL((k_wave<DT, E, VPT, RPW, kMaskKeep, EPI>), grid, dim3(kThreads), 0, stream, a, rbase, xcd);
    } else if (a.mask.kind == kMaskNone) {
      hipLaunchKernelGGL((k_wave<DT, E, VPT, RPW, kMaskNone, EPI>), grid, dim3(kThreads), 0, stream, a, rbase, xcd);
    } else if (a.mask.kind == kMaskValidLen) {
      hipLaunchKernelGGL((k_wave<DT, E, VPT, RPW, kMaskValidLen, EPI>), grid, dim3(kThreads), 0, stream, a, rbase, xcd);
    } else {
      hipLaunchKernelGGL((k_wave<DT, E, VPT, RPW, kMaskCausal, EPI>), grid, dim3(kThreads), 0, stream, a, rbase, xcd);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// the smallest register budget that holds the row; short rows go several to
// a wave
template <int DT, int E, int EPI>
hipError_t launch_e(const RowArgs& a, hipStream_t stream) {
  const int64_t per_vpt = 64 * E;
  const int64_t need = (a.cols + per_vpt - 1) / per_vpt;
  if constexpr (E == 1) {
    if (need <= 2) return launch_vpt<DT, E, 2, 4, EPI>(a, stream);
    if (need <= 8) return launch_vpt<DT, E, 8, 2, EPI>(a, stream);
    return launch_vpt<DT, E, 32, 1, EPI>(a, stream);
  } else {
    if (need <= 1) return launch_vpt<DT, E, 1, 4, EPI>(a, stream);
    if (need <= 2) return launch_vpt<DT, E, 2, 2, EPI>(a, stream);
    if (need <= 4) return launch_vpt<DT, E, 4, 1, EPI>(a, stream);
    return launch_vpt<DT, E, 8, 1, EPI>(a, stream);
  }
}

template <int EPI>
hipError_t launch_epi(const RowArgs& a, int dtype, bool vec, hipStream_t stream) {
  switch (dtype) {
    case kF32:
      return vec ? launch_e<kF32, 4, EPI>(a, stream) : launch_e<kF32, 1, EPI>(a, stream);
    case kF16:
      return vec ? launch_e<kF16, 8, EPI>(a, stream) : launch_e<kF16, 1, EPI>(a, stream);
    default:
      return vec ? launch_e<kBF16, 8, EPI>(a, stream) : launch_e<kBF16, 1, EPI>(a, stream);
  }
}

}  // namespace

int64_t wave_max_cols(int dtype, bool vec) { return vec ? 64 * 8 * vec_elems(dtype) : 64 * 32; }

hipError_t launch_wave(const RowArgs& a, int dtype, bool vec, int epi, hipStream_t stream) {
  if (epi == kEpiSoftmax) return launch_epi<kEpiSoftmax>(a, dtype, vec, stream);
  if (epi == kEpiLogSoftmax) return launch_epi<kEpiLogSoftmax>(a, dtype, vec, stream);
  return launch_epi<kEpiXent>(a, dtype, vec, stream);
}

}  // namespace smx
