// k_lds.hip — one workgroup per row, the row staged in LDS.
//
// The row's valid prefix is copied from HBM straight into LDS with gfx950's
// direct global->LDS 128-bit loads (global_load_lds_dwordx4): the copy needs
// no VGPRs, so a workgroup can have the whole row in flight at once. Input
// and output stream through the caches with the nontemporal bit set. The row
// is read from HBM exactly once ("Stable softmax: keep the normalizer
// consistent as tiles arrive", paragraph on fused rows); every thread then
// takes its packs out of LDS into registers, and the max, the sum of
// shifted exponentials and the normalized stores follow as in the wave
// kernel, with workgroup-wide reductions.
#include "smx_device.hpp"

namespace smx {
namespace {

constexpr int kPiece = 64 * 16;  // bytes one wave's direct load moves
constexpr int kAuxNT = 2;        // cache-policy operand: the nontemporal bit

// MK: the mask class, fixed at compile time so that a row's first loads go
// out after a handful of scalar instructions: kMaskNone (the whole row),
// kMaskValidLen (a valid prefix: valid lengths or causal) or kMaskKeep.
// One workgroup per row: row0 + blockIdx.x (the host launches slices of at
// most kMaxGrid rows), so the row's loads are the first thing a wave issues.
template <int DT, int NT, int VPT, int MK, int EPI>
__global__ __launch_bounds__(NT) void k_lds(RowArgs a, int64_t row0) {
  constexpr bool KEEP = MK == kMaskKeep;
  constexpr int S = Fmt<DT>::S;
  constexpr int E = 16 / S;
  constexpr bool ACC = DT == kF32;
  constexpr int NW = NT / 64;
  extern __shared__ __attribute__((aligned(1024))) char row_lds[];
  __shared__ RedScratch red;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t cols = a.cols;

  const int64_t row = row0 + blockIdx.x;
  const int64_t prefix = MK == kMaskValidLen ? valid_prefix(a.mask, row, cols) : cols;
  const char* xr = a.x + row * cols * S;
  char* yr = a.y + row * cols * S;
  // cross-entropy: the row's target lane (-1: ignored row), read before the
  // row is staged so its latency overlaps the copy
  const int64_t t = EPI == kEpiXent ? row_target(a.target, row, cols) : -1;
  const int slot = target_slot<NT, E>(t, tid);

  // stage the valid prefix: wave w copies pieces w, w + NW, ..., at most
  // VPT of them (the row has at most VPT * NT packs, 64 to a piece)
  const int ipre = (int)prefix;  // rows on this path hold at most 2^14 lanes
  const int icols = (int)cols;
  const int nvec = (ipre + E - 1) / E;
  const int npieces = (nvec + 63) >> 6;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int pc = k * NW + wid;
    if (pc < npieces) {
      const int vi = pc * 64 + lane;
      const int vsrc = vi < nvec ? vi : nvec - 1;  // stays inside the row
      __builtin_amdgcn_global_load_lds(
          (const void*)(xr + (int64_t)vsrc * 16),
          (__attribute__((address_space(3))) void*)(row_lds + pc * kPiece), 16, 0, kAuxNT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // packs out of LDS; masked lanes become -inf. A pack holds `rem` valid
  // lanes (E inside the prefix, 0 past it), so each lane's test is a 32-bit
  // compare with a constant. The cross-entropy's target lane becomes -inf
  // too: it stays out of the sum of the others (its logit xt, read below,
  // joins the maximum and the total), and its gradient is stored apart.
  float v[VPT][E];
  float mx = -kInf;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int vi = k * NT + tid;
    const int left = ipre - vi * E;
    const int rem = left <= 0 ? 0 : (left >= E ? E : left);
    Pack<DT, E> p;
    p.fill(0);
    uint64_t kb = ~0ull;
    if (rem > 0) {
      const uint4 w = *reinterpret_cast<const uint4*>(row_lds + vi * 16);
      p.w[0] = w.x;
      p.w[1] = w.y;
      p.w[2] = w.z;
      p.w[3] = w.w;
      if constexpr (KEEP) kb = load_keep<E>(a.mask.keep + row * cols + vi * E);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ok = e < rem && (!KEEP || keep_lane(kb, e)) && (EPI != kEpiXent || k * E + e != slot);
      v[k][e] = ok ? p.get(e) : -kInf;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) mx = vmax(mx, v[k][e]);
  }
  // cross-entropy: the target's logit, taken from the staged row (after
  // the barrier above: any wave's piece may hold it).
  float xt = -kInf;
  if constexpr (EPI == kEpiXent) {
    if (t >= 0 && t < prefix && (!KEEP || a.mask.keep[row * cols + t] != 0)) {
      if constexpr (S == 4) {
        xt = dec<DT>(*reinterpret_cast<const uint32_t*>(row_lds + t * S));
      } else {
        xt = dec<DT>(*reinterpret_cast<const uint16_t*>(row_lds + t * S));
      }
    }
    mx = vmax(mx, xt);  // the target's logit counts toward the maximum and the policy
  }
  // the maximum propagates NaN, so one reduction gives the row's maximum
  // and its policy: NaN or +inf in a valid lane poisons the row
  mx = block_max<NW>(mx, red);
  const bool poisoned = !(mx < kInf);

  if constexpr (EPI == kEpiXent) {
    if (t < 0) {  // ignored row: loss 0, gradient 0
      if (tid == 0) a.loss[row] = 0.0f;
      if (a.y != nullptr) {
        Pack<DT, E> z;
        z.fill(0u);
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
          const int j0 = (k * NT + tid) * E;
          if (j0 < icols) z.template store<true>(yr + j0 * S);
        }
      }
      return;
    }
  }

  if (poisoned || mx == -kInf) {
    if constexpr (EPI == kEpiLogSoftmax) {
      if (tid == 0) write_lse(a.lse, row, poisoned, mx, 0.0f);
    }
    if constexpr (EPI == kEpiXent) {
      if (tid == 0) a.loss[row] = poisoned ? u2f(0x7FC00000u) : kInf;
    }
    if (a.y != nullptr) {
      const uint32_t fill = poisoned ? Fmt<DT>::kNaN : (EPI == kEpiLogSoftmax ? Fmt<DT>::kNegInf : 0u);
#pragma unroll
      for (int k = 0; k < VPT; ++k) {
        const int j0 = (k * NT + tid) * E;
        if (j0 < icols) {
          uint32_t h[E];
#pragma unroll
          for (int e = 0; e < E; ++e) h[e] = (!poisoned && k * E + e == slot) ? enc<DT>(-1.0f) : fill;
          Pack<DT, E> p;
          p.put(h);
          p.template store<true>(yr + j0 * S);
        }
      }
    }
    return;
  }

  // exp(x - m) * 2^64 and the sums. The cross-entropy sums the lanes other
  // than the target and adds the target's exponential (recomputed bit for
  // bit by every thread) after the one reduction.
  float total, others = 0.0f;
  if constexpr (ACC) {
    KahanSum ks;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float te = exp_acc_b64(v[k][e], mx);
        if constexpr (EPI != kEpiLogSoftmax) v[k][e] = te;
        ks.add(te);
      }
    float hi = ks.hi(), lo = ks.lo();
    block_pair_reduce<NW>(hi, lo, red);
    if constexpr (EPI == kEpiXent) {
      others = hi + lo;
      pair_add(hi, lo, exp_acc_b64(xt, mx), 0.0f);
    }
    total = hi + lo;
  } else {
    float s = 0.0f;
    if (EPI == kEpiSoftmax && __builtin_fabsf(mx) < kBiasMaxAbs) {
      const float c = row_exp_bias(mx);
#pragma unroll
      for (int k = 0; k < VPT; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          v[k][e] = exp_hw_bias(v[k][e], c);
          s += v[k][e];
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
          const float te = EPI == kEpiSoftmax      ? exp_hw_b64(v[k][e], mx)
                           : EPI == kEpiLogSoftmax ? exp_acc_sum(v[k][e], (double)mx)
                                                   : exp_acc_b64(v[k][e], mx);
          if constexpr (EPI != kEpiLogSoftmax) v[k][e] = te;
          s += te;
        }
    }
    total = block_sum<NW>(s, red);
    if constexpr (EPI == kEpiLogSoftmax) total *= 18446744073709551616.0f;  // into the 2^64 scale (exact)
    if constexpr (EPI == kEpiXent) {
      others = total;
      total = others + exp_acc_b64(xt, mx);
    }
  }

  float inv = 0.0f;  // softmax / cross-entropy: the reciprocal 2^-64 / l
  Lse lse{0.0f, 0.0f};  // log-softmax: m + log l as hi + lo
  if constexpr (EPI == kEpiLogSoftmax) {
    const float lsum = total * 5.42101086242752217e-20f;  // remove 2^64 (exact)
    lse = make_lse(mx, lsum);
    if (tid == 0) write_lse(a.lse, row, false, mx, lsum);
    if (a.y == nullptr) return;
  } else {
    inv = 1.0f / total;
  }
  // cross-entropy target lane: -(others / l), correctly rounded (exactly -1
  // when the target lane is masked)
  const float at_t = (0.0f - others) / total;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int j0 = (k * NT + tid) * E;
    if (a.y != nullptr && j0 < icols) {
      float o[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if constexpr (EPI == kEpiLogSoftmax) {
          o[e] = minus_lse(v[k][e], lse);
        } else {
          o[e] = v[k][e] * inv;  // 0 at the cross-entropy's target, stored apart below
        }
      }
      Pack<DT, E> p;
      p.put_values(o);
      p.template store<true>(yr + j0 * S);
    }
  }
  // the cross-entropy's gradient at the target, over the 0 its pack wrote
  // (the same thread, so the two stores land in order)
  if constexpr (EPI == kEpiXent) {
    if (slot >= 0 && a.y != nullptr) store_one<DT>(yr + t * S, at_t);
  }
  // the loss last, once the row's values are no longer live
  if constexpr (EPI == kEpiXent) {
    if (tid == 0) {
      a.loss[row] = xent_loss(mx, xt, others * 5.42101086242752217e-20f, total * 5.42101086242752217e-20f);
    }
  }
}

// rows up to 8 packs per thread of a 256-thread workgroup: 32 KiB of LDS,
// 32 (f32) or 64 (16-bit) register-resident values per thread (longer rows
// take k_lds_res, which keeps them in LDS)
constexpr int64_t kMaxRowBytes = 256 * 8 * 16;

// rows per launch: the grid's work-items stay far below 2^32
constexpr int64_t kMaxGrid = (int64_t)1 << 20;

template <int DT, int NT, int VPT, int EPI>
hipError_t launch_vpt(const RowArgs& a, hipStream_t s) {
  constexpr int S = Fmt<DT>::S;
  const int64_t bytes = ((a.cols * S + kPiece - 1) / kPiece) * kPiece;
  for (int64_t row0 = 0; row0 < a.rows; row0 += kMaxGrid) {
    const unsigned grid = (unsigned)(a.rows - row0 < kMaxGrid ? a.rows - row0 : kMaxGrid);
    if (a.mask.kind == kMaskKeep) {
      hipLaunchKernelGGL((k_lds<DT, NT, VPT, kMaskKeep, EPI>), dim3(grid), dim3(NT), (size_t)bytes, s, a, row0);
    } else if (a.mask.kind == kMaskNone) {
      hipLaunchKernelGGL((k_lds<DT, NT, VPT, kMaskNone, EPI>), dim3(grid), dim3(NT), (size_t)bytes, s, a, row0);
    } else {
      hipLaunchKernelGGL((k_lds<DT, NT, VPT, kMaskValidLen, EPI>), dim3(grid), dim3(NT), (size_t)bytes, s, a,
                         row0);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Four-wave workgroups hold the row in 2, 4 or 8 packs per thread (two-wave
// and eight-wave shapes measured slower on the 8192 x 4096 bf16 workload).
template <int DT, int EPI>
hipError_t launch_dt(const RowArgs& a, hipStream_t s) {
  constexpr int E = 16 / Fmt<DT>::S;
  const int64_t packs = (a.cols + E - 1) / E;
  if (packs <= 256 * 2) return launch_vpt<DT, 256, 2, EPI>(a, s);
  if (packs <= 256 * 4) return launch_vpt<DT, 256, 4, EPI>(a, s);
  return launch_vpt<DT, 256, 8, EPI>(a, s);
}

template <int EPI>
hipError_t launch_epi(const RowArgs& a, int dtype, hipStream_t s) {
  switch (dtype) {
    case kF32:
      return launch_dt<kF32, EPI>(a, s);
    case kF16:
      return launch_dt<kF16, EPI>(a, s);
    default:
      return launch_dt<kBF16, EPI>(a, s);
  }
}

}  // namespace

int64_t lds_max_cols(int dtype) { return lds_res_max_cols(dtype); }

hipError_t launch_lds(const RowArgs& a, int dtype, int epi, hipStream_t s) {
  // rows past the register budget stay in LDS for all three passes
  if (a.cols * elem_size(dtype) > kMaxRowBytes) return launch_lds_res(a, dtype, epi, s);
  if (epi == kEpiSoftmax) return launch_epi<kEpiSoftmax>(a, dtype, s);
  if (epi == kEpiLogSoftmax) return launch_epi<kEpiLogSoftmax>(a, dtype, s);
  return launch_epi<kEpiXent>(a, dtype, s);
}

}  // namespace smx
