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

template <int DT, int NT, int VPT, bool KEEP, int EPI>
__global__ __launch_bounds__(NT) void k_lds(RowArgs a) {
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

  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const int64_t prefix = valid_prefix(a.mask, row, cols);
    const char* xr = a.x + row * cols * S;
    char* yr = a.y + row * cols * S;

    // stage the valid prefix: wave w copies pieces w, w + 4, ...
    const int64_t nvec = (prefix + E - 1) / E;
    const int64_t npieces = (nvec + 63) / 64;
    for (int64_t pc = wid; pc < npieces; pc += NW) {
      const int64_t vi = pc * 64 + lane;
      const int64_t vsrc = vi < nvec ? vi : nvec - 1;  // stays inside the row
      __builtin_amdgcn_global_load_lds(
          (const void*)(xr + vsrc * 16),
          (__attribute__((address_space(3))) void*)(row_lds + pc * kPiece), 16, 0, kAuxNT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    float v[VPT][E];
    float mx = -kInf;
    bool bad = false;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int64_t vi = (int64_t)k * NT + tid;
      const int64_t j0 = vi * E;
      Pack<DT, E> p;
      p.fill(0);
      uint64_t kb = ~0ull;
      const bool ld = j0 < prefix;
      if (ld) {
        const uint4 w = *reinterpret_cast<const uint4*>(row_lds + vi * 16);
        p.w[0] = w.x;
        p.w[1] = w.y;
        p.w[2] = w.z;
        p.w[3] = w.w;
        if constexpr (KEEP) kb = load_keep<E>(a.mask.keep + row * cols + j0);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool ok = ld && (j0 + e < prefix) && (!KEEP || keep_lane(kb, e));
        const float f = ok ? p.get(e) : -kInf;
        bad |= !(f < kInf);
        mx = fmaxf(mx, f);
        v[k][e] = f;
      }
    }
    // the reductions' barriers also release the LDS row for the next one; a
    // thread that saw NaN or +inf contributes +inf, so the row is poisoned
    // exactly when its maximum is +inf
    mx = block_max<NW>(bad ? kInf : mx, red);
    const bool poisoned = mx == kInf;

    // cross-entropy: the row's target lane (-1: ignored row) and its logit
    int64_t t = -1;
    float xt = -kInf;
    if constexpr (EPI == kEpiXent) {
      t = row_target(a.target, row, cols);
      if (t < 0) {  // ignored row: loss 0, gradient 0
        if (tid == 0) a.loss[row] = 0.0f;
        if (a.y != nullptr) {
          Pack<DT, E> z;
          z.fill(0u);
#pragma unroll
          for (int k = 0; k < VPT; ++k) {
            const int64_t j0 = ((int64_t)k * NT + tid) * E;
            if (j0 < cols) z.template store<true>(yr + j0 * S);
          }
        }
        continue;
      }
      if (t < prefix && (!KEEP || a.mask.keep[row * cols + t] != 0)) {
        Pack<DT, 1> q;
        q.load(a.x + (row * cols + t) * S);
        xt = q.get(0);
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
          const int64_t j0 = ((int64_t)k * NT + tid) * E;
          if (j0 < cols) {
            uint32_t h[E];
#pragma unroll
            for (int e = 0; e < E; ++e) h[e] = (!poisoned && j0 + e == t) ? enc<DT>(-1.0f) : fill;
            Pack<DT, E> p;
            p.put(h);
            p.template store<true>(yr + j0 * S);
          }
        }
      }
      continue;
    }

    float total, others = 0.0f;
    if constexpr (ACC) {
      KahanSum ks, ko;
#pragma unroll
      for (int k = 0; k < VPT; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float te = exp_acc_b64(v[k][e], mx);
          if constexpr (EPI != kEpiLogSoftmax) v[k][e] = te;
          ks.add(te);
          if constexpr (EPI == kEpiXent) ko.add(((int64_t)k * NT + tid) * E + e == t ? 0.0f : te);
        }
      total = block_sum_pair<NW>(ks.hi(), ks.lo(), red);
      if constexpr (EPI == kEpiXent) others = block_sum_pair<NW>(ko.hi(), ko.lo(), red);
    } else {
      float s = 0.0f, so = 0.0f;
#pragma unroll
      for (int k = 0; k < VPT; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float te = exp_hw_b64(v[k][e], mx);
          if constexpr (EPI != kEpiLogSoftmax) v[k][e] = te;
          s += te;
          if constexpr (EPI == kEpiXent) so += ((int64_t)k * NT + tid) * E + e == t ? 0.0f : te;
        }
      total = block_sum<NW>(s, red);
      if constexpr (EPI == kEpiXent) others = block_sum<NW>(so, red);
    }

    float inv = 0.0f;  // softmax / cross-entropy: the reciprocal 2^-64 / l
    Lse lse{0.0f, 0.0f};  // log-softmax: m + log l as hi + lo
    if constexpr (EPI == kEpiLogSoftmax) {
      const float lsum = total * 5.42101086242752217e-20f;  // remove 2^64 (exact)
      lse = make_lse(mx, lsum);
      if (tid == 0) write_lse(a.lse, row, false, mx, lsum);
      if (a.y == nullptr) continue;
    } else {
      inv = 1.0f / total;
      if constexpr (EPI == kEpiXent) {
        if (tid == 0) {
          a.loss[row] = xent_loss(mx, xt, others * 5.42101086242752217e-20f, total * 5.42101086242752217e-20f);
        }
        if (a.y == nullptr) continue;
      }
    }
    // cross-entropy target lane: -(others / l), correctly rounded (exactly -1
    // when the target lane is masked)
    const float at_t = (0.0f - others) / total;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int64_t j0 = ((int64_t)k * NT + tid) * E;
      if (j0 < cols) {
        uint32_t h[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float val;
          if constexpr (EPI == kEpiLogSoftmax) {
            val = minus_lse(v[k][e], lse);
          } else {
            val = (EPI == kEpiXent && j0 + e == t) ? at_t : v[k][e] * inv;
          }
          h[e] = enc<DT>(val);
        }
        Pack<DT, E> p;
        p.put(h);
        p.template store<true>(yr + j0 * S);
      }
    }
  }
}

// rows up to 8 packs per thread of a 256-thread workgroup: 32 KiB of LDS,
// 32 (f32) or 64 (16-bit) register-resident values per thread
constexpr int64_t kMaxRowBytes = 256 * 8 * 16;

template <int DT, int NT, int VPT, int EPI>
hipError_t launch_vpt(const RowArgs& a, hipStream_t s) {
  constexpr int S = Fmt<DT>::S;
  const int64_t bytes = ((a.cols * S + kPiece - 1) / kPiece) * kPiece;
  const unsigned grid = (unsigned)(a.rows < (1 << 20) ? a.rows : (1 << 20));
  if (a.mask.kind == kMaskKeep) {
    hipLaunchKernelGGL((k_lds<DT, NT, VPT, true, EPI>), dim3(grid), dim3(NT), (size_t)bytes, s, a);
  } else {
    hipLaunchKernelGGL((k_lds<DT, NT, VPT, false, EPI>), dim3(grid), dim3(NT), (size_t)bytes, s, a);
  }
  return hipGetLastError();
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

int64_t lds_max_cols(int dtype) { return kMaxRowBytes / elem_size(dtype); }

hipError_t launch_lds(const RowArgs& a, int dtype, int epi, hipStream_t s) {
  if (epi == kEpiSoftmax) return launch_epi<kEpiSoftmax>(a, dtype, s);
  if (epi == kEpiLogSoftmax) return launch_epi<kEpiLogSoftmax>(a, dtype, s);
  return launch_epi<kEpiXent>(a, dtype, s);
}

}  // namespace smx
