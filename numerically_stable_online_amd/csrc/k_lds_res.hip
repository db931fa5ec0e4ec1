// k_lds_res.hip — one workgroup per row, the whole row resident in LDS, for
// rows too long to hold in registers (above 32 KiB, up to 152 KiB).
//
// The row is copied from HBM straight into LDS by gfx950's direct
// global->LDS loads and is read from HBM exactly once ("Stable softmax: keep
// the normalizer consistent as tiles arrive", paragraph on fused rows: a row
// that fits on chip costs one read and one write). The maximum, the sum of
// shifted exponentials and the normalized stores are three passes over LDS
// ("Kernel visualization: online softmax", overview: the three quantities of
// the safe softmax, each a pass over the row, here over on-chip copies).
//
// Every wave of the NW owns the 1 KiB pieces k * NW + w of the row (w its
// index, k = 0, 1, ...): it loads them, and lane i of the wave only ever
// touches the 16 bytes at offset 16 i of each of its pieces. So no wave waits
// on another's loads: each waits (vmcnt) for its own pieces one at a time,
// and only the two row reductions need barriers. The loads are issued as instructions the
// compiler does not track, so it inserts no wait for them; the kernel waits
// itself.
//
// Workgroups are persistent (as many as are resident at once) and take rows
// row0, row0 + G, ...; in the normalize pass each piece's slot is refilled
// with the next row's piece as soon as its last read has returned, so the
// next row streams in under this row's arithmetic and stores.
#include "smx_device.hpp"

namespace smx {
namespace {

constexpr int kPiece = 64 * 16;    // bytes of one wave's direct load
constexpr int kResMaxPieces = 152;  // LDS pieces per row: 152 KiB
// Workgroups of 8 waves (up to 19 pieces each), or of 16 for 16-bit rows of
// 64 to 144 pieces (at most nine per wave: the LDS of one workgroup with its
// 1 KiB of scratch stays within the CU's 160 KiB). Measured against 8 waves
// in one process: 128 KiB bf16 rows 5.2 % faster, 98 KiB f16 1.4 %, 64 KiB
// bf16 2.2 %, but 64 KiB fp32 rows 5.8 % slower and 33 KiB bf16 rows 3.5 %
// slower (fewer pieces per wave, the same reductions over twice the waves).
// The cross-entropy takes 16 waves only from 80 pieces, where a CU holds
// one workgroup whatever its width: at 64 pieces (two workgroups per CU) it
// measured 108.7 us with 16 waves against 98.6 us with 8 on 4096 rows of
// 32768 bf16 logits, while from 80 to 144 pieces 16 waves were 3 to 6 %
// faster.
constexpr int kWideWaves = 16;
constexpr int kWideMinPieces = 64;
constexpr int kWideMinPiecesXent = 80;
constexpr int kWideMaxPieces = 144;
constexpr int kNarrowWaves = 8;
constexpr int kResMaxPerWave = kResMaxPieces / kNarrowWaves;  // 19, the most any wave holds

// One wave's direct 16-byte-per-lane global -> LDS load: lane i's 16 bytes
// land at LDS byte address lds + 16 i (lds is the same in every lane; it
// travels in m0, and the load may not read m0 in the instruction right
// after the write, hence the wait state). m0 is not declared clobbered (the
// compiler reserves it and ignores such a declaration); nothing the
// compiler emits in this file uses m0, which the build checks.
__device__ __forceinline__ void dma_piece(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(g), "s"(lds) : "memory");
}

// The same load into a slot this lane has just read: naming the 16 bytes of
// that read makes the compiler wait for it (lgkmcnt) before the load that
// overwrites the slot.
__device__ __forceinline__ void dma_piece_after(const void* g, uint32_t lds, const u32x4& read_value) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(g), "s"(lds), "v"(read_value)
               : "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight.
// Loads return in the order they were issued, so after this every load but
// the last N has landed, whatever the stores in between do. The "memory"
// clobber keeps the compiler from moving LDS reads above the wait.
template <int N>
__device__ __forceinline__ void vm_wait_const() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// the same for a wave-uniform n in [0, kResMaxPerWave): s_waitcnt takes an
// immediate, so a ladder of scalar branches picks it
template <int N = 0>
__device__ __forceinline__ void vm_wait(int n) {
  if constexpr (N + 1 < kResMaxPerWave) {
    if (n > N) {
      vm_wait<N + 1>(n);
      return;
    }
  }
  vm_wait_const<N>();
}

// A workgroup barrier that orders LDS accesses only: no global load or store
// is waited for (a plain __syncthreads() would also wait for every
// outstanding direct load and store of the wave).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A value every lane holds alike, as the compiler's wave-uniform value: the
// branches on a row's maximum and sum become scalar, and LDS addresses stay
// in scalar registers (m0 takes one).
__device__ __forceinline__ float uniform(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }

// A compile-time tag for the form of the exponential a loop uses.
template <int K>
struct Kind {
  static constexpr int value = K;
};

// One array per reduction of a row, so that no reduction writes what another
// may still be reading; consecutive rows use two copies in turn (a row's
// copy is written again only two rows on).
template <int NW>
struct ResScratch {
  float mx[NW];
  float hi[NW];
  float lo[NW];
  float xt;  // cross-entropy: the target's logit, from the lane that holds it
};

// Workgroup reductions over the NW waves; every thread combines the wave
// results in the same order, so all of them hold the same bits.
template <int NW>
__device__ __forceinline__ float res_max(float v, ResScratch<NW>& s) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) s.mx[threadIdx.x >> 6] = v;
  lds_barrier();
  float r = s.mx[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = vmax(r, s.mx[i]);
  return uniform(r);
}

template <int NW>
__device__ __forceinline__ float res_sum(float v, ResScratch<NW>& s) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) s.hi[threadIdx.x >> 6] = v;
  lds_barrier();
  float r = s.hi[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = r + s.hi[i];
  return uniform(r);
}

template <int NW>
__device__ __forceinline__ void res_pair(float& hi, float& lo, ResScratch<NW>& s) {
  wave_pair_reduce(hi, lo);
  if ((threadIdx.x & 63) == 0) {
    s.hi[threadIdx.x >> 6] = hi;
    s.lo[threadIdx.x >> 6] = lo;
  }
  lds_barrier();
  float rh = s.hi[0], rl = s.lo[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) pair_add(rh, rl, s.hi[i], s.lo[i]);
  hi = uniform(rh);
  lo = uniform(rl);
}

// MK: kMaskNone, kMaskValidLen (valid lengths or causal: a valid prefix) or
// kMaskKeep (the keep bytes are read from memory in each pass).
template <int DT, int MK, int EPI, int NW>
__global__ __launch_bounds__(NW * 64) void k_lds_res(RowArgs a) {
  constexpr bool KEEP = MK == kMaskKeep;
  constexpr int S = Fmt<DT>::S;
  constexpr int E = 16 / S;
  constexpr bool ACC = DT == kF32;
  extern __shared__ __attribute__((aligned(1024))) char row_lds[];
  __shared__ ResScratch<NW> red2[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t cols = a.cols;
  const int icols = (int)cols;  // rows on this path hold at most 152 KiB
  const int npc = (icols / E + 63) >> 6;                     // pieces covering the row
  const int pw = npc > wid ? (npc - wid + NW - 1) / NW : 0;  // of which this wave's
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)row_lds;

  // A row's valid prefix, and the pieces of it this wave loads: pieces past
  // the prefix are never fetched (their outputs are policy zeros).
  auto prefix_of = [&](int64_t r) -> int {
    if constexpr (MK == kMaskValidLen) {  // valid lengths and causal masks
      const int64_t v = a.mask.kind == kMaskCausal ? causal_len(a.mask, r) : load_readonly(a.mask.valid_len, r);
      return (int)(v < 0 ? 0 : (v > cols ? cols : v));
    } else {
      return icols;
    }
  };
  // cross-entropy: the row's target lane, -1 for an ignored row
  auto target_of = [&](int64_t r) -> int64_t {
    const int64_t v = load_readonly(a.target, r);
    return v >= 0 && v < cols ? v : -1;
  };
  auto loaded_of = [&](int prefix) {
    const int npv = ((prefix + E - 1) / E + 63) >> 6;
    return npv > wid ? (npv - wid + NW - 1) / NW : 0;
  };
  // lanes past the prefix in its last piece load the prefix's last pack
  // again (inside the row; masked below)
  auto src_of = [&](const char* xr, int k, int prefix) {
    const int vi = (k * NW + wid) * 64 + lane;
    const int last = (prefix + E - 1) / E - 1;
    return xr + (int64_t)(vi < last ? vi : last) * 16;
  };

  int64_t row = blockIdx.x;
  if (row >= a.rows) return;
  int prefix = prefix_of(row);
  int nld = loaded_of(prefix);
  // cross-entropy: the row's target lane (-1: an ignored row), read one row
  // ahead like the prefix, so its load is not waited for at the row's start
  int64_t t = EPI == kEpiXent ? target_of(row) : -1;
  {
    const char* xr = a.x + row * cols * S;
    for (int k = 0; k < nld; ++k) dma_piece(src_of(xr, k, prefix), uniform(lds0 + (k * NW + wid) * kPiece));
  }

  int par = 0;
  for (; row < a.rows; row += gridDim.x) {
    const int64_t nrow = row + gridDim.x;
    const bool more = nrow < a.rows;
    const int prefix_n = more ? prefix_of(nrow) : 0;
    const int nld_n = more ? loaded_of(prefix_n) : 0;
    const int64_t t_n = EPI == kEpiXent && more ? target_of(nrow) : -1;
    const char* const xn = a.x + (more ? nrow : row) * cols * S;
    char* const yr = a.y + row * cols * S;
    const uint8_t* const kr = KEEP ? a.mask.keep + row * cols : nullptr;

    // cross-entropy: the one thread holding the target lane t: element t is
    // slot te of pack t / E, which is lane (t / E) % 64 of piece (t / E) / 64,
    // owned by wave piece % NW as its piece number tk = piece / NW
    int tk = -1, te = 0;
    if (EPI == kEpiXent && t >= 0) {
      const int q = (int)t / E, pc = q >> 6;
      if (pc % NW == wid && (q & 63) == lane) {
        tk = pc / NW;
        te = (int)t % E;
      }
    }

    // The wave's piece holding the cross-entropy target (-1: none). A piece
    // needs no per-lane mask when every lane's pack lies inside the valid
    // prefix and it does not hold the target (keep masks always need one);
    // the test is wave-uniform, so the two forms are scalar branches.
    int tkw = -1;
    if (EPI == kEpiXent && t >= 0) {
      const int pc = ((int)t / E) >> 6;
      if (pc % NW == wid) tkw = pc / NW;
    }
    auto full = [&](int k) { return !KEEP && ((k * NW + wid) + 1) * 64 * E <= prefix && k != tkw; };
    auto read = [&](int k) {
      return *reinterpret_cast<const u32x4*>(row_lds + (k * NW + wid) * kPiece + lane * 16);
    };
    // The valid lanes of the pack w at slot k: -inf elsewhere (and at the
    // cross-entropy's target, whose logit joins the maximum and the total
    // apart from the others; xt_slot gets that logit, or -inf when masked).
    auto vals = [&](int k, const u32x4& w, float (&v)[E], float& xt_slot) {
      Pack<DT, E> p;
      p.w[0] = w.x;
      p.w[1] = w.y;
      p.w[2] = w.z;
      p.w[3] = w.w;
      if (full(k)) {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = p.get(e);
        return;
      }
      const int vi = (k * NW + wid) * 64 + lane;
      const int left = prefix - vi * E;
      const int rem = left <= 0 ? 0 : (left >= E ? E : left);
      uint64_t kb = ~0ull;
      if constexpr (KEEP) {
        if (rem > 0) kb = load_keep<E>(kr + vi * E);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool ok = e < rem && (!KEEP || keep_lane(kb, e));
        const bool target = EPI == kEpiXent && k == tk && e == te;
        if (target) xt_slot = ok ? p.get(e) : -kInf;
        v[e] = ok && !target ? p.get(e) : -kInf;
      }
    };

    // exp(x - m) * 2^64 against the row maximum m, three forms: fp32
    // (kind 0) the compensated exponential; 16-bit the hardware exponential
    // with the row's shift folded into one constant (kind 1, softmax with
    // |m| < 2^15) or subtracted (kind 2). The form is chosen once per row,
    // outside the loops.
    float m_row = -kInf;  // set after pass 1
    float c_row = 0.0f;
    auto ex = [&](auto kind, float x) {
      constexpr int K = decltype(kind)::value;
      if constexpr (K == 0) {
        return exp_acc_b64(x, m_row);
      } else if constexpr (K == 1) {
        return exp_hw_bias(x, c_row);
      } else {
        return exp_hw_b64(x, m_row);
      }
    };

    // pass 1: each lane's running maximum and sum of exponentials over its
    // packs, as the packs land (two at a time, each pair waited for): the
    // online recurrence of "Online stable softmax" ("Derive the update for
    // two blocks"), per lane. When the lane's reference moves up, the lane's
    // sum first takes the factor exp(ref_old - ref_new). The lane's sum is
    // kept against its own reference: 16-bit softmax the folded constant
    // c_l = 64 - m_l log2 e, so its terms are exp2(x log2 e + c_l); fp32
    // (compensated exponentials, a Kahan sum) and 16-bit log-softmax and
    // cross-entropy a reference r_l that moves only when the lane maximum
    // passes it by more than kRefSlack, so terms exp(x - r_l) stay below
    // e^16 and the accurate rescale factor (about 25 instructions, paid by
    // the whole wave whenever any lane takes it) is taken less often than
    // the maximum rises. Those terms are unscaled, with
    // x - r_l in fp64 (the loss and log-sum-exp are fp32 results; the
    // normalize pass takes its own exponentials, so these serve the sum
    // alone), and enter the 2^64 scale when the lanes merge (after one last
    // rescale to the lane's own maximum). The maximum
    // propagates NaN, so its reduction also gives the row's policy.
    constexpr bool FOLD = !ACC && EPI == kEpiSoftmax;
    constexpr float kRefSlack = 8.0f;
    float m_l = -kInf, r_l = -kInf, c_l = 0.0f, l_l = 0.0f;
    KahanSum ks;
    float xt_own = -kInf;
    auto fold_pack = [&](const float (&v)[E]) {
      const float mn = vmax(m_l, tree_max<E>(v));
      if constexpr (FOLD) {
        if (mn != m_l) {  // a new lane maximum (or NaN, whose row is poisoned)
          const float cn = row_exp_bias(mn);
          l_l = m_l == -kInf ? 0.0f : l_l * __builtin_amdgcn_exp2f(cn - c_l);
          c_l = cn;
        }
      } else if (!(mn <= r_l + kRefSlack)) {  // also taken for NaN
        const float f = exp_diff(r_l, mn);    // 0 when r_l is -inf
        if constexpr (ACC) {
          ks.s *= f;
          ks.c *= f;
        } else {
          l_l = r_l == -kInf ? 0.0f : l_l * f;
        }
        r_l = mn;
      }
      m_l = mn;
      float e[E];
      const float mref = r_l == -kInf ? 0.0f : r_l;  // an all-masked lane adds exact zeros
#pragma unroll
      for (int q = 0; q < E; ++q) {
        if constexpr (FOLD) {
          e[q] = exp_hw_bias(v[q], c_l);
        } else {
          e[q] = exp_acc_sum(v[q], (double)mref);
        }
      }
      if constexpr (ACC) {
        ks.add(tree_sum<E>(e));
      } else {
        l_l += tree_sum<E>(e);
      }
    };
    {
      int k = 0;
      for (; k + 1 < nld; k += 2) {
        vm_wait(nld - 2 - k);
        const u32x4 wa = read(k), wb = read(k + 1);
        float va[E], vb[E];
        vals(k, wa, va, xt_own);
        vals(k + 1, wb, vb, xt_own);
        fold_pack(va);
        fold_pack(vb);
      }
      if (k < nld) {
        vm_wait(0);
        const u32x4 wa = read(k);
        float va[E];
        vals(k, wa, va, xt_own);
        fold_pack(va);
      }
    }
    // each lane's sum brought to its own maximum (its reference lies at most
    // 16 below it), once per row: the merge factor below then drops only
    // lanes more than 120 below the row maximum, whose terms no fp32 result
    // can hold, and not lanes whose reference alone lies that far below
    if constexpr (!FOLD) {
      const float g = exp_diff(r_l, m_l);  // 1 when equal (also -inf, -inf)
      if constexpr (ACC) {
        ks.s *= g;
        ks.c *= g;
      } else {
        l_l *= g;
      }
    }
    // the row's reduction scratch: two copies, alternating from row to row
    ResScratch<NW>& red = red2[par];
    if (EPI == kEpiXent && tk >= 0) red.xt = xt_own;
    float mx = res_max(m_l, red);
    float xt = -kInf;
    if constexpr (EPI == kEpiXent) {
      if (t >= 0) xt = uniform(red.xt);
      mx = vmax(mx, xt);  // the target's logit counts toward the maximum and the policy
    }
    const bool poisoned = !(mx < kInf);
    const bool ignored = EPI == kEpiXent && t < 0;
    const bool fill = ignored || poisoned || mx == -kInf;
    m_row = mx;
    const bool bias = FOLD && __builtin_fabsf(mx) < kBiasMaxAbs;
    c_row = bias ? row_exp_bias(mx) : 0.0f;

    // the lanes' sums merged against the row maximum (factor exactly 1 for
    // a lane holding it, 0 for an all-masked lane), in the 2^64 scale of the
    // normalize pass's exponentials
    float total = 0.0f, others = 0.0f;
    if (!fill) {
      if constexpr (ACC) {
        // the factor in the 2^64 scale: a lane far below the maximum keeps
        // its relative precision, which the cross-entropy's loss of a
        // confident row is made of
        const float f = exp_diff_b64(m_l, mx);
        float hi = ks.hi() * f, lo = ks.lo() * f;
        res_pair(hi, lo, red);
        if constexpr (EPI == kEpiXent) {
          others = hi + lo;
          pair_add(hi, lo, exp_acc_b64(xt, mx), 0.0f);
        }
        total = hi + lo;
      } else if (FOLD && !bias) {
        // |m| >= 2^15: the folded constants are too coarse, so the sum is
        // taken again from LDS with the shift subtracted
        float sa = 0.0f;
        for (int k = 0; k < nld; ++k) {
          float v[E], unused;
          vals(k, read(k), v, unused);
#pragma unroll
          for (int q = 0; q < E; ++q) v[q] = ex(Kind<2>{}, v[q]);
          sa += tree_sum<E>(v);
        }
        total = res_sum(sa, red);
      } else {
        float f;
        if constexpr (FOLD) {
          f = m_l == mx ? 1.0f : (m_l == -kInf ? 0.0f : __builtin_amdgcn_exp2f(c_row - c_l));
        } else {
          f = exp_diff_b64(m_l, mx);  // the unscaled lane sum into the 2^64 scale, as above
        }
        total = res_sum(l_l * f, red);
        if constexpr (EPI == kEpiXent) {
          others = total;
          total = others + exp_acc_b64(xt, mx);
        }
      }
    }

    // the per-row scalars
    float inv = 0.0f;
    Lse lse{0.0f, 0.0f};
    if (fill) {
      if (EPI == kEpiLogSoftmax && tid == 0) write_lse(a.lse, row, poisoned, mx, 0.0f);
      if (EPI == kEpiXent && tid == 0) a.loss[row] = ignored ? 0.0f : (poisoned ? u2f(0x7FC00000u) : kInf);
    } else if constexpr (EPI == kEpiLogSoftmax) {
      const float lsum = total * 5.42101086242752217e-20f;  // remove 2^64 (exact)
      lse = make_lse(mx, lsum);
      if (tid == 0) write_lse(a.lse, row, false, mx, lsum);
    } else {
      inv = 1.0f / total;
    }
    // the cross-entropy's gradient at the target: -(others / l), exactly -1
    // when the target lane is masked (an empty row included)
    const float at_t = fill ? -1.0f : (0.0f - others) / total;

    // pass 3: the normalized stores, two pieces at a time, each slot refilled
    // with the next row's piece once its last read has returned; pieces past
    // the prefix (and every piece of a policy row) are stored without a read
    auto put = [&](int k, const Pack<DT, E>& out) {
      const int j0 = ((k * NW + wid) * 64 + lane) * E;
      if (a.y != nullptr && j0 < icols) out.template store<true>(yr + j0 * S);
    };
    auto refill = [&](int k, const u32x4& w) {
      if (k < nld_n) dma_piece_after(src_of(xn, k, prefix_n), uniform(lds0 + (k * NW + wid) * kPiece), w);
    };
    auto norm = [&](auto kind, int k, const u32x4& w) {
      float v[E], o[E], unused;
      vals(k, w, v, unused);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if constexpr (EPI == kEpiLogSoftmax) {
          o[e] = minus_lse(v[e], lse);
        } else {
          o[e] = ex(kind, v[e]) * inv;  // 0 at masked lanes and at the cross-entropy's target
        }
      }
      Pack<DT, E> out;
      out.put_values(o);
      return out;
    };
    const u32x4 none = {0u, 0u, 0u, 0u};
    auto store_pass = [&](auto kind) {
      int k = 0;
      for (; k + 1 < nld; k += 2) {
        const u32x4 wa = read(k), wb = read(k + 1);
        const Pack<DT, E> pa = norm(kind, k, wa), pb = norm(kind, k + 1, wb);
        put(k, pa);
        put(k + 1, pb);
        refill(k, wa);
        refill(k + 1, wb);
      }
      if (k < nld) {
        const u32x4 wa = read(k);
        put(k, norm(kind, k, wa));
        refill(k, wa);
        ++k;
      }
      Pack<DT, E> z;
      z.fill(EPI == kEpiLogSoftmax ? Fmt<DT>::kNegInf : 0u);
      for (; k < pw; ++k) {
        put(k, z);
        refill(k, none);
      }
    };
    if (fill) {
      Pack<DT, E> f;
      // an ignored row's gradient is +0.0 even when the row holds NaN or +inf
      f.fill(ignored ? 0u : (poisoned ? Fmt<DT>::kNaN : (EPI == kEpiLogSoftmax ? Fmt<DT>::kNegInf : 0u)));
      for (int k = 0; k < pw; ++k) {
        put(k, f);
        refill(k, none);
      }
    } else if constexpr (ACC) {
      store_pass(Kind<0>{});
    } else if (bias) {
      store_pass(Kind<1>{});
    } else {
      store_pass(Kind<2>{});
    }
    // the cross-entropy's gradient at the target, over the value its pack
    // wrote (the same thread, so the two stores land in order); the loss
    if constexpr (EPI == kEpiXent) {
      if (tk >= 0 && !ignored && !poisoned && a.y != nullptr) store_one<DT>(yr + t * S, at_t);
      if (!fill && tid == 0) {
        a.loss[row] = xent_loss(mx, xt, others * 5.42101086242752217e-20f, total * 5.42101086242752217e-20f);
      }
    }
    prefix = prefix_n;
    nld = nld_n;
    t = t_n;
    // the next row uses the other copy of the scratch; this row's copy is
    // written again two rows on, after the next row's first barrier, which
    // every thread reaches only once it has read this row's reductions
    par ^= 1;
  }
}

constexpr int kMaxDevices = 64;

// Launch one kernel instance with as many workgroups as are resident at once
// (capped by the rows): the CU count per device and the instance's resident
// workgroups per CU for each LDS size are looked up once and kept (0 = not
// yet known); the instance is also allowed the LDS it asks for once.
template <int DT, int MK, int EPI, int NW>
hipError_t launch_nw(const RowArgs& a, int pieces, hipStream_t s) {
  static int cu_count[kMaxDevices];
  static int per_cu[kMaxDevices][kResMaxPieces + 1];
  static int lds_allowed[kMaxDevices];
  auto kernel = k_lds_res<DT, MK, EPI, NW>;
  const size_t lds = (size_t)pieces * kPiece;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (__atomic_load_n(&lds_allowed[dev], __ATOMIC_RELAXED) == 0) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            kResMaxPieces * kPiece);
    if (e != hipSuccess) return e;
    __atomic_store_n(&lds_allowed[dev], 1, __ATOMIC_RELAXED);
  }
  int cus = __atomic_load_n(&cu_count[dev], __ATOMIC_RELAXED);
  if (cus == 0) {
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    __atomic_store_n(&cu_count[dev], cus, __ATOMIC_RELAXED);
  }
  int occ = __atomic_load_n(&per_cu[dev][pieces], __ATOMIC_RELAXED);
  if (occ == 0) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, NW * 64, lds);
    if (e != hipSuccess) return e;
    if (occ <= 0) return hipErrorInvalidConfiguration;
    __atomic_store_n(&per_cu[dev][pieces], occ, __ATOMIC_RELAXED);
  }
  const int64_t resident = (int64_t)cus * occ;
  const unsigned grid = (unsigned)(a.rows < resident ? a.rows : resident);
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

template <int DT, int MK, int EPI>
hipError_t launch_mk(const RowArgs& a, hipStream_t s) {
  constexpr int S = Fmt<DT>::S;
  const int pieces = (int)((a.cols * S + kPiece - 1) / kPiece);
  constexpr int kMin = EPI == kEpiXent ? kWideMinPiecesXent : kWideMinPieces;
  if (DT != kF32 && pieces >= kMin && pieces <= kWideMaxPieces)
    return launch_nw<DT, MK, EPI, kWideWaves>(a, pieces, s);
  return launch_nw<DT, MK, EPI, kNarrowWaves>(a, pieces, s);
}

template <int DT, int EPI>
hipError_t launch_dt(const RowArgs& a, hipStream_t s) {
  if (a.mask.kind == kMaskKeep) return launch_mk<DT, kMaskKeep, EPI>(a, s);
  if (a.mask.kind == kMaskNone) return launch_mk<DT, kMaskNone, EPI>(a, s);
  return launch_mk<DT, kMaskValidLen, EPI>(a, s);
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

int64_t lds_res_max_cols(int dtype) { return (int64_t)kResMaxPieces * kPiece / elem_size(dtype); }

hipError_t launch_lds_res(const RowArgs& a, int dtype, int epi, hipStream_t s) {
  if (epi == kEpiSoftmax) return launch_epi<kEpiSoftmax>(a, dtype, s);
  if (epi == kEpiLogSoftmax) return launch_epi<kEpiLogSoftmax>(a, dtype, s);
  return launch_epi<kEpiXent>(a, dtype, s);
}

}  // namespace smx
