// smx_device.hpp — gfx950 building blocks of the row-softmax kernels:
// element formats, 128-bit row access, wave64 DPP reductions, workgroup
// reductions and the (m, l) summary merge.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smx_internal.hpp"
#include "smx_math.hpp"

namespace smx {

constexpr float kInf = __builtin_huge_valf();
constexpr float kLog2e = 1.44269502162933349609375f;

// ---------------------------------------------------------------------------
// Element formats. DT: 0 = f32, 1 = f16, 2 = bf16.
// ---------------------------------------------------------------------------

template <int DT>
struct Fmt {
  static constexpr int S = DT == kF32 ? 4 : 2;  // bytes per element
  static constexpr uint32_t kNaN = DT == kF32 ? 0x7FC00000u : (DT == kF16 ? 0x7E00u : 0x7FC0u);
  static constexpr uint32_t kNegInf = DT == kF32 ? 0xFF800000u : (DT == kF16 ? 0xFC00u : 0xFF80u);
};

// Exact widening of one element's bits to fp32.
template <int DT>
__device__ __forceinline__ float dec(uint32_t h) {
  if constexpr (DT == kF32) {
    return u2f(h);
  } else if constexpr (DT == kF16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  } else {
    return u2f(h << 16);
  }
}

// Nearest-even rounding of an fp32 value (finite or -inf; non-negative for
// probabilities, non-positive for log-probabilities) to the element format,
// gradual underflow kept; fp16 overflows to -inf as IEEE rounding does. The
// 16-bit formats use gfx950's conversion instructions (v_cvt_f16_f32,
// v_cvt_pk_bf16_f32), which round to nearest-even and keep subnormals in the
// kernels' floating-point mode.
template <int DT>
__device__ __forceinline__ uint32_t enc(float f) {
  if constexpr (DT == kF32) {
    return f2u(f);
  } else if constexpr (DT == kF16) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
  } else {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
  }
}

// Two values rounded as enc does, packed low half first: one packed
// conversion (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32) for both.
template <int DT>
__device__ __forceinline__ uint32_t enc2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 v = {a, b};
  if constexpr (DT == kF16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
  }
}

// One element rounded as enc does, stored alone (2 or 4 bytes).
template <int DT>
__device__ __forceinline__ void store_one(char* p, float f) {
  if constexpr (DT == kF32) {
    *reinterpret_cast<uint32_t*>(p) = enc<DT>(f);
  } else {
    *reinterpret_cast<uint16_t*>(p) = (uint16_t)enc<DT>(f);
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// E consecutive elements: one 128-bit access (E * S == 16) or one element.
template <int DT, int E>
struct Pack {
  static constexpr int S = Fmt<DT>::S;
  static_assert(E == 1 || E * S == 16, "a pack is 16 bytes or one element");
  static constexpr int W = E == 1 ? 1 : 4;
  uint32_t w[W];

  // NT: a nontemporal access (the `nt` bit): the data streams through the
  // caches without displacing lines that are reused
  template <bool NT = false>
  __device__ __forceinline__ void load(const char* p) {
    if constexpr (E * S == 16) {
      const u32x4 v = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p))
                         : *reinterpret_cast<const u32x4*>(p);
      w[0] = v.x;
      w[1] = v.y;
      w[2] = v.z;
      w[3] = v.w;
    } else if constexpr (S == 4) {
      const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
      w[0] = NT ? __builtin_nontemporal_load(q) : *q;
    } else {
      const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
      w[0] = NT ? __builtin_nontemporal_load(q) : *q;
    }
  }
  template <bool NT = false>
  __device__ __forceinline__ void store(char* p) const {
    if constexpr (E * S == 16) {
      const u32x4 v = {w[0], w[1], w[2], w[3]};
      if constexpr (NT) {
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
      } else {
        *reinterpret_cast<u32x4*>(p) = v;
      }
    } else if constexpr (S == 4) {
      if constexpr (NT) {
        __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(p));
      } else {
        *reinterpret_cast<uint32_t*>(p) = w[0];
      }
    } else {
      if constexpr (NT) {
        __builtin_nontemporal_store((uint16_t)w[0], reinterpret_cast<uint16_t*>(p));
      } else {
        *reinterpret_cast<uint16_t*>(p) = (uint16_t)w[0];
      }
    }
  }
  __device__ __forceinline__ float get(int e) const {
    if constexpr (S == 4) {
      return dec<DT>(w[e]);
    } else if constexpr (DT == kBF16) {
      const uint32_t word = w[e >> 1];
      return u2f((e & 1) ? (word & 0xFFFF0000u) : (word << 16));
    } else {
      return dec<DT>((w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
    }
  }
  // fill from E element bit patterns
  __device__ __forceinline__ void put(const uint32_t (&h)[E]) {
    if constexpr (S == 4 || E == 1) {
#pragma unroll
      for (int i = 0; i < E; ++i) w[i] = h[i];
    } else {
#pragma unroll
      for (int i = 0; i < E / 2; ++i) w[i] = h[2 * i] | (h[2 * i + 1] << 16);
    }
  }
  // fill from E values, each rounded to the element format as enc does
  __device__ __forceinline__ void put_values(const float (&v)[E]) {
    if constexpr (S == 4 || E == 1) {
#pragma unroll
      for (int i = 0; i < E; ++i) w[i] = enc<DT>(v[i]);
    } else {
#pragma unroll
      for (int i = 0; i < E / 2; ++i) w[i] = enc2<DT>(v[2 * i], v[2 * i + 1]);
    }
  }
  __device__ __forceinline__ void fill(uint32_t h) {
    const uint32_t word = S == 4 || E == 1 ? h : (h | (h << 16));
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = word;
  }
};

// E keep bytes of a KEEP_BYTES mask, as one integer (byte e = lane e).
template <int E>
__device__ __forceinline__ uint64_t load_keep(const uint8_t* p) {
  if constexpr (E == 8) {
    return *reinterpret_cast<const uint64_t*>(p);
  } else if constexpr (E == 4) {
    return *reinterpret_cast<const uint32_t*>(p);
  } else {
    return *p;
  }
}

__device__ __forceinline__ bool keep_lane(uint64_t k, int e) { return ((k >> (8 * e)) & 0xFFu) != 0; }

// The causal valid length of row r, (r mod period) + 1 + offset, unclamped:
// r mod period takes a short 32-bit sequence when both fit, else the 64-bit one.
__device__ __forceinline__ int64_t causal_len(const MaskArgs& mk, int64_t r) {
  const int64_t q = (((uint64_t)r | (uint64_t)mk.period) >> 32) != 0 ? r % mk.period
                                                                     : (int64_t)((uint32_t)r % (uint32_t)mk.period);
  return q + 1 + mk.offset;
}

// Valid-prefix length of row r (the whole row for NONE and KEEP_BYTES).
__device__ __forceinline__ int64_t valid_prefix(const MaskArgs& mk, int64_t r, int64_t cols) {
  int64_t v = cols;
  if (mk.kind == kMaskValidLen) {
    v = mk.valid_len[r];
  } else if (mk.kind == kMaskCausal) {
    v = causal_len(mk, r);
  }
  return v < 0 ? 0 : (v > cols ? cols : v);
}

// p[i] of an int32 array that no thread of the kernel writes (a row's valid
// length or target), read through the constant address space. With a
// uniform index that is a scalar load, waited for by itself; a plain load
// placed after the kernel's own global stores (the next row of a persistent
// loop) may not go through the scalar cache, so it becomes a vector load and
// its wait, vmcnt(0), would also drain every store and every direct LDS load
// in flight.
__device__ __forceinline__ int64_t load_readonly(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// N consecutive int32 values p[0 .. N) loaded together, every one before any
// is used: off one base address with constant offsets (so the scalar loads
// share their address registers and go out back to back, or merge), except
// where fewer than N remain (n < N, the last rows), which clamps.
template <int N>
__device__ __forceinline__ void load_run(const int32_t* p, int64_t n, int64_t (&v)[N]) {
  if (n >= N) {
#pragma unroll
    for (int r = 0; r < N; ++r) v[r] = p[r];
  } else {
#pragma unroll
    for (int r = 0; r < N; ++r) v[r] = p[r < n ? r : n - 1];
  }
}

// Valid-prefix lengths of the N consecutive rows r0 .. r0 + N - 1 (0 for
// rows at or past `rows`; r0 < rows) under a mask of compile-time class MK:
// kMaskValidLen loads the valid lengths of all N rows before using any, so
// their latencies overlap instead of queuing one after another in front of
// the rows' loads; kMaskCausal computes them; any other class is the whole
// row.
template <int MK, int N>
__device__ __forceinline__ void valid_prefixes(const MaskArgs& mk, int64_t r0, int64_t rows, int64_t cols,
                                               int (&out)[N]) {
  int64_t v[N];
  if constexpr (MK == kMaskValidLen) {
    load_run<N>(mk.valid_len + r0, rows - r0, v);
  } else if constexpr (MK == kMaskCausal) {
#pragma unroll
    for (int r = 0; r < N; ++r) v[r] = causal_len(mk, r0 + r);
  } else {
#pragma unroll
    for (int r = 0; r < N; ++r) v[r] = cols;
  }
#pragma unroll
  for (int r = 0; r < N; ++r) out[r] = r0 + r < rows ? (int)(v[r] < 0 ? 0 : (v[r] > cols ? cols : v[r])) : 0;
}

// The cross-entropy targets of the N consecutive rows r0 .. (as row_target;
// -1 for rows at or past `rows`), loaded together like valid_prefixes.
template <int N>
__device__ __forceinline__ void row_targets(const int32_t* target, int64_t r0, int64_t rows, int64_t cols,
                                            int64_t (&out)[N]) {
  int64_t t[N];
  load_run<N>(target + r0, rows - r0, t);
#pragma unroll
  for (int r = 0; r < N; ++r) out[r] = (r0 + r < rows && t[r] >= 0 && t[r] < cols) ? t[r] : -1;
}

// ---------------------------------------------------------------------------
// Exponentials, scaled by 2^64 (a normal fp32 number down to exp(-131)).
// ---------------------------------------------------------------------------

// fp32 I/O: exp(x - m) * 2^64 from the hardware base-2 exponential
// (v_exp_f32, measured within 0.79 ulp on gfx950 for normal results) with
// the difference x - m taken exactly in fp64 and the rest of the argument
// carried past the exponential as a factor 1 + r (exp_dd_b64 in
// smx_math.hpp). The 2^64 scale rides in the exponential's argument, so the
// value is a normal fp32 number down to exp(-131) (v_exp_f32 itself flushes
// subnormal results). Masked lanes (x = -inf) and d < -120 give exactly 0.
// fp64 adds, fused multiply-adds and conversions issue at the fp32 rate on
// CDNA4: twelve instructions, where the same accuracy in fp32 alone (an
// exact two-difference and a three-term product error) took nineteen.
struct HwExp2 {
  __device__ float operator()(float t) const { return __builtin_amdgcn_exp2f(t); }
};
__device__ __forceinline__ float exp_acc_b64(float x, float m) { return exp_dd_b64(x, (double)m, HwExp2{}); }

// The same exponential unscaled, for sums only (exp_dd_sum in smx_math.hpp):
// results below 2^-126 flush to zero, which changes a sum that holds a term
// equal to 1 by less than 2^-126 relative; x - m is clamped at -160 in fp64,
// so -inf lanes give 0 and a NaN lane gives 0 (the caller's maximum carries
// NaN into the row's poison flag). Ten instructions. m64 is (double)m.
__device__ __forceinline__ float exp_acc_sum(float x, double m64) { return exp_dd_sum(x, m64, HwExp2{}); }

// 16-bit I/O: the hardware base-2 exponential, v_exp_f32. Its argument
// carries a relative error of about 2^-23 |x - m|, far below half an ulp of
// bf16 or fp16 wherever the result is not rounded to zero.
__device__ __forceinline__ float exp_hw_b64(float x, float m) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(x - m, kLog2e, 64.0f));
}

// The 16-bit softmax's exponential with the row's shift folded into one
// constant: 2^(x log2 e + c), c = 64 - m log2 e, one fused multiply-add and
// one v_exp_f32 per lane. Each lane's argument is rounded once; the rounding
// of c scales every lane of the row by the same factor 2^(delta c), which the
// normalization p = e / sum(e) divides out. That holds while c is small
// enough for delta c to stay tiny (|m| < 2^15: |delta c| <= 2^-9), so rows
// with a larger maximum take exp_hw_b64. Not for outputs that keep log(sum):
// there the common factor would show.
constexpr float kBiasMaxAbs = 32768.0f;
__device__ __forceinline__ float row_exp_bias(float m) { return __builtin_fmaf(-m, kLog2e, 64.0f); }
__device__ __forceinline__ float exp_hw_bias(float x, float c) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, c));
}

// Sum of N register values as a balanced binary tree: the same N - 1
// additions as a running sum, with the error bound growing as log2 N instead
// of N ("Softmax numerics architecture", fp32 accumulator section).
template <int N>
__device__ __forceinline__ float tree_sum(const float* a) {
  if constexpr (N == 1) {
    return a[0];
  } else {
    return tree_sum<N / 2>(a) + tree_sum<N - N / 2>(a + N / 2);
  }
}

template <bool ACC>
__device__ __forceinline__ float exp_b64(float x, float m) {
  if constexpr (ACC) {
    return exp_acc_b64(x, m);
  } else {
    return exp_hw_b64(x, m);
  }
}

// log(l) for the log-sum-exp (l >= 1): the library's correctly handled
// natural logarithm (an accurate expansion of v_log_f32, not the fast one).
__device__ __forceinline__ float log_l(float l) { return __builtin_logf(l); }

// LSE = m + log l carried as hi + lo (exact sum), so x - LSE can be formed as
// (x - hi) - lo: where x is close to the LSE the first difference is exact
// and the result keeps its own relative precision.
struct Lse {
  float hi, lo;
};
__device__ __forceinline__ Lse make_lse(float m, float lsum) {
  Lse r;
  two_sum(m, log_l(lsum), r.hi, r.lo);
  return r;
}
__device__ __forceinline__ float minus_lse(float x, const Lse& s) { return (x - s.hi) - s.lo; }

// The cross-entropy of a row from its maximum m, the target logit xt, the
// sum of the other lanes' exp(x - m) ("others") and of all lanes ("all"),
// both unscaled: LSE - xt = (m - xt) + log(all). When the target holds the
// maximum, all = fl(1 + others) and the loss is log1p(others); it is taken
// as log(w) * u / (w - 1) with w = all, u = others (Goldberg, "What Every
// Computer Scientist Should Know About Floating-Point Arithmetic", Theorem 4):
// w - 1 is exact, so the quotient cancels the rounding of w, and a confident
// prediction's tiny loss keeps full fp32 relative precision at the cost of
// one logarithm (the library log1p is a far longer dependency chain).
__device__ __forceinline__ float xent_loss(float m, float xt, float others, float all) {
  const float lg = log_l(all);
  if (xt != m) return (m - xt) + lg;
  const float w1 = all - 1.0f;
  return w1 == 0.0f ? others : lg * (others / w1);
}

// The target lane of a row, or -1 when the row is ignored (target outside
// [0, cols)).
__device__ __forceinline__ int64_t row_target(const int32_t* target, int64_t row, int64_t cols) {
  const int64_t t = target[row];
  return (t >= 0 && t < cols) ? t : -1;
}

// Where the target lane t sits among one thread's registers, when element j
// of the row is slot e of pack k of thread (j / E) mod NT, with
// j = (k * NT + thread) * E + e: k * E + e for the thread holding t, -1 for
// every other thread and for t < 0. Compared with compile-time k * E + e, it
// costs one 32-bit compare per element instead of a 64-bit index.
template <int NT, int E>
__device__ __forceinline__ int target_slot(int64_t t, int tid) {
  if (t < 0) return -1;
  const int64_t q = t / E;
  return (int)(q % NT) == tid ? (int)(q / NT) * E + (int)(t % E) : -1;
}

// The epilogue's per-row scalar for the log-softmax outputs.
__device__ __forceinline__ void write_lse(float* lse, int64_t row, bool poisoned, float m, float lsum) {
  if (lse == nullptr) return;
  float v;
  if (poisoned) {
    v = u2f(0x7FC00000u);
  } else if (m == -kInf) {
    v = -kInf;
  } else {
    v = m + log_l(lsum);
  }
  lse[row] = v;
}

// ---------------------------------------------------------------------------
// The summary merge ("Online stable softmax", "Derive the update for two
// blocks"): m' = max(m, m2), l' = exp(m - m') l + exp(m2 - m') l2, the side
// holding m' with factor exactly 1. The sum is formed as a rounded product
// plus a rounded product, so merge(a, b) == merge(b, a) bit for bit (the DPP
// butterflies below rely on that to leave every lane with the same value).
// ---------------------------------------------------------------------------

__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float mm = fmaxf(m, m2);
  const float fa = exp_diff(m, mm);
  const float fb = exp_diff(m2, mm);
  const float pa = l * fa;
  const float pb = l2 * fb;
  l = pa + pb;
  m = mm;
}

// ---------------------------------------------------------------------------
// Wave64 reductions: DPP within each 16-lane row (quad_perm xor 1, xor 2,
// half-row mirror, row mirror), then the four row results read into scalars
// and combined in a fixed order. Every lane returns the same value, and the
// grouping never changes, so results are bitwise reproducible.
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15 - i within 16

__device__ __forceinline__ float lane_read(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// The IEEE maximum that propagates NaN (v_maximum3_f32 on gfx950): a NaN in
// any operand makes the result NaN, so a row's maximum is NaN exactly when a
// valid lane holds NaN, and +inf exactly when one holds +inf and none NaN.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Maximum of N register values as a balanced tree (NaN-propagating).
template <int N>
__device__ __forceinline__ float tree_max(const float* a) {
  if constexpr (N == 1) {
    return a[0];
  } else {
    return vmax(tree_max<N / 2>(a), tree_max<N - N / 2>(a + N / 2));
  }
}

__device__ __forceinline__ float wave_max(float v) {
  v = vmax(v, dpp<kDppXor1>(v));
  v = vmax(v, dpp<kDppXor2>(v));
  v = vmax(v, dpp<kDppHalfMirror>(v));
  v = vmax(v, dpp<kDppMirror>(v));
  return vmax(vmax(lane_read(v, 0), lane_read(v, 16)), vmax(lane_read(v, 32), lane_read(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = v + dpp<kDppXor1>(v);
  v = v + dpp<kDppXor2>(v);
  v = v + dpp<kDppHalfMirror>(v);
  v = v + dpp<kDppMirror>(v);
  return (lane_read(v, 0) + lane_read(v, 16)) + (lane_read(v, 32) + lane_read(v, 48));
}

// compensated pair sum: (hi, lo) + (hi2, lo2) with the rounding error of the
// high parts carried into the low part
__device__ __forceinline__ void pair_add(float& hi, float& lo, float hi2, float lo2) {
  float s, e;
  two_sum(hi, hi2, s, e);
  hi = s;
  lo = (lo + lo2) + e;
}

template <int CTRL>
__device__ __forceinline__ void pair_step(float& hi, float& lo) {
  const float h2 = dpp<CTRL>(hi);
  const float l2 = dpp<CTRL>(lo);
  pair_add(hi, lo, h2, l2);
}

// the wave's sum of (hi, lo) pairs, left as a pair in (hi, lo)
__device__ __forceinline__ void wave_pair_reduce(float& hi, float& lo) {
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
  hi = h0;
  lo = l0;
}

__device__ __forceinline__ float wave_sum_pair(float hi, float lo) {
  wave_pair_reduce(hi, lo);
  return hi + lo;
}

template <int CTRL>
__device__ __forceinline__ void ml_step(float& m, float& l) {
  const float m2 = dpp<CTRL>(m);
  const float l2 = dpp<CTRL>(l);
  merge_ml(m, l, m2, l2);
}

__device__ __forceinline__ void wave_merge(float& m, float& l) {
  ml_step<kDppXor1>(m, l);
  ml_step<kDppXor2>(m, l);
  ml_step<kDppHalfMirror>(m, l);
  ml_step<kDppMirror>(m, l);
  float m0 = lane_read(m, 0), l0 = lane_read(l, 0);
  float m1 = lane_read(m, 16), l1 = lane_read(l, 16);
  float m2 = lane_read(m, 32), l2 = lane_read(l, 32);
  float m3 = lane_read(m, 48), l3 = lane_read(l, 48);
  merge_ml(m0, l0, m1, l1);
  merge_ml(m2, l2, m3, l3);
  merge_ml(m0, l0, m2, l2);
  m = m0;
  l = l0;
}

__device__ __forceinline__ bool wave_any(bool b) { return __ballot(b) != 0; }

// ---------------------------------------------------------------------------
// Workgroup reductions over NW waves through a small LDS scratch. Every
// thread combines the NW wave results in the same order; the trailing
// barrier lets the scratch be reused at once.
// ---------------------------------------------------------------------------

struct RedScratch {
  float a[16];
  float b[16];
  int flag[16];
};

template <int NW>
__device__ __forceinline__ float block_max(float v, RedScratch& s) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) s.a[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = s.a[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = vmax(r, s.a[i]);
  __syncthreads();
  return r;
}

template <int NW>
__device__ __forceinline__ bool block_any(bool b, RedScratch& s) {
  const bool w = wave_any(b);
  if ((threadIdx.x & 63) == 0) s.flag[threadIdx.x >> 6] = w ? 1 : 0;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) r |= s.flag[i];
  __syncthreads();
  return r != 0;
}

template <int NW>
__device__ __forceinline__ float block_sum(float v, RedScratch& s) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) s.a[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = s.a[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = r + s.a[i];
  __syncthreads();
  return r;
}

// the workgroup's sum of (hi, lo) pairs, left as a pair in (hi, lo): each
// wave's result as a pair, then the pairs across waves
template <int NW>
__device__ __forceinline__ void block_pair_reduce(float& hi, float& lo, RedScratch& s) {
  wave_pair_reduce(hi, lo);
  if ((threadIdx.x & 63) == 0) {
    s.a[threadIdx.x >> 6] = hi;
    s.b[threadIdx.x >> 6] = lo;
  }
  __syncthreads();
  float rh = s.a[0], rl = s.b[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) pair_add(rh, rl, s.a[i], s.b[i]);
  __syncthreads();
  hi = rh;
  lo = rl;
}

template <int NW>
__device__ __forceinline__ float block_sum_pair(float hi, float lo, RedScratch& s) {
  block_pair_reduce<NW>(hi, lo, s);
  return hi + lo;
}

// The workgroup's summaries merged in two reductions: M = the maximum of the
// m's, then L = the sum of l * exp(m - M) (factor exactly 1 where m == M, so
// (-inf, 0) contributes nothing and an all-empty group stays (-inf, 0)). This
// equals folding the summaries with merge_ml, at one exponential per thread
// instead of one per tree level.
template <int NW>
__device__ __forceinline__ void block_merge_max_sum(float& m, float& l, RedScratch& s) {
  const float mm = block_max<NW>(m, s);
  const float scaled = l * exp_diff(m, mm);
  l = block_sum_pair<NW>(scaled, 0.0f, s);
  m = mm;
}

// The same merge with the policy flag folded in: a thread that saw NaN or
// +inf contributes the maximum +inf, so the group is poisoned exactly when M
// is +inf (and the sum is skipped). Returns whether it is poisoned.
template <int NW>
__device__ __forceinline__ bool block_merge_flagged(float& m, float& l, bool bad, RedScratch& s) {
  const float mm = block_max<NW>(bad ? kInf : m, s);
  if (mm == kInf) return true;  // uniform across the workgroup
  l = block_sum_pair<NW>(l * exp_diff(m, mm), 0.0f, s);
  m = mm;
  return false;
}

template <int NW>
__device__ __forceinline__ void block_merge(float& m, float& l, RedScratch& s) {
  wave_merge(m, l);
  if ((threadIdx.x & 63) == 0) {
    s.a[threadIdx.x >> 6] = m;
    s.b[threadIdx.x >> 6] = l;
  }
  __syncthreads();
  float rm = s.a[0], rl = s.b[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) merge_ml(rm, rl, s.a[i], s.b[i]);
  __syncthreads();
  m = rm;
  l = rl;
}

}  // namespace smx
