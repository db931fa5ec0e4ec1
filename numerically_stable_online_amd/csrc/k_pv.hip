// k_pv.hip — softmax-weighted value sums on the matrix cores:
//   out[r, :] = sum_j softmax(s[r])_j v[g, j, :],   g = r / rows_per_group,
// computed online over column blocks. The row keeps its running maximum m,
// the running sum l and the unnormalized numerator o; when a block moves the
// maximum, l and o take the same factor exp(m - m') and the block's terms
// are added relative to m' ("Online stable softmax", sections on the
// weighted-value numerator and the reference summary; "Softmax numerics
// architecture", tiled attention: the output is o / l at the end).
//
// A workgroup of four waves owns 128 rows of one group; each wave owns 32 of
// them. Per block of 64 columns:
//  * the block of V (64 x D) is copied to LDS transposed (row d holds the
//    block's 64 values of column d), so each lane's matrix-core operand is
//    one 16-byte LDS read;
//  * each lane loads 32 consecutive scores of its row (lanes l and l + 32
//    share a row and take one half of the block each), folds them into the
//    running maximum (NaN-propagating: a NaN or +inf in a valid lane
//    poisons the row), rescales its l and its 16 * D / 32 accumulators, and
//    forms p = exp(x - m');
//  * the product o^T += V^T p^T runs on v_mfma_f32_32x32x16_{bf16,f16}: the
//    accumulator's column is the lane's row, so each lane rescales only its
//    own row. p enters as a high and a low 16-bit part (p = hi + lo to about
//    16 bits), so the weights carry nearly fp32 precision into the fp32
//    accumulation; the value vectors enter exactly.
// The column order inside a block is permuted consistently between the
// score operand and the value operand (the contraction does not depend on
// it), so every lane reads its scores as contiguous 64-byte runs.
#include "smx_device.hpp"

namespace smx {
namespace {

constexpr int kPvRows = 128;   // rows per workgroup (four waves of 32)
constexpr int kPvBlock = 64;   // columns per block (four matrix-core k-steps of 16)
constexpr int kVtPitch = kPvBlock + 8;  // LDS row pitch of the transposed V block, elements

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct PvArgs {
  const char* s;
  const char* v;
  char* out;
  int64_t rows;
  int64_t cols;
  int64_t rows_per_group;
  MaskArgs mask;
};

// A row's exponentials are taken against a reference maximum mr that only
// moves when a block's maximum exceeds it by more than kSlack (natural log
// units): weights stay below e^kSlack and the reference cancels in o / l, so
// most blocks skip rescaling the accumulators. fp16 weights are also raised
// by 2^12 (p 2^12 <= e^2 2^12 stays below the fp16 maximum) so that weights
// down to 2^-36 keep their precision instead of becoming fp16 subnormals; the
// factor is divided out with 1 / l.
template <int DT>
constexpr float kSlack = DT == kF16 ? 2.0f : 8.0f;
template <int DT>
constexpr float kWeightScale = DT == kF16 ? 4096.0f : 1.0f;
// rows whose reference exceeds this in magnitude take exp(x - mr) with an
// explicit subtraction; below it, 2^(x log2e + c) with one constant per row
constexpr float kBiasedMax = 32768.0f;

// Two fp32 weights as 16-bit hi + lo pairs (p = hi + lo to about 16 bits),
// packed two to a word: one packed conversion for the high parts, the exact
// residuals, one packed conversion for the low parts.
template <int DT>
__device__ __forceinline__ void split_pair(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  hi = enc2<DT>(p0, p1);
  const float r0 = p0 - dec<DT>(hi & 0xFFFFu);  // exact: hi holds p's leading bits
  const float r1 = p1 - dec<DT>(hi >> 16);
  lo = enc2<DT>(r0, r1);
}

template <int DT>
__device__ __forceinline__ f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
}

// the largest valid prefix among the workgroup's rows (the columns it visits)
__device__ __forceinline__ int64_t block_max_i64(int64_t v, int64_t* slot) {
  for (int off = 32; off > 0; off >>= 1) {
    const int64_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = v;
  __syncthreads();
  int64_t r = slot[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = slot[i] > r ? slot[i] : r;
  __syncthreads();
  return r;
}

template <int DT, int D, bool KEEP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_pv(PvArgs a) {
  constexpr int S = 2;
  constexpr int NT = D / 32;  // 32-wide accumulator tiles along d
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * kVtPitch];
  __shared__ int64_t red64[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int h = lane >> 5;  // which half of the block this lane's scores cover
  const int wid = tid >> 6;
  const int64_t cols = a.cols;
  const int64_t rpg = a.rows_per_group;
  const int64_t tiles_per_group = (rpg + kPvRows - 1) / kPvRows;
  const int64_t total = (a.rows / rpg) * tiles_per_group;
  const int64_t per_xcd = total / 8;

  for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
    // XCD-aware order: the eight XCDs take workgroups round-robin, so
    // consecutive logical tiles (the tiles of one group, which share V) are
    // given to one XCD and its L2; within a group the longest tiles (the
    // last rows of a causal group) come first
    const int64_t lb = (total % 8 == 0) ? (b % 8) * per_xcd + b / 8 : b;
    const int64_t g = lb / tiles_per_group;
    const int64_t tile = tiles_per_group - 1 - lb % tiles_per_group;
    const int64_t row0 = g * rpg + tile * kPvRows;
    const int64_t row_end = (row0 + kPvRows < (g + 1) * rpg) ? row0 + kPvRows : (g + 1) * rpg;
    const int64_t row = row0 + wid * 32 + (lane & 31);
    const bool row_ok = row < row_end;
    const int64_t prefix = row_ok ? valid_prefix(a.mask, row, cols) : 0;
    const int64_t extent = block_max_i64(prefix, red64);
    const char* srow = a.s + (row_ok ? row : row0) * cols * S;
    const char* vg = a.v + g * cols * D * S;

    float m = -kInf, l = 0.0f;
    f32x16 acc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = f32x16{};

    // the next block's V chunks and scores, loaded while the current block
    // is computed. Thread q of the copy takes 16-byte chunks q, q + 256, ...
    // of the 64 x D block (chunk -> V row q % 64, d block q / 64): lane i of
    // a wave takes V row i, so a wave's LDS stores fill consecutive
    // positions of one row of vt.
    constexpr int CH = kPvBlock * D / 8 / kThreads;
    Pack<DT, 8> vnext[CH], snext[4];
    uint64_t knext[4];
    auto fetch = [&](int64_t c0) {
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        const int q = tid + ch * kThreads;
        const int64_t j = c0 + q % kPvBlock;
        vnext[ch].fill(0);
        if (j < cols) vnext[ch].load(vg + (j * D + 8 * (q / kPvBlock)) * S);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t j0 = c0 + 32 * h + 8 * k;
        snext[k].fill(0);
        knext[k] = ~0ull;
        if (j0 < prefix) {
          snext[k].template load<true>(srow + j0 * S);
          if constexpr (KEEP) knext[k] = load_keep<8>(a.mask.keep + row * cols + j0);
        }
      }
    };
    if (extent > 0) fetch(0);

    for (int64_t c0 = 0; c0 < extent; c0 += kPvBlock) {
      __syncthreads();  // every wave is done with the previous block's vt
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        const int q = tid + ch * kThreads;
        const int vrow = q % kPvBlock;
        const int dblk = q / kPvBlock;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          vt[(8 * dblk + e) * kVtPitch + vrow] = (uint16_t)(vnext[ch].w[e >> 1] >> (16 * (e & 1)));
      }
      // this lane's 32 scores: columns c0 + 32 h .. + 31 of its row; lanes
      // are masked element by element only when some row of the wave ends
      // inside its half block (or for arbitrary keep masks)
      float x[32];
      if (KEEP || __ballot(prefix < c0 + 32 * h + 32) != 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t left = prefix - (c0 + 32 * h + 8 * k);
          const int rem = left <= 0 ? 0 : (left >= 8 ? 8 : (int)left);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool ok = e < rem && (!KEEP || keep_lane(knext[k], e));
            x[8 * k + e] = ok ? snext[k].get(e) : -kInf;
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e) x[8 * k + e] = snext[k].get(e);
      }
      __syncthreads();
      if (c0 + kPvBlock < extent) fetch(c0 + kPvBlock);

      float bm = -kInf;
#pragma unroll
      for (int i = 0; i < 32; ++i) bm = vmax(bm, x[i]);
      bm = vmax(bm, __shfl_xor(bm, 32));  // the other half of the row
      // the reference moves to the block's maximum when that exceeds it by
      // more than the slack (or is NaN / +inf, which poisons the row, or the
      // row was empty so far); the old state then takes the factor
      // exp(m - m'), exactly 1 when nothing moves
      const float m_new = (bm <= m + kSlack<DT>) ? m : vmax(m, bm);
      const bool moved = m_new != m && m != -kInf;  // an empty state holds zeros
      if (__ballot(moved) != 0) {
        const float alpha = moved ? __builtin_amdgcn_exp2f((m - m_new) * kLog2e) : 1.0f;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[i] *= alpha;
      }
      m = m_new;
      // exp(x - m) as 2^(x log2e + c), c = -m log2e: the rounding of c scales
      // the row's weights and its l alike and cancels in o / l; a row with no
      // finite lane yet uses m = 0, so masked lanes (-inf) give 0 without
      // forming -inf - -inf
      const float mu = m == -kInf ? 0.0f : m;

      // a wave holding a row with a large reference takes exp(x - m) with an
      // explicit subtraction (rare: scores beyond 2^15)
      float c = -mu * kLog2e;
      if (__ballot(!(__builtin_fabsf(mu) < kBiasedMax)) != 0) {
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] -= mu;
        c = 0.0f;
      }

      // per k-step: the weights p = exp(x - m) of this lane's scores 8k ..
      // 8k+7 (0 for masked lanes) as 16-bit hi + lo pairs, then o^T += V^T
      // p^T on the matrix cores with the same columns of V read from vt
      // (columns c0 + 32 h + 8k ..)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[8 * k + e], kLog2e, c));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[8 * k + e + 1], kLog2e, c));
          l += p0 + p1;
          split_pair<DT>(p0 * kWeightScale<DT>, p1 * kWeightScale<DT>, hw[e / 2], lw[e / 2]);
        }
        const u32x4 phi{hw[0], hw[1], hw[2], hw[3]};
        const u32x4 plo{lw[0], lw[1], lw[2], lw[3]};
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const u32x4 av = *reinterpret_cast<const u32x4*>(&vt[(32 * i + (lane & 31)) * kVtPitch + 32 * h + 8 * k]);
          acc[i] = mfma<DT>(av, phi, acc[i]);
          acc[i] = mfma<DT>(av, plo, acc[i]);
        }
      }
    }

    // o / l; the two halves of the row hold partial sums of l
    l += __shfl_xor(l, 32);
    if (!row_ok) continue;
    const bool poisoned = !(m < kInf);
    const bool empty = m == -kInf;
    const float inv = 1.0f / (l * kWeightScale<DT>);
    char* orow = a.out + row * D * S;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // accumulator values 4q .. 4q+3 are d = 32 i + 8 q + 4 h + 0..3
        uint32_t w0, w1;
        if (poisoned) {
          w0 = w1 = Fmt<DT>::kNaN | (Fmt<DT>::kNaN << 16);
        } else if (empty) {
          w0 = w1 = 0u;
        } else {
          w0 = enc2<DT>(acc[i][4 * q + 0] * inv, acc[i][4 * q + 1] * inv);
          w1 = enc2<DT>(acc[i][4 * q + 2] * inv, acc[i][4 * q + 3] * inv);
        }
        const int d0 = 32 * i + 8 * q + 4 * h;
        *reinterpret_cast<uint2*>(orow + d0 * S) = make_uint2(w0, w1);
      }
    }
  }
}

template <int DT, int D>
hipError_t launch_d(const PvArgs& a, hipStream_t s) {
  const int64_t tiles = (a.rows / a.rows_per_group) * ((a.rows_per_group + kPvRows - 1) / kPvRows);
  const unsigned grid = (unsigned)(tiles < (1 << 20) ? tiles : (1 << 20));
  if (a.mask.kind == kMaskKeep) {
    hipLaunchKernelGGL((k_pv<DT, D, true>), dim3(grid), dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_pv<DT, D, false>), dim3(grid), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const PvArgs& a, int64_t d, hipStream_t s) {
  if (d == 32) return launch_d<DT, 32>(a, s);
  if (d == 64) return launch_d<DT, 64>(a, s);
  return launch_d<DT, 128>(a, s);
}

}  // namespace

bool pv_supported_d(int64_t d) { return d == 32 || d == 64 || d == 128; }

hipError_t launch_pv(const char* s, const char* v, char* out, int64_t rows, int64_t cols, int64_t d,
                     int64_t rows_per_group, int dtype, const MaskArgs& mask, hipStream_t stream) {
  const PvArgs a{s, v, out, rows, cols, rows_per_group, mask};
  return dtype == kF16 ? launch_dt<kF16>(a, d, stream) : launch_dt<kBF16>(a, d, stream);
}

}  // namespace smx
