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

// fp16 weights are raised by 2^15 (p <= 1, so p 2^15 stays below the fp16
// maximum) so that weights down to 2^-39 keep their precision instead of
// becoming fp16 subnormals; the factor is divided out with 1 / l
template <int DT>
constexpr float kWeightScale = DT == kF16 ? 32768.0f : 1.0f;

// 16-bit pair rounding of an fp32 weight: p = hi + lo to about 16 bits
template <int DT>
__device__ __forceinline__ void split16(float p, uint16_t& hi, uint16_t& lo) {
  hi = (uint16_t)enc<DT>(p);
  const float r = p - dec<DT>(hi);  // exact: hi holds p's leading bits
  lo = (uint16_t)enc<DT>(r);
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
__global__ __launch_bounds__(kThreads) void k_pv(PvArgs a) {
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

    for (int64_t c0 = 0; c0 < extent; c0 += kPvBlock) {
      // the block of V, transposed into LDS: thread q copies 16-byte chunks
      // (8 values of one row of V); lane i of a wave takes V row i, so the
      // LDS stores of a wave fill consecutive positions of one row of vt
      __syncthreads();  // every wave is done with the previous block
#pragma unroll
      for (int q = tid; q < kPvBlock * D / 8; q += kThreads) {
        const int vrow = q % kPvBlock;
        const int dblk = q / kPvBlock;
        const int64_t j = c0 + vrow;
        Pack<DT, 8> p;
        p.fill(0);
        if (j < cols) p.load(vg + (j * D + 8 * dblk) * S);
#pragma unroll
        for (int e = 0; e < 8; ++e) vt[(8 * dblk + e) * kVtPitch + vrow] = (uint16_t)(p.w[e >> 1] >> (16 * (e & 1)));
      }
      __syncthreads();

      // this lane's 32 scores: columns c0 + 32 h .. + 31 of its row
      float x[32];
      const int64_t cb = c0 + 32 * h;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t j0 = cb + 8 * k;
        const int64_t left = prefix - j0;
        const int rem = left <= 0 ? 0 : (left >= 8 ? 8 : (int)left);
        Pack<DT, 8> p;
        p.fill(0);
        uint64_t kb = ~0ull;
        if (rem > 0) {
          p.template load<true>(srow + j0 * S);
          if constexpr (KEEP) kb = load_keep<8>(a.mask.keep + row * cols + j0);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool ok = e < rem && (!KEEP || keep_lane(kb, e));
          x[8 * k + e] = ok ? p.get(e) : -kInf;
        }
      }
      float bm = -kInf;
#pragma unroll
      for (int i = 0; i < 32; ++i) bm = vmax(bm, x[i]);
      bm = vmax(bm, __shfl_xor(bm, 32));  // the other half of the row
      const float m_new = vmax(m, bm);
      // the old state's factor: exactly 1 when the maximum does not move
      // (also when both are -inf: no -inf - -inf); 0 for an empty state
      const float alpha = m == m_new ? 1.0f : __builtin_amdgcn_exp2f((m - m_new) * kLog2e);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[i] *= alpha;

      // weights p = exp(x - m) (0 for masked lanes), split into 16-bit pairs
      u32x4 phi[4], plo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint16_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xv = x[8 * k + e];
          const float p = xv == -kInf ? 0.0f : __builtin_amdgcn_exp2f((xv - m) * kLog2e);
          l += p;
          split16<DT>(p * kWeightScale<DT>, hi[e], lo[e]);
        }
        phi[k] = u32x4{hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16),
                       hi[4] | ((uint32_t)hi[5] << 16), hi[6] | ((uint32_t)hi[7] << 16)};
        plo[k] = u32x4{lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16),
                       lo[4] | ((uint32_t)lo[5] << 16), lo[6] | ((uint32_t)lo[7] << 16)};
      }

      // o^T += V^T p^T: k-step k pairs this lane's scores 8k .. 8k+7 (columns
      // cb + 8k ..) with the same columns of V, read from vt
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const u32x4 av = *reinterpret_cast<const u32x4*>(&vt[(32 * i + (lane & 31)) * kVtPitch + 32 * h + 8 * k]);
          acc[i] = mfma<DT>(av, phi[k], acc[i]);
          acc[i] = mfma<DT>(av, plo[k], acc[i]);
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
