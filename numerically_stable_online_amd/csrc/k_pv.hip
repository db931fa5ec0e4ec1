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
// them. Blocks of 64 columns of the scores and of V travel HBM -> LDS by
// direct loads into a two-stage ring (the next block loads while the
// current one is computed). Per block:
//  * each lane takes 32 consecutive scores of its row (lanes l and l + 32
//    share a row and take one half of the block each), folds them into the
//    running maximum (NaN-propagating: a NaN or +inf in a valid lane
//    poisons the row), rescales its l and its 16 * D / 32 accumulators when
//    the reference moves, and forms p = exp(x - m');
//  * V stays in LDS as it is in memory; gfx950's transposing LDS read
//    (ds_read_b64_tr_b16) hands each lane the column of V its matrix-core
//    operand needs;
//  * the product o^T += V^T p^T runs on v_mfma_f32_32x32x16_{bf16,f16}: the
//    accumulator's column is the lane's row, so each lane rescales only its
//    own row. p enters as a high and a low 16-bit part (p = hi + lo to about
//    16 bits), so the weights carry nearly fp32 precision into the fp32
//    accumulation; the value vectors enter exactly.
// The column order inside a block is permuted consistently between the
// score operand and the value operand (the contraction does not depend on
// it), so every lane's scores are 64 contiguous bytes of its row.
#include "smx_device.hpp"

namespace smx {
namespace {

constexpr int kPvRows = 128;    // rows per workgroup (four waves of 32)
constexpr int kPvBlock = 64;    // columns per block (four matrix-core k-steps of 16)
constexpr int kPvStages = 2;    // blocks resident in the LDS ring: one computed, one loading
constexpr int kPiece = 64 * 16; // bytes one wave's direct global->LDS load moves
constexpr int kSBytes = kPvRows * kPvBlock * 2;  // one score block: 128 rows of 128 bytes

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

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

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding and leaves the other counters alone (vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 at its maximum, lgkmcnt 11:8 at its maximum)
constexpr int vmcnt_at_most(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (7 << 4) | (0xF << 8); }

// One wave's direct 16-byte-per-lane global -> LDS load: lane i's 16 bytes
// land at LDS byte address lds + 16 i (lds must be the same in every lane).
// Issued as an instruction the compiler does not track, so that it inserts
// no wait for it before later LDS accesses (which would empty the pipeline);
// the kernel waits for these loads itself (vmcnt) before its barriers.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds, bool nt) {
  if (nt) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(g), "s"(lds) : "memory", "m0");
  } else {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(lds) : "memory", "m0");
  }
}

// A workgroup barrier that orders LDS accesses only: the wave's LDS stores
// complete before it, but no global load is waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS layout of a stage: the score block (128 rows of 128 bytes), then the
// V block (64 rows of D values, untransposed). Both are stored in 16-byte
// chunks whose position in their row is XOR-swizzled by the row, so that
// the reads below spread over the LDS banks.
__device__ __forceinline__ int s_pos(int row, int chunk) { return chunk ^ (row & 7); }
template <int D>
__device__ __forceinline__ int v_pos(int row, int chunk) {
  constexpr int kMask = D / 8 - 1 < 7 ? D / 8 - 1 : 7;
  return chunk ^ ((2 * row) & kMask);
}

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

// v_mfma_f32_32x32x16_{bf16,f16}: A 32 x 16 (lane l: row l % 32, k 8 (l / 32)
// .. + 7), B 16 x 32 (lane l: column l % 32, the same k), D 32 x 32 (lane l:
// column l % 32, value v at row 8 (v / 4) + 4 (l / 32) + v % 4). Operands
// are passed as whole vectors.
template <int DT>
__device__ __forceinline__ f32x16 mfma(const i16x8& a, const u32x4& b, const f32x16& c) {
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
  constexpr int NT = D / 32;                          // 32-wide accumulator tiles along d
  constexpr int kVBytes = kPvBlock * D * S;
  constexpr int kStage = kSBytes + kVBytes;
  constexpr int kSPieces = kSBytes / kPiece / kWaves;  // 4 per wave
  constexpr int kVPieces = kVBytes / kPiece;           // 16, 8 or 4
  constexpr int kVPerWave = kVPieces / kWaves;         // 4, 2 or 1
  constexpr int kLoads = kSPieces + kVPerWave;         // direct loads per wave per block
  constexpr int kVRowsPerPiece = kPiece / (D * S);
  constexpr int kVChunks = D / 8;
  __shared__ __attribute__((aligned(1024))) char ring[kPvStages * kStage];
  __shared__ int64_t red64[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int h = lane >> 5;  // which half of the block's columns this lane's scores cover
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)ring;
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
    const int64_t nblocks = (extent + kPvBlock - 1) / kPvBlock;
    const char* vg = a.v + g * cols * D * S;

    // this lane's share of a block's direct loads. Scores: wave w fills
    // pieces 4w .. 4w+3 (8 rows each); lane i fills LDS row 8p + i / 8 at
    // chunk position i % 8 with the chunk that position holds; a chunk past
    // its row's valid prefix is replaced by the row's first chunk (cached,
    // never used), so masked scores cost no HBM traffic. V: wave w fills
    // pieces of kVRowsPerPiece rows; a row past the end is replaced by the
    // last row (finite, weight 0).
    const char* ld_base[kSPieces];
    int64_t ld_prefix[kSPieces];
#pragma unroll
    for (int q = 0; q < kSPieces; ++q) {
      const int r = 8 * (wid * kSPieces + q) + lane / 8;
      const bool ok = row0 + r < row_end;
      ld_base[q] = a.s + (ok ? row0 + r : row0) * cols * S;
      ld_prefix[q] = ok ? valid_prefix(a.mask, row0 + r, cols) : 0;
    }
    auto issue = [&](int64_t blk) {
      const uint32_t st = ring_lds + (uint32_t)(blk % kPvStages) * kStage;
      const int64_t c0 = blk * kPvBlock;
#pragma unroll
      for (int q = 0; q < kSPieces; ++q) {
        const int r = 8 * (wid * kSPieces + q) + lane / 8;
        const int64_t col = c0 + 8 * s_pos(r, lane % 8);
        dma16(ld_base[q] + (col < ld_prefix[q] ? col : 0) * S, st + (wid * kSPieces + q) * kPiece, true);
      }
#pragma unroll
      for (int q = 0; q < kVPerWave; ++q) {
        const int piece = wid * kVPerWave + q;
        const int r = piece * kVRowsPerPiece + lane / kVChunks;
        const int64_t vrow = c0 + r < cols ? c0 + r : cols - 1;
        dma16(vg + (vrow * D + 8 * v_pos<D>(r, lane % kVChunks)) * S, st + kSBytes + piece * kPiece, false);
      }
    };

    float m = -kInf, l = 0.0f;
    f32x16 acc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = f32x16{};

#pragma unroll
    for (int pre = 0; pre < kPvStages - 1; ++pre)
      if (pre < nblocks) issue(pre);

    for (int64_t blk = 0; blk < nblocks; ++blk) {
      const int64_t c0 = blk * kPvBlock;
      // this wave's loads of block blk have landed (at most the later
      // blocks' are outstanding); after the barrier every wave's have, and
      // every wave is done with the stage that the next issue refills
      if (blk + kPvStages - 2 < nblocks && kPvStages > 2) {
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kLoads * (kPvStages - 2)));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
      }
      lds_barrier();
      if (blk + kPvStages - 1 < nblocks) issue(blk + kPvStages - 1);

      const char* st = ring + (int)(blk % kPvStages) * kStage;
      const char* vs = st + kSBytes;
      const int r_lds = wid * 32 + (lane & 31);

      // this lane's 32 scores, columns c0 + 32 h .. + 31 of its row; lanes
      // are masked element by element only when some row of the wave ends
      // inside its half block (or for arbitrary keep masks)
      Pack<DT, 8> sp[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(st + r_lds * 128 + s_pos(r_lds, 4 * h + k) * 16);
        sp[k].w[0] = w.x;
        sp[k].w[1] = w.y;
        sp[k].w[2] = w.z;
        sp[k].w[3] = w.w;
      }
      float x[32];
      if (KEEP || __ballot(prefix < c0 + 32 * h + 32) != 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t j0 = c0 + 32 * h + 8 * k;
          const int64_t left = prefix - j0;
          const int rem = left <= 0 ? 0 : (left >= 8 ? 8 : (int)left);
          uint64_t kb = ~0ull;
          if constexpr (KEEP) {
            if (rem > 0) kb = load_keep<8>(a.mask.keep + row * cols + j0);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool ok = e < rem && (!KEEP || keep_lane(kb, e));
            x[8 * k + e] = ok ? sp[k].get(e) : -kInf;
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e) x[8 * k + e] = sp[k].get(e);
      }

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
      // forming -inf - -inf. A wave holding a row with a large reference
      // subtracts it explicitly (rare: scores beyond 2^15).
      const float mu = m == -kInf ? 0.0f : m;
      float c = -mu * kLog2e;
      if (__ballot(!(__builtin_fabsf(mu) < kBiasedMax)) != 0) {
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] -= mu;
        c = 0.0f;
      }

      // per k-step t: the weights of this lane's scores 8t .. 8t+7 (columns
      // c0 + 32 h + 8t ..) as 16-bit hi + lo pairs, then o^T += V^T p^T on
      // the matrix cores. V's operand is read transposed from the same
      // columns of the V block: within each 16-lane group, lane 4e + q points
      // at 4 values of V row (32 h + 8t + e) and the read hands lane i the 4
      // consecutive rows of column i; a second read takes the next 4 rows.
      const int i16 = lane & 15, ee = i16 >> 2, qq = i16 & 3, dh = (lane >> 4) & 1;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float q0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[8 * t + e], kLog2e, c));
          const float q1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[8 * t + e + 1], kLog2e, c));
          l += q0 + q1;
          split_pair<DT>(q0 * kWeightScale<DT>, q1 * kWeightScale<DT>, hw[e / 2], lw[e / 2]);
        }
        const u32x4 phi{hw[0], hw[1], hw[2], hw[3]};
        const u32x4 plo{lw[0], lw[1], lw[2], lw[3]};
        const int vr0 = 32 * h + 8 * t + ee;
        const int vr1 = vr0 + 4;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const int d0 = 32 * i + 16 * dh + 4 * qq;
          const char* a0 = vs + vr0 * D * S + v_pos<D>(vr0, d0 / 8) * 16 + (d0 % 8) * S;
          const char* a1 = vs + vr1 * D * S + v_pos<D>(vr1, d0 / 8) * 16 + (d0 % 8) * S;
          const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a0);
          const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a1);
          const i16x8 av = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[i] = mfma<DT>(av, phi, acc[i]);
          acc[i] = mfma<DT>(av, plo, acc[i]);
        }
      }
    }
    lds_barrier();  // every wave is done with the ring before the next tile's loads

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
