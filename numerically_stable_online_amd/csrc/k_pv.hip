// k_pv.hip — softmax-weighted value sums on the matrix cores:
//   out[r, :] = sum_j softmax(s[r])_j v[g, j, :],   g = r / rows_per_group,
// computed online over column blocks. The row keeps its running maximum m,
// the running sum l and the unnormalized numerator o; when a block moves the
// maximum, l and o take the same factor exp(m - m') and the block's terms
// are added relative to m' ("Online stable softmax", sections on the
// weighted-value numerator and the reference summary; "Softmax numerics
// architecture", tiled attention: the output is o / l at the end).
//
// A tile is 128 rows of one group; a workgroup of four waves takes one tile
// at a time (each wave 32 of its rows), and the workgroups stay resident,
// taking tiles round by round. Blocks of 64 columns of the scores and of V travel HBM -> LDS by
// direct loads into a ring (scores three stages deep, issued two blocks
// ahead; V two stages, one block ahead); score chunks wholly past a row's
// valid prefix are loaded from a -inf chunk instead of from HBM. Per block:
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
//    accumulation; the value vectors enter exactly;
//  * a wave whose rows all end before the block skips its work.
// The column order inside a block is permuted consistently between the
// score operand and the value operand (the contraction does not depend on
// it), so every lane's scores are 64 contiguous bytes of its row.
#include "smx_device.hpp"

namespace smx {
namespace {

constexpr int kPvRows = 128;    // rows per workgroup (four waves of 32)
constexpr int kPvBlock = 64;    // columns per block (four matrix-core k-steps of 16)
constexpr int kSStages = 3;     // score blocks in LDS: one read, two loading
constexpr int kVStages = 2;     // V blocks in LDS: one read, one loading
constexpr int kPiece = 64 * 16; // bytes one wave's direct global->LDS load moves
constexpr int kSBytes = kPvRows * kPvBlock * 2;        // one score block: 128 rows of 128 bytes
constexpr int kSPieces = kSBytes / kPiece / kWaves;    // direct score loads per wave per block (4)

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
constexpr float kLog2WeightScale = DT == kF16 ? 12.0f : 0.0f;
// below this reference magnitude a row's weights are 2^(x log2e + c) with
// one rounded constant c per row; once a row of a wave reaches it, the wave
// subtracts the reference explicitly for the rest of its tile
constexpr float kBiasedMax = 32768.0f;

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding and leaves the other counters alone (vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 at its maximum, lgkmcnt 11:8 at its maximum)
constexpr int vmcnt_at_most(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (7 << 4) | (0xF << 8); }

// One wave's direct 16-byte-per-lane global -> LDS load: lane i's 16 bytes
// land at LDS byte address lds + 16 i (lds must be the same in every lane;
// it travels in m0, and the load may not read m0 in the instruction right
// after the write, hence the wait state). Issued as instructions the
// compiler does not track, so that it inserts no wait for them before later
// LDS accesses (which would empty the pipeline); the kernel waits for these
// loads itself (vmcnt) before its barriers. m0 is not declared clobbered
// (the compiler reserves it and ignores such a declaration): nothing the
// compiler emits in this file uses m0, whose only writers are these two
// statements.
__device__ __forceinline__ void dma16_global(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(g), "s"(lds) : "memory");
}
// the same from a wave-uniform base plus a 32-bit per-lane offset
__device__ __forceinline__ void dma16_offset(uint32_t off, const void* base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "s"(lds) : "memory");
}

// 16 bytes of -inf in each 16-bit format (fp16, bf16): the source of every
// score chunk that lies wholly past its row's valid prefix
__device__ __attribute__((aligned(16))) const uint16_t kNegInfChunk[2][8] = {
    {0xFC00, 0xFC00, 0xFC00, 0xFC00, 0xFC00, 0xFC00, 0xFC00, 0xFC00},
    {0xFF80, 0xFF80, 0xFF80, 0xFF80, 0xFF80, 0xFF80, 0xFF80, 0xFF80}};

// A workgroup barrier that orders LDS accesses only: the wave's LDS stores
// complete before it, but no global load is waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS layout: a score block holds 128 rows of 128 bytes (eight 16-byte
// chunks of 8 scores), a V block 64 rows of D values as they are in memory.
// Chunks sit at a position XOR-swizzled by the row so that every read below
// is free of bank conflicts, whether the LDS serves 128 or 256 bytes a
// clock: the score reads take one chunk of 16 consecutive rows (position
// and the row's parity, which selects the 128-byte half, must differ for
// every row); the transposing V reads take two adjacent chunks of 4
// consecutive rows for each of two column groups.
__device__ __forceinline__ int s_pos(int row, int chunk) { return chunk ^ (row & 7) ^ ((row >> 3) & 1); }
template <int D>
__device__ __forceinline__ int v_pos(int row, int chunk) {
  if constexpr (D == 128) {
    return chunk ^ ((row & 1) ? 10 : 0) ^ (((row >> 1) & 1) ? 4 : 0);
  } else if constexpr (D == 64) {
    return chunk ^ (2 * (row & 3));
  } else {
    return chunk ^ (2 * ((row >> 1) & 1));
  }
}

// The value of lane i ^ 32 beside lane i's own: v_permlane32_swap exchanges
// the upper 32 lanes of its first operand with the lower 32 of its second,
// so with both holding v, the first becomes (v[0..31], v[0..31]) and the
// second (v[32..63], v[32..63]); one VALU instruction instead of an LDS
// permute. The wait states cover a VALU write of either operand just before.
__device__ __forceinline__ void halves(float v, float& lo_half, float& hi_half) {
  lo_half = v;
  hi_half = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo_half), "+v"(hi_half));
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
__device__ __forceinline__ int block_max_int(int v, int* slot) {
  for (int off = 32; off > 0; off >>= 1) {
    const int o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = slot[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = slot[i] > r ? slot[i] : r;
  __syncthreads();
  return r;
}

template <int DT, int D, bool KEEP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_pv(PvArgs a) {
  constexpr int S = 2;
  constexpr int NT = D / 32;                       // 32-wide accumulator tiles along d
  constexpr int kVBytes = kPvBlock * D * S;        // one V block
  constexpr int kVPieces = kVBytes / kPiece;       // 16, 8 or 4
  constexpr int kVPerWave = kVPieces / kWaves;     // 4, 2 or 1
  constexpr int kVRowsPerPiece = kPiece / (D * S);
  constexpr int kVChunks = D / 8;
  constexpr int kSRing = kSStages * kSBytes;
  __shared__ __attribute__((aligned(1024))) char ring[kSRing + kVStages * kVBytes];
  int* const slot = reinterpret_cast<int*>(ring);  // between tiles only, when no load is in flight

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
  const void* const ninf = kNegInfChunk[DT == kBF16 ? 1 : 0];
  const bool out16 = ((uintptr_t)a.out & 15) == 0;  // rows of 64 to 256 bytes then start 16-byte aligned

  // Lane constants. This lane's row is r_lds of the tile; of each block it
  // takes chunks 4h .. 4h+3 (columns 32h .. 32h+31).
  const int r_lds = wid * 32 + (lane & 31);
  int s_off[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) s_off[k] = r_lds * 128 + 16 * s_pos(r_lds, 4 * h + k);
  // Its direct score loads: piece q of wave w is LDS rows 32w + 8q .. + 7;
  // lane i fills row 32w + 8q + i/8 at position i % 8, which holds chunk
  // (i % 8) ^ (i / 8) ^ (q & 1).
  int cc[kSPieces];
#pragma unroll
  for (int q = 0; q < kSPieces; ++q) cc[q] = 8 * ((lane & 7) ^ (lane >> 3) ^ (q & 1));
  // Its direct V loads: piece q of wave w is 1 KiB of consecutive V rows
  const int vrow_in_piece = lane / kVChunks;
  const uint32_t voff = (uint32_t)((wid * kVPerWave * kVRowsPerPiece + vrow_in_piece) * D * S +
                                   16 * v_pos<D>(vrow_in_piece, lane % kVChunks));
  // Its transposing V reads (k-step 0; k-step t adds 8 t rows): within each
  // 16-lane group, lane 4e + q points at V row 32h + e, columns d0 .. d0+3
  const int i16 = lane & 15, ee = i16 >> 2, qq = i16 & 3, dh = (lane >> 4) & 1;
  int tr_off[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int vr = 32 * h + ee;
    const int d0 = 32 * i + 16 * dh + 4 * qq;
    tr_off[i] = vr * D * S + v_pos<D>(vr, d0 / 8) * 16 + (d0 % 8) * S;
  }

  // The workgroups stay resident and take tiles round by round. XCD-aware
  // order: the eight XCDs take workgroups round-robin, so each XCD is given
  // a contiguous eighth of the logical tiles (whole groups, which share V,
  // stay in its L2); within a group the longest tiles (the last rows of a
  // causal group) come first, and the XCD's workgroups walk its tiles in a
  // snake, reversing direction every round, so that a workgroup that took a
  // long tile of a group takes a short one next (causal tiles of one group
  // differ in length by up to 16 times).
  const bool xcd = total % 8 == 0 && gridDim.x % 8 == 0;
  const int64_t per = gridDim.x / 8;  // workgroups per XCD (when xcd)
  const int64_t u = blockIdx.x / 8;
  const int64_t rounds = xcd ? (per_xcd + per - 1) / per : (total - blockIdx.x + gridDim.x - 1) / gridDim.x;
  for (int64_t k = 0; k < rounds; ++k) {
    int64_t lb = blockIdx.x + k * gridDim.x;
    if (xcd) {
      const int64_t p = k * per + ((k & 1) ? per - 1 - u : u);
      if (p >= per_xcd) continue;  // uniform across the workgroup
      lb = (blockIdx.x % 8) * per_xcd + p;
    }
    const int64_t g = lb / tiles_per_group;
    const int64_t tile = tiles_per_group - 1 - lb % tiles_per_group;
    const int64_t row0 = g * rpg + tile * kPvRows;
    const int64_t row_end = (row0 + kPvRows < (g + 1) * rpg) ? row0 + kPvRows : (g + 1) * rpg;
    const int64_t row = row0 + r_lds;
    const bool row_ok = row < row_end;
    const int prefix = row_ok ? (int)valid_prefix(a.mask, row, cols) : 0;
    const int extent = block_max_int(prefix, slot);
    const int nb = (extent + kPvBlock - 1) / kPvBlock;
    const char* const vg = a.v + g * cols * D * S;

    // this lane's score loads: the chunk at c0 + cc[q] of its piece rows, or
    // the -inf chunk once that chunk lies past the row's valid prefix (so
    // masked scores cost no HBM traffic and arrive masked)
    const char* sptr[kSPieces];
    int slim[kSPieces];
#pragma unroll
    for (int q = 0; q < kSPieces; ++q) {
      const int64_t r = row0 + wid * 32 + 8 * q + (lane >> 3);
      const bool ok = r < row_end;
      sptr[q] = a.s + ((ok ? r : row0) * cols + cc[q]) * S;
      slim[q] = ok ? (int)valid_prefix(a.mask, r, cols) - cc[q] : -1;
    }
    auto issue_s = [&](int blk) {
      const int c0 = blk * kPvBlock;
      const uint32_t st = ring_lds + (uint32_t)((blk % kSStages) * kSBytes + wid * kSPieces * kPiece);
#pragma unroll
      for (int q = 0; q < kSPieces; ++q) {
        const void* src = c0 < slim[q] ? (const void*)(sptr[q] + (int64_t)c0 * S) : ninf;
        dma16_global(src, st + q * kPiece);
      }
    };
    auto issue_v = [&](int blk) {
      const int c0 = blk * kPvBlock;
      const uint32_t st = ring_lds + (uint32_t)(kSRing + (blk & 1) * kVBytes + wid * kVPerWave * kPiece);
      const char* base = vg + (int64_t)c0 * D * S;
      if (c0 + kPvBlock <= cols) {
#pragma unroll
        for (int q = 0; q < kVPerWave; ++q) dma16_offset(voff + q * kPiece, base, st + q * kPiece);
      } else {
        // the last block of rows whose length is not a multiple of the
        // block: V rows past the end re-read the last row (weight 0)
#pragma unroll
        for (int q = 0; q < kVPerWave; ++q) {
          const int r = (wid * kVPerWave + q) * kVRowsPerPiece + vrow_in_piece;
          const int rr = c0 + r < cols ? r : (int)(cols - 1 - c0);
          dma16_offset((uint32_t)(rr * D * S + 16 * v_pos<D>(r, lane % kVChunks)), base, st + q * kPiece);
        }
      }
    };

    float m = -kInf, l = 0.0f;  // the running maximum (the reference) and sum
    uint64_t wide_rows = 0;  // lanes whose reference reached 2^15 this tile (the wave's form)
    f32x16 acc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = f32x16{};

    // this lane's 32 scores of block blk: x[8k + e] is column c0 + 32h + 8k
    // + e. Chunks past the valid prefix arrived as -inf; the chunk a row's
    // prefix ends inside (and keep masks) are masked element by element.
    auto load_scores = [&](int blk, float (&x)[32]) {
      const char* st = ring + (blk % kSStages) * kSBytes;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(st + s_off[k]);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * k + 2 * e] = dec<DT>(ws[e] & 0xFFFFu);
          x[8 * k + 2 * e + 1] = dec<DT>(ws[e] >> 16);
        }
      }
      const int lim = prefix - (blk * kPvBlock + 32 * h);  // valid lanes: i < lim
      if constexpr (KEEP) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint64_t kb =
              8 * k < lim ? load_keep<8>(a.mask.keep + row * cols + blk * kPvBlock + 32 * h + 8 * k) : 0;
#pragma unroll
          for (int e = 0; e < 8; ++e) x[8 * k + e] = (8 * k + e < lim && keep_lane(kb, e)) ? x[8 * k + e] : -kInf;
        }
      } else if (__ballot(lim > 0 && lim < 32 && (lim & 7) != 0) != 0) {
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = i < lim ? x[i] : -kInf;
      }
    };

    // the weights of k-step t (x[8t .. 8t+7]) as 16-bit hi + lo pairs
    auto weights = [&](const float (&x)[32], int t, float c, u32x4& wh, u32x4& wl) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float q0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[8 * t + e], kLog2e, c));
        const float q1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[8 * t + e + 1], kLog2e, c));
        l += q0 + q1;
        split_pair<DT>(q0, q1, hw[e / 2], lw[e / 2]);
      }
      wh = u32x4{hw[0], hw[1], hw[2], hw[3]};
      wl = u32x4{lw[0], lw[1], lw[2], lw[3]};
    };

    // o^T += V^T p^T for k-step t of the V block in stage vst: V's operand
    // is read transposed (each 16-lane group's read hands lane i rows
    // k .. k+3 of column i; a second read takes rows k+4 .. k+7)
    auto products = [&](int vst, int t, const u32x4& wh, const u32x4& wl) {
      const char* vs = ring + kSRing + vst * kVBytes + t * 8 * D * S;
      i16x8 av[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const i16x4 lo4 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vs + tr_off[i]));
        const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vs + tr_off[i] + 4 * D * S));
        av[i] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[i] = mfma<DT>(av[i], wh, acc[i]);
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[i] = mfma<DT>(av[i], wl, acc[i]);
    };

    // Loads: the scores of block blk are issued two blocks ahead, V one
    // block ahead; at the top of block blk its scores and V have landed.
    if (nb > 0) {
      issue_s(0);
      issue_v(0);
      if (nb > 1) issue_s(1);
    }
    for (int blk = 0; blk < nb; ++blk) {
      if (blk + 1 < nb) {
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kSPieces));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
      }
      lds_barrier();
      if (blk + 1 < nb) issue_v(blk + 1);
      if (blk + 2 < nb) issue_s(blk + 2);

      // a block past every row of the wave adds nothing (its weights are
      // all 0): the wave keeps its loads and barriers but skips the work
      if (__ballot(prefix > blk * kPvBlock) == 0) continue;

      float x[32];
      load_scores(blk, x);
      // The reference moves to the block's maximum when that exceeds it by
      // more than the slack (or is NaN / +inf, which poisons the row, or
      // the row was empty so far).
      float bm = -kInf;
#pragma unroll
      for (int i = 0; i < 32; ++i) bm = vmax(bm, x[i]);
      {
        float a0, a1;
        halves(bm, a0, a1);  // the two halves of the row
        bm = vmax(a0, a1);
      }
      const float m_new = (bm <= m + kSlack<DT>) ? m : vmax(m, bm);
      // exp(x - m) as 2^(x log2e + c), c = -m log2e plus the log2 of the
      // fp16 weight scale, rounded once (the folded form). A row with no
      // finite reference uses 0, so masked lanes (-inf) give 0 without
      // forming -inf - -inf. Once a row of the wave has a large reference
      // (|m| >= 2^15, rare) the wave subtracts the reference explicitly
      // instead, for the rest of the tile (the explicit form): x - m is exact
      // wherever the weight is not negligible, so the constant is then
      // exactly the scale's log2 minus m log2e.
      //
      // The state (l and the accumulators) carries the constant its weights
      // were formed with. When the reference moves, the state takes 2^(c' -
      // c), the difference of the two constants as they were formed: in the
      // folded form that is the difference of the two rounded constants, so
      // earlier and later terms keep one common factor, which cancels in o /
      // l. When the wave turns to the explicit form, the state first takes
      // the rounding error of its folded constant, 2^(exact - rounded), the
      // exact constant held as an unevaluated sum (the product split by a
      // fused multiply-add, the difference by a two-sum). Either factor is
      // exactly 1 when nothing changes; an empty state holds zeros and is
      // left alone.
      const float mu = __builtin_fabsf(m_new) < kInf ? m_new : 0.0f;
      const bool was_wide = wide_rows != 0;
      wide_rows |= __ballot(!(__builtin_fabsf(mu) < kBiasedMax));
      const bool wide = wide_rows != 0;
      float c = kLog2WeightScale<DT> - mu * kLog2e;
      if (wide) {
        if (!was_wide) {
          const float mo = __builtin_fabsf(m) < kInf ? m : 0.0f;
          const float mp = mo * kLog2e;
          const float e = __builtin_fmaf(mo, kLog2e, -mp);  // mo log2e = mp + e
          const float h = kLog2WeightScale<DT> - mp;         // the folded constant
          const float bb = h - kLog2WeightScale<DT>;         // two-sum of the scale and -mp
          const float lo = ((kLog2WeightScale<DT> - (h - bb)) + (-mp - bb)) - e;
          const float alpha = m > -kInf ? __builtin_amdgcn_exp2f(lo) : 1.0f;  // exact = h + lo
          l *= alpha;
#pragma unroll
          for (int i = 0; i < NT; ++i) acc[i] *= alpha;
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] -= mu;
        c = kLog2WeightScale<DT>;
      }
      const bool moved = m_new != m && m > -kInf;
      if (__ballot(moved) != 0) {
        const float mo = __builtin_fabsf(m) < kInf ? m : 0.0f;
        const float d = wide ? (mo - mu) * kLog2e : c - (kLog2WeightScale<DT> - mo * kLog2e);
        const float alpha = moved ? __builtin_amdgcn_exp2f(d) : 1.0f;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[i] *= alpha;
      }
      m = m_new;

      // the products of k-step t run while the weights of k-step t + 1 form
      const int vst = blk & 1;
      u32x4 wh[2], wl[2];
      weights(x, 0, c, wh[0], wl[0]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < 3) weights(x, t + 1, c, wh[(t + 1) & 1], wl[(t + 1) & 1]);
        products(vst, t, wh[t & 1], wl[t & 1]);
      }
    }
    lds_barrier();  // every wave is done with the ring before the next tile's loads

    // o / l; the two halves of the row hold partial sums of l
    l += __shfl_xor(l, 32);
    const bool poisoned = !(m < kInf);
    const bool empty = m == -kInf;
    const float inv = 1.0f / l;  // l holds the scaled weights too
    char* orow = a.out + (row_ok ? row : 0) * D * S;
    // accumulator values 4q .. 4q+3 of tile i are d = 32 i + 8 q + 4 h + 0..3
    auto pack = [&](int i, int q, uint32_t& w0, uint32_t& w1) {
      if (poisoned) {
        w0 = w1 = Fmt<DT>::kNaN | (Fmt<DT>::kNaN << 16);
      } else if (empty) {
        w0 = w1 = 0u;
      } else {
        w0 = enc2<DT>(acc[i][4 * q + 0] * inv, acc[i][4 * q + 1] * inv);
        w1 = enc2<DT>(acc[i][4 * q + 2] * inv, acc[i][4 * q + 3] * inv);
      }
    };
    if (out16) {
      // The two lanes of a row trade halves (v_permlane32_swap, as in
      // halves() above: the lane of the first half takes both halves of the
      // even 8-value groups, the other lane those of the odd ones), then the
      // wave stages its 32 output rows in its own slices of score stages 1
      // and 2 (free at a tile's end, every score block consumed; stage 0
      // holds the workgroup's reduction slot), chunks XOR-swizzled by the row
      // so that neither side conflicts, and writes them back as contiguous
      // 1 KiB pieces. Against 8-byte stores straight from the accumulators:
      // 392.6 -> 382.2 us on the causal attention shape with 128-wide values
      // (one process, outputs bitwise equal).
      constexpr int CH = D / 8;    // 16-byte chunks per output row
      constexpr int RPI = 64 / CH; // rows per store instruction
      char* const stg = ring + wid * (32 * 128);
      auto slot16 = [&](int r, int chunk) {
        const int L = r * D * S;
        return stg + (1 + L / 4096) * kSBytes + (L % 4096) + 16 * (chunk ^ (r % CH));
      };
#pragma unroll
      for (int i = 0; i < NT; ++i) {
#pragma unroll
        for (int qe = 0; qe < 4; qe += 2) {
          uint32_t x0, x1, y0, y1;
          pack(i, qe, x0, x1);
          pack(i, qe + 1, y0, y1);
          asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3"
                       : "+v"(x0), "+v"(y0), "+v"(x1), "+v"(y1));
          const int q = h ? qe + 1 : qe;
          *reinterpret_cast<u32x4*>(slot16(lane & 31, 4 * i + q)) = u32x4{x0, x1, y0, y1};
        }
      }
      const int64_t wrow0 = row0 + wid * 32;
#pragma unroll
      for (int k = 0; k < 32 / RPI; ++k) {
        const int rr = k * RPI + lane / CH, cc = lane % CH;
        const u32x4 val = *reinterpret_cast<const u32x4*>(slot16(rr, cc));
        if (wrow0 + rr < row_end) *reinterpret_cast<u32x4*>(a.out + (wrow0 + rr) * D * S + cc * 16) = val;
      }
    } else if (row_ok) {  // an output only 8-byte aligned
#pragma unroll
      for (int i = 0; i < NT; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t w0, w1;
          pack(i, q, w0, w1);
          *reinterpret_cast<uint2*>(orow + (32 * i + 8 * q + 4 * h) * S) = make_uint2(w0, w1);
        }
      }
    }
  }
}

constexpr int kMaxDevices = 64;

// As many workgroups as the device holds at once (the occupancy the runtime
// reports for the kernel, times the CU count), at most one per tile.
template <int DT, int D, bool KEEP>
hipError_t launch_keep(const PvArgs& a, int64_t tiles, hipStream_t s) {
  static int resident[kMaxDevices];
  auto kernel = k_pv<DT, D, KEEP>;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int res = __atomic_load_n(&resident[dev], __ATOMIC_RELAXED);
  if (res == 0) {
    int occ = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kThreads, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    res = (occ > 0 ? occ : 1) * cus;
    __atomic_store_n(&resident[dev], res, __ATOMIC_RELAXED);
  }
  const unsigned grid = (unsigned)(tiles < res ? tiles : res);
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_d(const PvArgs& a, hipStream_t s) {
  const int64_t tiles = (a.rows / a.rows_per_group) * ((a.rows_per_group + kPvRows - 1) / kPvRows);
  if (a.mask.kind == kMaskKeep) return launch_keep<DT, D, true>(a, tiles, s);
  return launch_keep<DT, D, false>(a, tiles, s);
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
