// gemm.hip -- persistent grouped GEMM over expert segments on CDNA4 matrix cores.
//
// For each expert e and permuted row p in [offsets[e], offsets[e+1]):
//     acc[p, n] = sum_k A[p, k] * B[e, n, k]          (fp32 accumulate)
// followed by one of two epilogues: store acc, or store silu(gate) * up where
// gate and up are B rows n and N/2 + n.  This is the grouped GEMM with equal N
// and K per group (group_gemm_same_nk) and the SiLU(fc1_1) * fc1_2 step of the
// LlamaFactory PR #10481 write-up, section 1; the grouped_mm expert backend of
// "트랜스포머에서 전문가 혼합 (MoEs)".  Only rows below offsets[E] get tiles, and
// rows [offsets[E], M_rows) of C are written as zeros (the transformers PR
// #45621 write-up: section 2 excludes sentinel rows from the work, section 3
// traces a NaN to sentinel outputs left unwritten).
//
// Design (gfx950):
//  * Persistent grid of (#CU x occupancy) workgroups.  Every workgroup reads
//    offsets from device memory and builds the per-expert m-tile prefix in
//    LDS, so the launch needs no host knowledge of the expert loads.
//  * Tile order: expert-major, then n-tile, then m-tile fastest, so the few
//    m-tiles sharing one weight panel run back to back.  The tile index is
//    remapped so that consecutive tiles go to workgroups of the same XCD
//    (workgroup w is dispatched to XCD w % 8): tiles that share a weight
//    panel and an activation panel meet in that XCD's L2.
//  * K is walked in 128-byte slices (64 bf16 / 32 f32 / 128 e4m3 per row).
//    bf16 and e4m3 tiles fill a ring of ST LDS stages with direct global->LDS
//    loads, ST-1 slices in flight while one feeds the MFMAs; f32 tiles (the
//    reference-precision configuration) double-buffer through registers.  Each
//    LDS row is 128 bytes = eight 16-byte chunks stored XOR-swizzled, so that
//    the 16 rows read by one MFMA operand fetch hit distinct banks.
//  * Modes: A read directly or gathered through a row map (token rows read
//    through the permutation); K-grouped (weight gradients: each expert's own K
//    range, every expert's full output); decode-size tiles (16 rows, one or two
//    waves, deep rings) for launches with at most 8 rows per expert.
//  * MFMA operand roles are swapped: weight rows are the 16-row src0 operand
//    and activation rows the src1 operand, so each lane's results are output
//    columns of one activation row.  Inside each wave the weight rows are
//    placed in LDS in an order that makes every lane's columns contiguous
//    (4 x subtiles), which turns the epilogue into 16-byte row stores.
//  * bf16: v_mfma_f32_16x16x32_bf16; f32: v_mfma_f32_16x16x4_f32; e4m3:
//    v_mfma_f32_16x16x128_f8f6f4 with one 128-deep MFMA per 128x128 weight
//    block, whose fp32 result is scaled by (activation scale x weight block
//    scale) and added to the accumulator.
//  * e4m3 output (h of the fp8 layer): the 128 columns of a tile form one
//    quantisation group; its |max| is reduced across lanes and waves, then
//    scale = amax / 448 and codes = RNE(value / scale).

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace moe {

enum class AbType { F32, BF16, FP8 };
enum class CType { F32, BF16, FP8 };

template <AbType T> struct AbTraits;
template <> struct AbTraits<AbType::BF16> {
  static constexpr int kEsize = 2, kSteps = 2, kChunksPerLane = 1;
};
template <> struct AbTraits<AbType::F32> {
  static constexpr int kEsize = 4, kSteps = 2, kChunksPerLane = 1;
};
template <> struct AbTraits<AbType::FP8> {
  static constexpr int kEsize = 1, kSteps = 1, kChunksPerLane = 2;
};

struct GemmArgs {
  const uint8_t* A;
  const float* a_scales;
  const uint8_t* B;
  const float* b_scales;
  const int* offsets;
  int E;
  int M_rows;
  int N;        // B rows per expert
  int K;        // elements
  uint8_t* C;
  float* c_scales;
  int N_out;    // columns of C
  int n_tiles;  // ceil(N_out / BN_out)
  // K-grouped mode (weight gradients), when koff is set: C[e] [M_rows, N_out] =
  // A_e B_e^T for e < E, where A_e [M_rows, kpad_e] sits at element
  // M_rows * koff[e] of A and B_e [N, kpad_e] at element N * koff[e] of B
  // (expert-major blocks, rows of kpad_e = koff[e+1] - koff[e] elements, a
  // multiple of 64)
  const int* koff;
  int lda;      // A row stride (elements); the M-grouped mode uses K
  int ldb;      // B row stride (elements); the M-grouped mode uses K
  // Gathered A (M-grouped mode), when a_rows is set: row p of the product reads
  // A row a_rows[p] / a_div of the a_total rows of A (token rows read through the
  // permutation, so no permuted copy is made); a_scales is then [K/128, a_total].
  // Without it, A has M_rows rows and row p is A row p (a_total = M_rows).
  const int* a_rows;
  int a_div;
  int a_total;
  // fp8 with a row map and a_scales_by_row set: a_scales is [K/128, M_rows], the scales
  // already stored at the product rows (consecutive for a tile's rows).
  int a_scales_by_row;
  // SiLU*up with bf16 operands and C (M-grouped mode): when pre_out is set, also
  // store the f32 pre-activations, gate at column c and up at column N_out + c of
  // pre_out [M_rows, 2 N_out] (rows below offsets[E]; the layer's backward reads them).
  float* pre_out;
};

#define MOE_INLINE __attribute__((always_inline))

constexpr int kSliceBytes = 128;  // bytes of K per LDS row
constexpr int kMaxExperts = 1024;

// Tile shapes (BM, BNB, WM, WN, PF, ST): rows x weight rows per tile, waves along
// M and N, loader (PF = 0: direct global->LDS loads; 1 or 2: slices prefetched
// through registers) and LDS stages.  Overridable at compile time.
#ifndef MOE_TILE_BF16_SILU
#define MOE_TILE_BF16_SILU 192, 192, 4, 2, 0, 3
#endif
#ifndef MOE_TILE_BF16_NONE
#define MOE_TILE_BF16_NONE 192, 192, 4, 2, 0, 3
#endif
#ifndef MOE_TILE_FP8_SILU
#define MOE_TILE_FP8_SILU 128, 256, 2, 4, 0, 3
#endif
// Decode-size bf16 launches (few routed rows per expert): one-wave tiles of 16 rows
// by 16 output columns (SiLU*up: 16 gate + 16 up weight rows) or 32 (no epilogue),
// and an 8-stage LDS ring.  The weights stream through many small tiles with more
// bytes in flight per CU, where 192-row tiles would leave most CUs idle and most MFMA
// rows empty.  With at most 2 rows per expert the no-epilogue tiles narrow to 16
// columns as well (twice the tiles; at more rows the wider tile is as fast).
#ifndef MOE_TILE_BF16_SILU_DEC
#define MOE_TILE_BF16_SILU_DEC 16, 32, 1, 1, 0, 8
#endif
#ifndef MOE_TILE_BF16_NONE_DEC
#define MOE_TILE_BF16_NONE_DEC 16, 32, 1, 1, 0, 8
#endif
#ifndef MOE_TILE_BF16_NONE_DEC_NARROW
#define MOE_TILE_BF16_NONE_DEC_NARROW 16, 16, 1, 1, 0, 8
#endif
// Decode-size fp8 tiles: 16 rows, two waves (one loads the tile's activation scales,
// the other the weight block scales).  Gate/up: 16 gate + 16 up weight rows per wave,
// 32 output columns (f32 or bf16 h: a 128-column e4m3 group spans four such tiles, so
// h is quantised in a second pass); down: 64 output columns.  fp8 output (the fused
// quantising epilogue) keeps the 128-column tiles.
#ifndef MOE_TILE_FP8_SILU_DEC
#define MOE_TILE_FP8_SILU_DEC 16, 64, 1, 2, 0, 6
#endif
#ifndef MOE_TILE_FP8_NONE_DEC
#define MOE_TILE_FP8_NONE_DEC 16, 64, 1, 2, 0, 6
#endif
// bf16 launches of at most this many rows per expert (M_rows <= this * E) use them
#ifndef MOE_DECODE_ROWS_PER_EXPERT
#define MOE_DECODE_ROWS_PER_EXPERT 8
#endif
// bf16 launches of more than that and at most MOE_MID_ROWS_PER_EXPERT rows per expert take
// mid-size tiles: 32 rows (an expert's rows usually fit one m-tile, so its weights stream
// once) by 64 weight rows.  SiLU*up: four waves of 16x32 and six LDS stages; down: two waves
// of 16x64 and four stages (0: no mid tier)
#ifndef MOE_MID_ROWS_PER_EXPERT
#define MOE_MID_ROWS_PER_EXPERT 32
#endif
#ifndef MOE_TILE_BF16_SILU_MID
#define MOE_TILE_BF16_SILU_MID 32, 64, 2, 2, 0, 6
#endif
#ifndef MOE_TILE_BF16_NONE_MID
#define MOE_TILE_BF16_NONE_MID 32, 64, 2, 1, 0, 4
#endif
// B-as-[K, N] launches (the backward's data-gradient products) of at most this many rows
// per expert take 128x256 tiles (eight 64x64 waves, three stages)
#ifndef MOE_BT_SHORT_ROWS_PER_EXPERT
#define MOE_BT_SHORT_ROWS_PER_EXPERT 384
#endif
#ifndef MOE_TILE_BF16_BT_SHORT
#define MOE_TILE_BF16_BT_SHORT 128, 256, 2, 4, 0, 3
#endif
// m-tiles per block of an expert's tile order (see the tile decode)
#ifndef MOE_M_BLOCK
#define MOE_M_BLOCK 4
#endif
// fp8 SiLU*up tiles: split each expert's rows evenly over its m-tiles (see the tile decode)
#ifndef MOE_EVEN_SPLIT_FP8
#define MOE_EVEN_SPLIT_FP8 1
#endif
// spread the last, partial round of tiles over all XCDs (see the tile loop)
#ifndef MOE_SPREAD_LAST_ROUND
#define MOE_SPREAD_LAST_ROUND 1
#endif
#ifndef MOE_DECODE_NARROW_ROWS_PER_EXPERT
#define MOE_DECODE_NARROW_ROWS_PER_EXPERT 2
#endif
#ifndef MOE_TILE_FP8_NONE
#define MOE_TILE_FP8_NONE 128, 256, 2, 4, 0, 3
#endif

// Swizzle of the 16-byte chunk index within a 128-byte LDS row: logical chunk c
// of row r is stored at chunk c ^ (r & 7).  The MFMA operand fetch (16 rows at
// one logical chunk per 16 lanes) reads without bank conflicts on gfx950 in
// this layout (measured with SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int swz(int row) { return row & 7; }
// Swizzle of a [K, N] weight tile's k-row (see the kernel's BT mode).  A transposing
// read takes 4 consecutive k-rows, of which rows r and r + 2 start in the same bank
// half (128-byte rows); their swizzles differ by 4, which maps the four chunks a lane
// group reads in one row onto the four chunks the other row leaves free.  Rows r and
// r + 4 share a swizzle, so the second read of a fragment is the first plus 512 bytes.
__device__ __forceinline__ int bt_swz(int row) { return (row & 1) | ((row & 2) << 1); }

// One wave-wide direct global->LDS load: lane i's 16 bytes at base + voff land
// at LDS byte address lds_addr + 16*i (gfx950 global_load_lds_dwordx4; the LDS
// address comes from M0).  The wait for it is explicit (s_waitcnt vmcnt), as
// the compiler does not track this load.  M0 is declared clobbered: the
// compiler sets M0 right before each of its own uses.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(uint32_t lds_addr, const void* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(base)
               : "memory", "m0");
}
// Same with 4 bytes per lane (global_load_lds_dword): lane i's word lands at
// lds_addr + 4*i.
__device__ __forceinline__ void dma4(uint32_t lds_addr, const void* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most n slices of PER direct loads each are outstanding (n <= N; vmcnt
// takes an immediate, so each count has its own instruction).  LGKM: also drain LDS reads.
template <int PER, int N, bool LGKM>
__device__ __forceinline__ void wait_slices(int n) {
  if constexpr (N == 0) {
    if constexpr (LGKM)
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (n >= N) {
      if constexpr (LGKM)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N * PER) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N * PER) : "memory");
    } else {
      wait_slices<PER, N - 1, LGKM>(n);
    }
  }
}

__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  // readfirstlane yields a signed int: widen through uint32_t so the low half is
  // zero-extended (a sign-extended low half would corrupt the upper address bits)
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(lo | (hi << 32));
}

template <AbType AB, CType CT, bool SILU, int BM, int BNB, int WM, int WN, int PF, int ST, bool STG = false>
struct GemmCfg {
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int kWRows = BM / WM;            // activation rows per wave
  static constexpr int kSM = kWRows / 16;           // activation subtiles per wave
  static constexpr int kWNB = BNB / WN;             // weight rows per wave
  static constexpr int kSNB = kWNB / 16;            // weight subtiles per wave
  static constexpr int kSNO = SILU ? kSNB / 2 : kSNB;  // output subtiles per wave
  static constexpr int kBNOut = SILU ? BNB / 2 : BNB;  // output columns per tile
  static constexpr int kWNOut = kBNOut / WN;        // output columns per wave (= 16 kSNO)
  static constexpr int kTileBytes = (BM + BNB) * kSliceBytes;
  static constexpr int kAIters = BM * 8 / kThreads;
  static constexpr int kBIters = BNB * 8 / kThreads;
  static_assert(BM % (16 * WM) == 0 && BNB % (16 * WN) == 0, "tile/wave mismatch");
  static_assert(!SILU || kSNB % 2 == 0, "SiLU needs gate and up subtiles in every wave");
  static_assert((BM * 8) % kThreads == 0 && (BNB * 8) % kThreads == 0, "loader mismatch");
  static_assert(kThreads / 8 % 8 == 0, "loader rows must keep the swizzle phase");
  static_assert(PF >= 0 && PF <= 2, "PF: 0 = direct-to-LDS loads, 1/2 = register prefetch depth");
  static constexpr int kNW = WM * WN;
  static constexpr int kDmaA = BM / 8 / kNW;       // direct loads per wave per slice (8 rows each)
  static constexpr int kDmaB = BNB / 8 / kNW;
  static_assert(PF != 0 || (BM % (8 * kNW) == 0 && BNB % (8 * kNW) == 0),
                "direct loads need whole 8-row groups per wave");
  static_assert(ST == 2 || (PF == 0 && ST >= 3 && ST <= 8), "LDS stages: 2, or 3 to 8 with direct loads");
  static constexpr int kDmaPerSlice = kDmaA + kDmaB;
  static_assert(CT != CType::FP8 || (SILU && kBNOut == 128), "fp8 output needs 128-column tiles");
  // fp8 runs on direct loads only.  Each LDS stage then also holds the slice's
  // block scales: one 256-byte area per wave, filled by one 4-byte-per-lane direct
  // load per wave (waves [0, BM/64): the tile rows' activation scales; the other
  // waves: the weight scales, read from the first of them).
  static_assert(AB != AbType::FP8 || PF == 0, "fp8 needs direct loads");
  static constexpr bool kLdsScales = AB == AbType::FP8;
  static constexpr int kScaleWaves = (BM + 63) / 64;   // a wave loads the scales of 64 rows
  static_assert(!kLdsScales || ((BM % 64 == 0 || BM < 64) && kScaleWaves < kNW && 2 * WN <= 64),
                "fp8 tiles: BM below 64 or a multiple of it, and a spare wave for the weight scales");
  static constexpr int kScaleBytes = kLdsScales ? kNW * 256 : 0;
  static constexpr int kStageBytes = kTileBytes + kScaleBytes;
  static constexpr int kDmaTotal = kDmaPerSlice + (kLdsScales ? 1 : 0);   // loads per wave per slice
  static_assert(PF != 0 || (ST - 2) * kDmaTotal <= 63, "outstanding direct loads must fit vmcnt");
  // Epilogues without SiLU and with bf16 or f32 C go through LDS: each wave writes its
  // kWRows x kWNOut block there (rows padded by 16 bytes, so that the 16 rows a lane group
  // writes at one column start in 16 different bank groups) and stores it back row by row,
  // so that the 64 lanes of a store cover whole 128-byte lines.  Written straight from the
  // MFMA layout, a store's 64 pieces of 16 bytes touch ~3 lines in each of 16 rows, and the
  // L1->L2 requests of the partial lines made the weight-gradient stores run at ~3 TB/s.
  // One MFMA row group (16 rows) of the wave's block at a time, so that the staging area
  // always fits in the K loop's stages.  Used by the backward's launches (STG: the
  // K-grouped weight gradients and the B-as-[K, N] products), whose wide outputs gain
  // (gradients bit-identical; gpt-oss-20b backward -4% with bf16 and -12% with f32
  // gradients, DeepSeek-V3 fp8 backward -6%); the forward's GEMMs measured up to 2.7%
  // slower staged and store directly.
  static constexpr bool kStagedOut = STG && !SILU && CT != CType::FP8 && AB != AbType::FP8;
  static constexpr int kOutEsize = CT == CType::F32 ? 4 : 2;
  static constexpr int kStgRowBytes = kWNOut * kOutEsize + 16;
  static constexpr int kStgWaveBytes = 16 * kStgRowBytes;
  static constexpr int kStgChunksPerRow = kWNOut * kOutEsize / 16;
  static_assert(!kStagedOut || (kWNOut * kOutEsize) % 16 == 0, "staged rows are whole 16-byte chunks");
  static_assert(!kStagedOut || kNW * kStgWaveBytes <= ST * kStageBytes, "staging fits in the stages");
};

// Output column (within the wave's slab) held by MFMA row ii of subtile s.
template <int SN>
__device__ __forceinline__ int slab_col(int s, int ii) {
  return 4 * SN * (ii >> 2) + 4 * s + (ii & 3);
}

// BT: B is stored [E][K][N] (row stride ldb = N elements, N contiguous) instead of
// [E][N][K].  Its LDS tile then holds BNB/64 blocks of 64 columns, each 64 k-rows of
// 128 bytes (16-byte chunk c of k-row r at chunk c ^ bt_swz(r)), filled by the same
// 1 KB direct loads (one load: 8 k-rows of one block), and the MFMA weight fragments
// are read with the transposing LDS read (ds_read_b64_tr_b16): in each 16-lane group,
// lane 4j + c addresses 4 columns X(c) of k-row j, and lane i receives the k-rows
// 0..3 of column X(i >> 2) + (i & 3).  Two such reads (k-rows +0..3, +4..7) give a
// lane the 8 consecutive k of its column that the bf16 MFMA operand holds.
template <AbType AB, CType CT, bool SILU, int BM, int BNB, int WM, int WN, int PF, int ST, bool BT = false,
          bool STG = false>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_kernel(GemmArgs args) {
  using Cfg = GemmCfg<AB, CT, SILU, BM, BNB, WM, WN, PF, ST, STG>;
  using Tr = AbTraits<AB>;
  static_assert(!BT || (AB == AbType::BF16 && !SILU && PF == 0 && BNB % 64 == 0),
                "B as [K, N] rows: bf16 operands, direct loads, no SiLU, whole 64-column blocks");
  constexpr int THREADS = Cfg::kThreads;
  constexpr int SM = Cfg::kSM, SNB = Cfg::kSNB, SNO = Cfg::kSNO;

  __shared__ __attribute__((aligned(16))) uint8_t smem[ST][Cfg::kStageBytes];
  __shared__ int s_mt_pre[kMaxExperts + 1];
  __shared__ float s_red[(CT == CType::FP8) ? WN * BM : 1];

  const int tid = threadIdx.x;
  int lane = tid & 63;
  const int wave = (int)__builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: lives in an SGPR
  const int wm = wave % WM;
  const int wn = wave / WM;
  int ii = lane & 15;         // MFMA row/column index of this lane
  int g = lane >> 4;          // MFMA k-group of this lane
  int rd_swz = swz(ii);       // fragment reads: swizzle of the lane's rows
  // The lane index is made opaque to the compiler at the top of every tile and
  // before every epilogue, so that values derived from it (load rows, epilogue
  // columns) are recomputed there instead of being hoisted out of the tile loop
  // and held in VGPRs through the K loop.  Held there, they pushed the fp8
  // kernels into spills, and each spill reload waits for every outstanding
  // load, the direct loads of the next slices included.
  auto relane = [&]() MOE_INLINE {
    asm volatile("" : "+v"(lane));
    ii = lane & 15;
    g = lane >> 4;
    rd_swz = swz(ii);
  };
  const int E = args.E;
  const int* __restrict__ offsets = args.offsets;
  // offsets as read from memory, clamped to [0, M_rows] so that no row index
  // can leave A or C even for inconsistent input
  auto off_at = [&](int e) MOE_INLINE { return min(max(offsets[e], 0), args.M_rows); };
  // A row of product row p (p in [0, M_rows)); clamped so that an inconsistent
  // permutation cannot leave A
  auto a_row_of = [&](int p) MOE_INLINE {
    if (args.a_rows == nullptr) return p;
    return min(max(args.a_rows[p] / args.a_div, 0), args.a_total - 1);
  };

  const bool kg = args.koff != nullptr;   // K-grouped mode (wave-uniform)
  constexpr bool kEvenSplit = AB == AbType::FP8 && SILU && MOE_EVEN_SPLIT_FP8;

  // ---- per-expert m-tile prefix (wave 0, serial per lane + shuffle scan)
  if (wave == 0 && !kg) {
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) local += (max(off_at(e + 1) - off_at(e), 0) + BM - 1) / BM;
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < E) {
        s_mt_pre[e] = run;
        run += (max(off_at(e + 1) - off_at(e), 0) + BM - 1) / BM;
      }
    }
    if (lane == 63) s_mt_pre[E] = incl;
  }
  __syncthreads();

  const int n_tiles = args.n_tiles;
  const int mt_all = (args.M_rows + BM - 1) / BM;   // K-grouped mode: m-tiles of every expert
  const int total_tiles = kg ? E * mt_all * n_tiles : s_mt_pre[E] * n_tiles;
  const int G = gridDim.x;
  const int slot = (G % 8 == 0) ? (int)((blockIdx.x % 8) * (G / 8) + blockIdx.x / 8) : (int)blockIdx.x;
  // Tiles go out in rounds of G.  In a full round, XCD x (workgroups b with b % 8 == x)
  // takes the contiguous tiles [x G/8, (x+1) G/8) of the round.  The last, partial round
  // of `tail` tiles would fill the first XCDs and leave the others idle; it is cut into
  // eight contiguous chunks of ceil(tail/8) instead, one per XCD, so that each XCD's L2
  // serves fewer busy CUs while tiles that share panels still meet in one L2.
  const int full_rounds = total_tiles / G;
  const int tail = total_tiles - full_rounds * G;
  const bool spread = MOE_SPREAD_LAST_ROUND && G % 8 == 0;
  const int tail_chunk = (tail + 7) / 8;
  auto tile_at = [&](int r) MOE_INLINE {   // this workgroup's tile of round r, or -1
    if (r < full_rounds) return r * G + slot;
    if (r > full_rounds || tail == 0) return -1;
    if (!spread) return slot < tail ? r * G + slot : -1;
    const int j = (int)blockIdx.x / 8;
    const int i = (int)(blockIdx.x % 8) * tail_chunk + j;
    return (j < tail_chunk && i < tail) ? r * G + i : -1;
  };

  const int K = args.K;
  const int N_out = args.N_out;
  // operand row strides in bytes (the M-grouped mode: K)
  const uint32_t lda_all = (uint32_t)args.lda * Tr::kEsize;
  const uint32_t ldb_all = (uint32_t)args.ldb * Tr::kEsize;

  // loader geometry: thread owns chunk (tid & 7) of rows (tid >> 3) + i * THREADS/8
  const int ld_ch = tid & 7;
  const int ld_row0 = tid >> 3;
  constexpr int LD_ROW_STEP = THREADS / 8;
  const int ld_lds = ld_row0 * kSliceBytes + ((ld_ch ^ swz(ld_row0)) << 4);

  // ---- a tile's geometry: (expert, n-tile, m-tile) -> rows, K, operand bases.
  // K-grouped mode: every expert has all m-tiles of A, and its own K range.
  struct TileGeo {
    int e, seg_end, m0, out_row0, k_bytes, KT, rows_valid, n0;
    uint32_t lda_b, ldb_b;
    const uint8_t* a_src;
    const uint8_t* b_exp;
  };
  auto decode = [&](int tile) MOE_INLINE {
    TileGeo t;
    int nt, ml;
    t.a_src = args.A;
    if (kg) {
      const int per_e = mt_all * n_tiles;
      t.e = tile / per_e;
      const int local = tile - t.e * per_e;
      nt = local / mt_all;
      ml = local - nt * mt_all;
      t.seg_end = args.M_rows;
      t.m0 = ml * BM;
      t.out_row0 = t.e * args.M_rows + t.m0;   // C[e] follows C[e-1]
      // koff is clamped to [0, lda] (lda bounds the padded column count)
      const int k0 = min(max(args.koff[t.e], 0), args.lda);
      const int k1 = min(max(args.koff[t.e + 1], k0), args.lda);
      t.k_bytes = (k1 - k0) * Tr::kEsize;
      t.a_src = args.A + (long long)args.M_rows * k0 * Tr::kEsize;
      t.b_exp = args.B + (long long)args.N * k0 * Tr::kEsize;
      t.lda_b = t.ldb_b = (uint32_t)t.k_bytes;   // both blocks have rows of the expert's K
    } else {
      const int q = tile / n_tiles;   // s_mt_pre[e] <= q identifies the expert
      int lo = 0, hi = E;             // largest e with s_mt_pre[e] <= q
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_mt_pre[mid] <= q) lo = mid; else hi = mid;
      }
      t.e = lo;
      const int mt_e = s_mt_pre[t.e + 1] - s_mt_pre[t.e];
      const int local = tile - s_mt_pre[t.e] * n_tiles;
      // the expert's m-tiles in blocks of up to MOE_M_BLOCK; within a block n-tile, then
      // m-tile fastest, so that an XCD's consecutive tiles form a near-square block of
      // activation and weight panels (an expert with few m-tiles is one block)
      const int mb = min(local / (MOE_M_BLOCK * n_tiles), (mt_e - 1) / MOE_M_BLOCK);
      const int h = min(MOE_M_BLOCK, mt_e - mb * MOE_M_BLOCK);
      const int within = local - mb * MOE_M_BLOCK * n_tiles;
      nt = within / h;
      ml = mb * MOE_M_BLOCK + (within - nt * h);
      if (kEvenSplit) {
        // the expert's rows split evenly over its m-tiles (sizes differ by at most one
        // row), so that the m-tiles sharing a weight panel stream the same number of lines
        // and read it in step; rows past a tile's end repeat its last row
        const int e0 = off_at(t.e);
        const int m_e = max(off_at(t.e + 1) - e0, 0);
        t.m0 = e0 + (int)((long long)ml * m_e / mt_e);
        t.seg_end = e0 + (int)((long long)(ml + 1) * m_e / mt_e);
      } else {
        t.seg_end = off_at(t.e + 1);
        t.m0 = off_at(t.e) + ml * BM;
      }
      t.out_row0 = t.m0;
      t.k_bytes = K * Tr::kEsize;
      t.b_exp = args.B + (long long)t.e * (BT ? args.K : args.N) * ldb_all;
      t.lda_b = lda_all;
      t.ldb_b = ldb_all;
    }
    t.KT = (t.k_bytes + kSliceBytes - 1) / kSliceBytes;
    t.rows_valid = min(BM, t.seg_end - t.m0);
    t.n0 = nt * Cfg::kBNOut;
    return t;
  };

  // direct-load source rows of this wave for tile t: rowA[j] / rowB[j] are byte offsets
  // of the row that lane i of load j fills (8-row groups; the weight rows follow the
  // tile's LDS order, gate then up for SiLU, each wave slab's columns permuted)
  auto dma_rows = [&](const TileGeo& t, uint32_t(&ra)[Cfg::kDmaA], uint32_t(&rb)[Cfg::kDmaB]) MOE_INLINE {
#pragma unroll
    for (int j = 0; j < Cfg::kDmaA; ++j) {
      const int r = (wave * Cfg::kDmaA + j) * 8 + (lane >> 3);
      ra[j] = (uint32_t)a_row_of(min(t.m0 + r, t.seg_end - 1)) * t.lda_b;
    }
#pragma unroll
    for (int j = 0; j < Cfg::kDmaB; ++j) {
      if constexpr (BT) {
        // load q fills k-rows 8 (q % 8) + [0, 8) of column block q / 8; lane i the
        // k-row 8 (q % 8) + i / 8 at physical chunk i % 8.  The k-row's slice offset
        // and the clamp at K are added at issue (bt_voff).
        const int q = wave * Cfg::kDmaB + j;
        const int kr = ((q & 7) << 3) + (lane >> 3);
        const int lc = (lane & 7) ^ bt_swz(kr);
        const int col = min(t.n0 + (q >> 3) * 64 + lc * 8, N_out - 8);
        rb[j] = (uint32_t)kr * t.ldb_b + (uint32_t)col * 2u;
        continue;
      }
      const int qrow = (wave * Cfg::kDmaB + j) * 8 + (lane >> 3);
      int half = 0, qq = qrow;
      if constexpr (SILU) {
        half = qrow / Cfg::kBNOut;
        qq = qrow - half * Cfg::kBNOut;
      }
      constexpr int SLAB = Cfg::kWNOut;
      const int within = qq % SLAB;
      const int col = min(t.n0 + (qq - within) + slab_col<SNO>(within >> 4, within & 15), N_out - 1);
      rb[j] = (uint32_t)(half * N_out + col) * t.ldb_b;
    }
  };

  int gk = 0;         // slices this workgroup has consumed (selects the direct-load stage)
  for (int r = 0, tile = tile_at(0); tile >= 0; tile = tile_at(++r)) {
    relane();
    const TileGeo tg = decode(tile);
    const int e = tg.e, seg_end = tg.seg_end, m0 = tg.m0, out_row0 = tg.out_row0, k_bytes = tg.k_bytes;
    const int KT = tg.KT, rows_valid = tg.rows_valid, n0 = tg.n0;
    const uint32_t lda_b = tg.lda_b, ldb_b = tg.ldb_b;
    const uint8_t* a_src = tg.a_src;
    const uint8_t* b_exp = tg.b_exp;

    // ---- byte offsets of this thread's source rows (A from its base, B from the expert's slab)
    uint32_t a_off[Cfg::kAIters];
#pragma unroll
    for (int i = 0; i < Cfg::kAIters; ++i) {
      const int r = min(m0 + ld_row0 + i * LD_ROW_STEP, seg_end - 1);
      a_off[i] = (uint32_t)a_row_of(r) * lda_b;
    }
    uint32_t b_off[Cfg::kBIters];
#pragma unroll
    for (int i = 0; i < Cfg::kBIters; ++i) {
      const int qrow = ld_row0 + i * LD_ROW_STEP;          // LDS row within the weight tile
      int half = 0, qq = qrow;
      if constexpr (SILU) {
        half = qrow / Cfg::kBNOut;
        qq = qrow - half * Cfg::kBNOut;
      }
      constexpr int SLAB = Cfg::kWNOut;
      const int within = qq % SLAB;
      const int col = n0 + (qq - within) + slab_col<SNO>(within >> 4, within & 15);
      const int colc = min(col, N_out - 1);
      b_off[i] = (uint32_t)(half * N_out + colc) * ldb_b;
    }

    // Global loads always use an in-bounds address (the last chunk of the row
    // for chunks past K); such chunks are replaced by zeros when stored to LDS.
    auto load_to = [&](uint4(&ra)[Cfg::kAIters], uint4(&rb)[Cfg::kBIters], int kt) MOE_INLINE {
      const int kb = min(kt * kSliceBytes + ld_ch * 16, k_bytes - 16);
#pragma unroll
      for (int i = 0; i < Cfg::kAIters; ++i)
        ra[i] = *reinterpret_cast<const uint4*>(a_src + a_off[i] + kb);
#pragma unroll
      for (int i = 0; i < Cfg::kBIters; ++i)
        rb[i] = *reinterpret_cast<const uint4*>(b_exp + b_off[i] + kb);
    };
    auto store_from = [&](const uint4(&ra)[Cfg::kAIters], const uint4(&rb)[Cfg::kBIters], int buf,
                          int kt) MOE_INLINE {
      // all-ones when the chunk lies inside K, else zero (a mask keeps the arrays in registers)
      const uint32_t keep = (kt * kSliceBytes + ld_ch * 16 < k_bytes) ? 0xffffffffu : 0u;
      auto masked = [keep](uint4 v) MOE_INLINE {
        return make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
      };
      uint8_t* base = smem[buf];
#pragma unroll
      for (int i = 0; i < Cfg::kAIters; ++i)
        *reinterpret_cast<uint4*>(base + ld_lds + i * LD_ROW_STEP * kSliceBytes) = masked(ra[i]);
#pragma unroll
      for (int i = 0; i < Cfg::kBIters; ++i)
        *reinterpret_cast<uint4*>(base + BM * kSliceBytes + ld_lds + i * LD_ROW_STEP * kSliceBytes) =
            masked(rb[i]);
    };

    f32x4 acc[SM][SNB];
#pragma unroll
    for (int t = 0; t < SM; ++t)
#pragma unroll
      for (int s = 0; s < SNB; ++s) acc[t][s] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Activation subtile t of wave wm holds tile rows 16*(t*WM + wm) + [0, 16): the
    // waves of a column interleave, so a short tile still spreads over all of them.
    // FULL = every subtile has valid rows; otherwise subtiles past rows_valid skip
    // their LDS reads and MFMAs.
    // Register-prefetch path (bf16 and f32): per slice, all fragments of a step are
    // read, then that step's MFMAs issue.
    auto compute = [&](auto full_tag, int buf, int kt, bool k_tail) MOE_INLINE {
      static_assert(AB != AbType::FP8, "fp8 runs on direct loads");
      constexpr bool FULL = decltype(full_tag)::value;
      const uint8_t* sA = smem[buf];
      const uint8_t* sB = smem[buf] + BM * kSliceBytes;
      bool live[SM];
#pragma unroll
      for (int t = 0; t < SM; ++t) live[t] = FULL || 16 * (t * WM + wm) < rows_valid;

#pragma unroll
      for (int step = 0; step < Tr::kSteps; ++step) {
        uint4 af[SM], wf[SNB];
        const int ch = step * 4 + g;
        const int coff = (ch ^ rd_swz) << 4;
#pragma unroll
        for (int s = 0; s < SNB; ++s) {
          int wrow;
          if constexpr (SILU) {
            const int half = s / SNO, ss = s - half * SNO;
            wrow = half * Cfg::kBNOut + wn * Cfg::kWNOut + 16 * ss + ii;
          } else {
            wrow = wn * Cfg::kWNB + 16 * s + ii;
          }
          wf[s] = *reinterpret_cast<const uint4*>(sB + wrow * kSliceBytes + coff);
        }
#pragma unroll
        for (int t = 0; t < SM; ++t)
          if (live[t]) af[t] = *reinterpret_cast<const uint4*>(sA + (16 * (t * WM + wm) + ii) * kSliceBytes + coff);
        if (k_tail) {
          // chunks past K hold copies of the row's last chunk: zero the activation side
          const uint32_t keep = (kt * kSliceBytes + ch * 16 < k_bytes) ? 0xffffffffu : 0u;
#pragma unroll
          for (int t = 0; t < SM; ++t) af[t] = make_uint4(af[t].x & keep, af[t].y & keep, af[t].z & keep, af[t].w & keep);
        }
#pragma unroll
        for (int t = 0; t < SM; ++t) {
          if (!live[t]) continue;
#pragma unroll
          for (int s = 0; s < SNB; ++s) {
            if constexpr (AB == AbType::BF16) {
              acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, wf[s]), __builtin_bit_cast(bf16x8, af[t]), acc[t][s], 0, 0, 0);
            } else {
              const float4 w4 = __builtin_bit_cast(float4, wf[s]);
              const float4 a4 = __builtin_bit_cast(float4, af[t]);
              acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(w4.x, a4.x, acc[t][s], 0, 0, 0);
              acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(w4.y, a4.y, acc[t][s], 0, 0, 0);
              acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(w4.z, a4.z, acc[t][s], 0, 0, 0);
              acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(w4.w, a4.w, acc[t][s], 0, 0, 0);
            }
          }
        }
      }
    };

    // ---- K loop: direct loads into an ST-stage LDS ring (PF = 0), or an LDS double buffer
    //      fed from registers with PF slices of loads in flight (PF = 1, 2)
    auto k_loop = [&](auto full_tag) MOE_INLINE {
      if constexpr (PF == 0) {
        // Direct global->LDS loads into ST LDS stages, ST-1 slices in flight.  The
        // stage of a slice follows the workgroup's running slice count gk, so the
        // first slices of the next tile never land in a stage that other waves
        // may still be reading.
        const uint8_t* a_u = uniform_ptr(a_src);
        const uint8_t* b_u = uniform_ptr(b_exp);
        const uint32_t wave_u = uniform_u32((uint32_t)wave);
        const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)&smem[0][0];
        // lane i of a load fills row i/8 of an 8-row group at physical chunk i%8,
        // i.e. logical chunk (i%8) ^ swz(row) = (i%8) ^ (i/8)
        const uint32_t cc = 16u * ((lane & 7) ^ (lane >> 3));
        uint32_t rowA[Cfg::kDmaA], rowB[Cfg::kDmaB];
        dma_rows(tg, rowA, rowB);
        // fp8 block scales of slice kt: the activation-scale waves load the scales of
        // tile rows wave*64 + lane (block-major layout: row-contiguous per K block;
        // rows past the buffer repeat its last row; gathered A: the scales of the
        // row's A row), the others the weight scales
        // of (wave column q/2, half q%2) in lane q < 2*WN (other lanes repeat lane 0)
        const uint8_t* sc_u = nullptr;
        uint32_t sc_off = 0, sc_step = 0;
        if constexpr (Cfg::kLdsScales) {
          if (wave < Cfg::kScaleWaves) {
            const int pr = min(m0 + wave * 64 + lane, args.M_rows - 1);
            const int r = args.a_scales_by_row ? pr : a_row_of(pr);
            sc_u = uniform_ptr(reinterpret_cast<const uint8_t*>(args.a_scales));
            sc_off = (uint32_t)r * 4u;
            sc_step = (uint32_t)(args.a_scales_by_row ? args.M_rows : args.a_total) * 4u;
          } else {
            const int q = lane < 2 * WN ? lane : 0;
            const int wq = q >> 1, hq = q & 1;
            const int NB = args.N / 128;
            int nb = SILU ? (hq * N_out + n0 + wq * Cfg::kWNOut) / 128 : (n0 + wq * Cfg::kWNB) / 128;
            nb = min(nb, NB - 1);
            sc_u = uniform_ptr(reinterpret_cast<const uint8_t*>(args.b_scales + (long long)e * NB * (K / 128)));
            sc_off = (uint32_t)(nb * (K / 128)) * 4u;
            sc_step = 4u;
          }
        }
        // load j of this wave for slice kt (j < kDmaA: activation rows; < kDmaPerSlice:
        // weight rows; fp8: then the block scales)
        if constexpr (AB == AbType::FP8) {
          // fp8 K is a multiple of 128 (whole slices): each lane's offset within a
          // slice is fixed for the tile, and the slice offset goes into the scalar base
#pragma unroll
          for (int j = 0; j < Cfg::kDmaA; ++j) rowA[j] += cc;
#pragma unroll
          for (int j = 0; j < Cfg::kDmaB; ++j) rowB[j] += cc;
        }
        // BT: offset of load jb's source for slice kt: the lane's k-row kt*KS + kr (KS bf16
        // k-rows per slice), clamped to the last k-row of B (rows past K meet zeroed
        // activations).  rb already holds kr * ldb_b, so the clamp adds (kt*KS - over) rows,
        // which may be negative for K < KS; the unsigned arithmetic wraps to the right offset.
        auto bt_voff = [&](uint32_t rb, int jb, int kt) MOE_INLINE {
          constexpr int KS = kSliceBytes / 2;
          const int kr = (((wave * Cfg::kDmaB + jb) & 7) << 3) + (lane >> 3);
          const int over = max(kt * KS + kr - (K - 1), 0);
          return rb + (uint32_t)(kt * KS - over) * ldb_b;
        };
        auto issue_one = [&](int j, int kt, int stage) MOE_INLINE {
          const uint32_t sb = lds0 + (uint32_t)stage * Cfg::kStageBytes;
          if constexpr (AB == AbType::FP8) {
            const uint32_t ko = (uint32_t)kt * kSliceBytes;
            if (j < Cfg::kDmaA)
              dma16(sb + (wave_u * Cfg::kDmaA + j) * 1024u, a_u + ko, rowA[j]);
            else if (j < Cfg::kDmaPerSlice)
              dma16(sb + BM * kSliceBytes + (wave_u * Cfg::kDmaB + (j - Cfg::kDmaA)) * 1024u, b_u + ko,
                    rowB[j - Cfg::kDmaA]);
            else
              dma4(sb + Cfg::kTileBytes + wave_u * 256u, sc_u + (uint32_t)kt * sc_step, sc_off);
            return;
          }
          const uint32_t o = min((uint32_t)(kt * kSliceBytes) + cc, (uint32_t)(k_bytes - 16));
          if (j < Cfg::kDmaA)
            dma16(sb + (wave_u * Cfg::kDmaA + j) * 1024u, a_u, rowA[j] + o);
          else if (j < Cfg::kDmaPerSlice)
            dma16(sb + BM * kSliceBytes + (wave_u * Cfg::kDmaB + (j - Cfg::kDmaA)) * 1024u, b_u,
                  BT ? bt_voff(rowB[j - Cfg::kDmaA], j - Cfg::kDmaA, kt) : rowB[j - Cfg::kDmaA] + o);
          else
            dma4(sb + Cfg::kTileBytes + wave_u * 256u, sc_u, sc_off + (uint32_t)kt * sc_step);
        };
        auto issue = [&](int kt, int stage) MOE_INLINE {
#pragma unroll
          for (int j = 0; j < Cfg::kDmaTotal; ++j) issue_one(j, kt, stage);
        };
        const bool has_tail = (k_bytes % kSliceBytes) != 0;
        int st = gk % ST;                       // stage of slice kt
        if constexpr (AB == AbType::BF16) {
          // Software pipeline over the two 32-deep MFMA steps of a slice.  Step s+1's
          // fragments are read into the other register set while step s's MFMAs
          // issue, and the slice barrier sits between the two steps, so that the
          // MFMAs of step 1 (operands already in registers) cover the LDS reads of
          // the next slice's step 0 instead of the whole workgroup stalling on them.
          // The reads go out a share per MFMA row (the row's activation fragment and
          // SNB/SM weight fragments before its MFMAs), not as one burst per step: the
          // LDS serves the 8 waves' reads and the direct loads' writes in about the
          // time the MFMAs take, and spreading the reads keeps it busy evenly
          // (gpt-oss-20b and Mixtral-8x7B layers 1-2% faster, outputs bit-identical).
          //
          // ST stages, ST-1 slices in flight.  Stage reuse: the loads of slice
          // kt+ST-1 land in the stage of slice kt-1.  Every wave has finished reading
          // slice kt-1 before barrier kt-1 (its reads are drained with lgkmcnt(0)
          // there), and slice kt+ST-1's loads are issued after it, in the body of
          // slice kt.
          constexpr bool FULL = decltype(full_tag)::value;
          bool live[SM];
#pragma unroll
          for (int t = 0; t < SM; ++t) live[t] = FULL || 16 * (t * WM + wm) < rows_valid;
          // fragments of step `step` from LDS stage `stage`: weight subtiles [s_lo, s_hi)
          // and activation subtiles [t_lo, t_hi) (constant ranges once inlined)
          auto read_range = [&](int stage, int step, uint4(&fa)[SM], uint4(&fw)[SNB], int s_lo, int s_hi,
                                int t_lo, int t_hi) MOE_INLINE {
            const uint8_t* sA = smem[stage];
            const uint8_t* sB = smem[stage] + BM * kSliceBytes;
            const int coff = ((step * 4 + g) ^ rd_swz) << 4;
            if constexpr (BT) {
              // lane 16g + 4j + c addresses k-row step*32 + 8g + j, columns X(c) =
              // the wave's column of MFMA row 4c of subtile s (slab_col keeps each
              // lane's 4 columns contiguous), and receives its own column's k-rows
              typedef short v4s __attribute__((ext_vector_type(4)));
              typedef __attribute__((address_space(3))) v4s lds_v4s;
              const int jr = (lane & 15) >> 2, cq = lane & 3;
              const auto lB = (__attribute__((address_space(3))) uint8_t*)sB;
#pragma unroll
              for (int s = 0; s < SNB; ++s) {
                if (s < s_lo || s >= s_hi) continue;
                const int X = wn * Cfg::kWNB + slab_col<SNO>(s, 4 * cq);
                const int off = (X >> 6) * (64 * kSliceBytes) + (step * 32 + 8 * g + jr) * kSliceBytes +
                                ((((X & 63) >> 3) ^ bt_swz(jr)) << 4) + (X & 7) * 2;
                const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(lB + off));
                const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(lB + off + 4 * kSliceBytes));
                fw[s] = make_uint4((uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                                   (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                                   (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                                   (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16));
              }
            } else {
#pragma unroll
              for (int s = 0; s < SNB; ++s) {
                if (s < s_lo || s >= s_hi) continue;
                int wrow;
                if constexpr (SILU) {
                  const int half = s / SNO, ss = s - half * SNO;
                  wrow = half * Cfg::kBNOut + wn * Cfg::kWNOut + 16 * ss + ii;
                } else {
                  wrow = wn * Cfg::kWNB + 16 * s + ii;
                }
                fw[s] = *reinterpret_cast<const uint4*>(sB + wrow * kSliceBytes + coff);
              }
            }
            // every subtile is read (its LDS rows always exist); dead ones skip only
            // their MFMAs, so the reads need no exec mask
#pragma unroll
            for (int t = 0; t < SM; ++t)
              if (t >= t_lo && t < t_hi)
                fa[t] = *reinterpret_cast<const uint4*>(sA + (16 * (t * WM + wm) + ii) * kSliceBytes + coff);
          };
          auto read_step = [&](int stage, int step, uint4(&fa)[SM], uint4(&fw)[SNB]) MOE_INLINE {
            read_range(stage, step, fa, fw, 0, SNB, 0, SM);
          };
          // keep: all-ones, or zero for a K chunk past the end (its bytes are copies
          // of the row's last chunk); zeroing the activation side suffices
          auto mma_row = [&](int t, const uint4(&fa)[SM], const uint4(&fw)[SNB], uint32_t keep) MOE_INLINE {
            if (!live[t]) return;
            const uint4 a = make_uint4(fa[t].x & keep, fa[t].y & keep, fa[t].z & keep, fa[t].w & keep);
#pragma unroll
            for (int s = 0; s < SNB; ++s)
              acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fw[s]),
                                                                  __builtin_bit_cast(bf16x8, a), acc[t][s], 0, 0, 0);
          };
          // Prologue: the tile's first ST-1 slices.  They are issued after the previous
          // tile's epilogue stores, so waiting for slice 0 needs no wait for those stores
          // (loads complete in order among themselves).  Issuing them before that
          // epilogue instead, to overlap its latency, measured 1-2% slower: the wait
          // then had to cover the stores too.  The stages they land in never hold the
          // previous tile's last slice, the only one a wave may still be reading.
          uint4 fa0[SM], fw0[SNB], fa1[SM], fw1[SNB];
          {
            const int npro = min(ST - 1, KT);
            for (int s2 = 0; s2 < npro; ++s2) issue(s2, (st + s2) % ST);
            wait_slices<Cfg::kDmaPerSlice, ST - 2, false>(npro - 1);   // slice 0 has landed
          }
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          read_step(st, 0, fa0, fw0);
          // one slice; LAST = no next slice (no barrier, no reads of it).  The last
          // slice is peeled off so that the body is straight-line code and the
          // compiler's LDS wait counts stay exact.
          // Within an MFMA row, one LDS fragment read after each MFMA (then the row's
          // remaining MFMAs) rather than the reads as a group before the MFMAs, so that the
          // LDS sees an even stream of reads (gpt-oss-20b and Mixtral-8x7B layers 0.3-1.7%
          // faster, outputs bit-identical; two MFMAs per read and reads after MFMA pairs
          // measured slower).  Instructions outside these classes (the direct loads) are
          // placed by the scheduler.
          auto interleave_row = []() MOE_INLINE {
            constexpr int kR = SNB / SM + 1, kM = SNB, kI = kR < kM ? kR : kM;
#pragma unroll
            for (int q = 0; q < kI; ++q) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kM - kI, 0);
          };
          auto body = [&](int kt, auto last_tag) MOE_INLINE {
            constexpr bool LAST = decltype(last_tag)::value;
            const bool tail = LAST && has_tail;
            const uint32_t keep0 = (tail && kt * kSliceBytes + g * 16 >= k_bytes) ? 0u : ~0u;
            const uint32_t keep1 = (tail && kt * kSliceBytes + (4 + g) * 16 >= k_bytes) ? 0u : ~0u;
            const bool more = kt + ST - 1 < KT;
            const int stn = (st == 0) ? ST - 1 : st - 1;   // stage of slice kt+ST-1 (= of kt-1)
#pragma unroll
            for (int t = 0; t < SM; ++t) {
              read_range(st, 1, fa1, fw1, t * SNB / SM, (t + 1) * SNB / SM, t, t + 1);
              mma_row(t, fa0, fw0, keep0);
              if (!LAST && more) {
#pragma unroll
                for (int j = 0; j < Cfg::kDmaPerSlice; ++j)
                  if (j * SM / Cfg::kDmaPerSlice == t) issue_one(j, kt + ST - 1, stn);
              }
              interleave_row();
              __builtin_amdgcn_sched_barrier(0);
            }
            const int st1 = (st == ST - 1) ? 0 : st + 1;
            if constexpr (!LAST) {
              // slice kt+1 has landed once only the slices after it are outstanding
              wait_slices<Cfg::kDmaPerSlice, ST - 2, true>(min(ST - 2, KT - 2 - kt));
              __builtin_amdgcn_s_barrier();
              asm volatile("" ::: "memory");
            }
#pragma unroll
            for (int t = 0; t < SM; ++t) {
              if constexpr (!LAST) read_range(st1, 0, fa0, fw0, t * SNB / SM, (t + 1) * SNB / SM, t, t + 1);
              mma_row(t, fa1, fw1, keep1);
              interleave_row();
              __builtin_amdgcn_sched_barrier(0);
            }
            st = st1;
          };
          for (int kt = 0; kt + 1 < KT; ++kt) body(kt, std::integral_constant<bool, false>{});
          body(KT - 1, std::integral_constant<bool, true>{});
          gk += KT;
        } else {
          static_assert(AB == AbType::FP8, "direct loads serve bf16 and fp8");
          // Software pipeline over the two column halves of a slice (the slice's K is
          // one 128-deep MFMA).  The second half's weight fragments are read while the
          // first half's MFMAs issue, and the slice barrier sits between the halves,
          // so that the second half's MFMAs cover the reads of the next slice's
          // activations, first-half weights and block scales.  Stage reuse as in the
          // bf16 loop: slice kt+2's loads go to the stage of slice kt-1 and are issued
          // after barrier kt-1.  Each 128-deep MFMA gives one K block's partial sums,
          // which are scaled by (activation scale x weight scale) into the accumulator.
          // The reads go out a share per MFMA row rather than in one burst per half
          // (as in the bf16 loop): DeepSeek-V3-shaped layer 4.87 -> 4.66 ms, outputs
          // bit-identical.  The second half's rows read the next slice's first SM/2
          // activation rows, its scales and first-half weights; its last SM/2 activation
          // rows are read by the first rows of that slice's first half, for their MFMAs
          // rows later, which evens out the LDS reads between the halves (another -1%).
          static_assert(SNB % 2 == 0, "two column halves");
          constexpr int SH = SNB / 2;   // weight subtiles per half (SiLU: gate, then up)
          constexpr bool FULL = decltype(full_tag)::value;
          bool live[SM];
#pragma unroll
          for (int t = 0; t < SM; ++t) live[t] = FULL || 16 * (t * WM + wm) < rows_valid;
          // fragments are kept as the MFMA's 8-register operands (two 16-byte reads each)
          struct ASet {
            i32x8 a[SM];
            float sa[SM];
            float sb[2];
          };
          auto ld32 = [](const uint8_t* base, int row, int c0) MOE_INLINE {
            const uint4 lo = *reinterpret_cast<const uint4*>(base + row * kSliceBytes + (((c0) ^ swz(row)) << 4));
            const uint4 hi = *reinterpret_cast<const uint4*>(base + row * kSliceBytes + (((c0 + 1) ^ swz(row)) << 4));
            return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          };
          // fragment reads from LDS stage `stage`: activation row group t with its
          // scale, the two weight-block scales, weight subtile sl of column half h
          auto read_a_row = [&](int stage, ASet& x, int t) MOE_INLINE {
            const uint8_t* sA = smem[stage];
            const uint8_t* scs = smem[stage] + Cfg::kTileBytes;
            const int row = 16 * (t * WM + wm) + ii;
            x.a[t] = ld32(sA, row, 2 * g);
            x.sa[t] = *reinterpret_cast<const float*>(scs + row * 4);
          };
          auto read_sb = [&](int stage, ASet& x) MOE_INLINE {
            const uint8_t* scs = smem[stage] + Cfg::kTileBytes;
            x.sb[0] = *reinterpret_cast<const float*>(scs + Cfg::kScaleWaves * 256 + (2 * wn) * 4);
            x.sb[1] = *reinterpret_cast<const float*>(scs + Cfg::kScaleWaves * 256 + (2 * wn + 1) * 4);
          };
          auto read_w_one = [&](int stage, int h, int sl, i32x8(&w)[SH]) MOE_INLINE {
            const uint8_t* sB = smem[stage] + BM * kSliceBytes;
            const int sidx = h * SH + sl;
            int wrow;
            if constexpr (SILU) {
              const int half = sidx / SNO, ss = sidx - half * SNO;
              wrow = half * Cfg::kBNOut + wn * Cfg::kWNOut + 16 * ss + ii;
            } else {
              wrow = wn * Cfg::kWNB + 16 * sidx + ii;
            }
            w[sl] = ld32(sB, wrow, 2 * g);
          };
          auto read_w = [&](int stage, int h, i32x8(&w)[SH]) MOE_INLINE {
#pragma unroll
            for (int sl = 0; sl < SH; ++sl) read_w_one(stage, h, sl, w);
          };
          // within a row, partial sums are scaled one MFMA behind, so no FMA waits on
          // the MFMA just issued
          auto mma_half = [&](int h, ASet& x, const i32x8(&w)[SH], auto&& dma_row) MOE_INLINE {
#pragma unroll
            for (int t = 0; t < SM; ++t) {
              dma_row(t);
              if (!live[t]) continue;
              const float f = x.sa[t] * x.sb[h];
              f32x4 prev;
#pragma unroll
              for (int sl = 0; sl < SH; ++sl) {
                const f32x4 cur = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    w[sl], x.a[t], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                // keep the previous MFMA's scaling after this MFMA's issue
                __builtin_amdgcn_sched_barrier(0);
                if (sl > 0) {
#pragma unroll
                  for (int r = 0; r < 4; ++r) acc[t][h * SH + sl - 1][r] = fmaf(prev[r], f, acc[t][h * SH + sl - 1][r]);
                }
                prev = cur;
              }
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[t][h * SH + SH - 1][r] = fmaf(prev[r], f, acc[t][h * SH + SH - 1][r]);
            }
          };
          auto next_stage = [](int x) MOE_INLINE { return (x + 1 == ST) ? 0 : x + 1; };
          ASet A0, A1;
          i32x8 w0[SH], w1[SH];
          {
            const int npro = min(ST - 1, KT);
            for (int s2 = 0; s2 < npro; ++s2) issue(s2, (st + s2) % ST);
            wait_slices<Cfg::kDmaTotal, ST - 2, false>(npro - 1);   // slice 0 has landed
          }
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          // activation rows of a slice read ahead of its first half (the rest inside it)
          constexpr int kEarly = SM >= 2 ? SM / 2 : SM;
#pragma unroll
          for (int t = 0; t < kEarly; ++t) read_a_row(st, A0, t);
          read_sb(st, A0);
          read_w(st, 0, w0);
          auto body = [&](int kt, ASet& cur, ASet& nxt, auto last_tag) MOE_INLINE {
            constexpr bool LAST = decltype(last_tag)::value;
            const bool more = kt + ST - 1 < KT;
            const int stn = (st == 0) ? ST - 1 : st - 1;   // stage of slice kt+ST-1 (= of kt-1)
            mma_half(0, cur, w0, [&](int t) MOE_INLINE {
              if (t < SM - kEarly) read_a_row(st, cur, kEarly + t);
#pragma unroll
              for (int sl = 0; sl < SH; ++sl)
                if ((sl < SM - 1 ? sl : SM - 1) == t) read_w_one(st, 1, sl, w1);
              if (!LAST && more) {
#pragma unroll
                for (int j = 0; j < Cfg::kDmaTotal; ++j)
                  if (j * SM / Cfg::kDmaTotal == t) issue_one(j, kt + ST - 1, stn);
              }
              __builtin_amdgcn_sched_barrier(0);
            });
            __builtin_amdgcn_sched_barrier(0);
            const int st1 = next_stage(st);
            if constexpr (!LAST) {
              // slice kt+1 has landed once only the slices after it are outstanding
              wait_slices<Cfg::kDmaTotal, ST - 2, true>(min(ST - 2, KT - 2 - kt));
              __builtin_amdgcn_s_barrier();
              asm volatile("" ::: "memory");
            }
            mma_half(1, cur, w1, [&](int t) MOE_INLINE {
              if constexpr (!LAST) {
                if (t == 0) read_sb(st1, nxt);
                if (t < kEarly) read_a_row(st1, nxt, t);
#pragma unroll
                for (int sl = 0; sl < SH; ++sl)
                  if ((sl < SM - 1 ? sl : SM - 1) == t) read_w_one(st1, 0, sl, w0);
              }
              __builtin_amdgcn_sched_barrier(0);
            });
            __builtin_amdgcn_sched_barrier(0);
            st = st1;
          };
          using F_ = std::integral_constant<bool, false>;
          using T_ = std::integral_constant<bool, true>;
          int kt = 0;
          for (; kt + 2 < KT; kt += 2) {
            body(kt, A0, A1, F_{});
            body(kt + 1, A1, A0, F_{});
          }
          if (kt + 2 == KT) {
            body(kt, A0, A1, F_{});
            body(kt + 1, A1, A0, T_{});
          } else {
            body(kt, A0, A1, T_{});
          }
          gk += KT;
        }
      } else {
        uint4 ra0[Cfg::kAIters], rb0[Cfg::kBIters];
        if constexpr (PF == 1) {
          load_to(ra0, rb0, 0);
          store_from(ra0, rb0, 0, 0);
          __syncthreads();
          for (int kt = 0; kt < KT; ++kt) {
            if (kt + 1 < KT) load_to(ra0, rb0, kt + 1);
            compute(full_tag, kt & 1, kt, false);
            if (kt + 1 < KT) store_from(ra0, rb0, (kt + 1) & 1, kt + 1);
            __syncthreads();
          }
        } else {
          uint4 ra1[Cfg::kAIters], rb1[Cfg::kBIters];
          load_to(ra0, rb0, 0);
          if (KT > 1) load_to(ra1, rb1, 1);
          store_from(ra0, rb0, 0, 0);
          __syncthreads();
          for (int kt = 0; kt < KT; kt += 2) {
            // slice kt is in LDS buffer 0; slice kt+1 is in flight in set 1
            if (kt + 2 < KT) load_to(ra0, rb0, kt + 2);
            compute(full_tag, 0, kt, false);
            if (kt + 1 < KT) store_from(ra1, rb1, 1, kt + 1);
            __syncthreads();
            if (kt + 1 >= KT) break;
            // slice kt+1 is in LDS buffer 1; slice kt+2 is in flight in set 0
            if (kt + 3 < KT) load_to(ra1, rb1, kt + 3);
            compute(full_tag, 1, kt + 1, false);
            if (kt + 2 < KT) store_from(ra0, rb0, 0, kt + 2);
            __syncthreads();
          }
        }
      }
    };
    // (K-grouped mode: an expert with no rows has K = 0; its tiles store zeros)
    if (KT > 0) {
      if (rows_valid >= BM)
        k_loop(std::integral_constant<bool, true>{});
      else
        k_loop(std::integral_constant<bool, false>{});
    }

    // ---- epilogue: lane holds columns [cbase, cbase + 4*SNO) of tile row 16*(t*WM+wm) + ii
    relane();
    if constexpr (Cfg::kStagedOut) {
      if constexpr (SILU && CT == CType::BF16) {
        // the f32 pre-activations (backward's recompute) keep direct stores
        if (args.pre_out != nullptr) {
          const int cb = n0 + wn * Cfg::kWNOut + 4 * SNO * g;
#pragma unroll
          for (int t = 0; t < SM; ++t) {
            const int rloc = 16 * (t * WM + wm) + ii;
            if (rloc >= rows_valid) continue;
            float* pg = args.pre_out + ((long long)out_row0 + rloc) * 2 * N_out + cb;
#pragma unroll
            for (int s2 = 0; s2 < SNO; ++s2)
              if (cb + 4 * s2 + 4 <= N_out) {
                *reinterpret_cast<float4*>(pg + 4 * s2) =
                    make_float4(acc[t][s2][0], acc[t][s2][1], acc[t][s2][2], acc[t][s2][3]);
                *reinterpret_cast<float4*>(pg + N_out + 4 * s2) = make_float4(
                    acc[t][SNO + s2][0], acc[t][SNO + s2][1], acc[t][SNO + s2][2], acc[t][SNO + s2][3]);
              }
          }
        }
      }
      // every wave has finished reading the last slice's stage before its block is written
      __syncthreads();
      uint8_t* stg = &smem[0][0] + wave * Cfg::kStgWaveBytes;
      constexpr int CPR = Cfg::kStgChunksPerRow;
      constexpr int kChunks = 16 * CPR;
      constexpr int kColsPerChunk = 16 / Cfg::kOutEsize;
      const int col0 = n0 + wn * Cfg::kWNOut;
#pragma unroll
      for (int t = 0; t < SM; ++t) {
        // row ii of the group: tile row 16 (t WM + wm) + ii; columns as held.  (A wave's
        // LDS accesses run in order, so the writes of group t+1 follow the reads of t.)
        uint8_t* srow = stg + ii * Cfg::kStgRowBytes + 4 * SNO * g * Cfg::kOutEsize;
#pragma unroll
        for (int s2 = 0; s2 < SNO; ++s2) {
          float o4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            o4[r] = SILU ? silu_mul(acc[t][s2][r], acc[t][SNO + s2][r]) : acc[t][s2][r];
          if constexpr (CT == CType::F32) {
            *reinterpret_cast<float4*>(srow + 16 * s2) = make_float4(o4[0], o4[1], o4[2], o4[3]);
          } else {
            *reinterpret_cast<uint2*>(srow + 8 * s2) =
                make_uint2(pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3]));
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the group's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        const int rbase = 16 * (t * WM + wm);
#pragma unroll
        for (int q0 = 0; q0 < kChunks; q0 += kWave) {
          const int q = q0 + lane;
          if (q < kChunks) {
            const int lr = q / CPR, cq = q - (q / CPR) * CPR;
            const int rloc = rbase + lr;
            const int col = col0 + cq * kColsPerChunk;
            if (rloc < rows_valid && col + kColsPerChunk <= N_out) {
              const uint4 val = *reinterpret_cast<const uint4*>(stg + lr * Cfg::kStgRowBytes + cq * 16);
              *reinterpret_cast<uint4*>(args.C + ((long long)(out_row0 + rloc) * N_out + col) * Cfg::kOutEsize) = val;
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
      // the next tile's first loads land in the stages this block overlays
      __syncthreads();
    } else {
    const int cbase = n0 + wn * Cfg::kWNOut + 4 * SNO * g;
    // fp8 output: the scale of each row's 128 columns needs the amax over the WN waves
    // that hold them; every row group's partial amax goes through LDS at once, so that
    // a tile's epilogue takes two barriers instead of two per row group
    [[maybe_unused]] float fp8_scale[SM];
    if constexpr (CT == CType::FP8) {
#pragma unroll
      for (int t = 0; t < SM; ++t) {
        float am = 0.f;
#pragma unroll
        for (int s = 0; s < SNO; ++s)
#pragma unroll
          for (int r = 0; r < 4; ++r) am = fmaxf(am, fabsf(silu_mul(acc[t][s][r], acc[t][SNO + s][r])));
        am = fmaxf(am, __shfl_xor(am, 16, 64));
        am = fmaxf(am, __shfl_xor(am, 32, 64));
        if (g == 0) s_red[wn * BM + 16 * (t * WM + wm) + ii] = am;
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < SM; ++t) {
        float amax = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < WN; ++w2) amax = fmaxf(amax, s_red[w2 * BM + 16 * (t * WM + wm) + ii]);
        fp8_scale[t] = (amax == 0.f) ? 1.f : amax / 448.f;
      }
      __syncthreads();
    }
#pragma unroll
    for (int t = 0; t < SM; ++t) {
      const int rloc = 16 * (t * WM + wm) + ii;
      const bool row_ok = rloc < rows_valid;
      const long long m = (long long)out_row0 + rloc;
      float v[4 * SNO];
#pragma unroll
      for (int s = 0; s < SNO; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[4 * s + r] = SILU ? silu_mul(acc[t][s][r], acc[t][SNO + s][r]) : acc[t][s][r];

      if constexpr (CT == CType::FP8) {
        const float scale = fp8_scale[t];
        if (row_ok && cbase + 4 * SNO <= N_out) {
          uint32_t wd[SNO];
#pragma unroll
          for (int s = 0; s < SNO; ++s)
            wd[s] = cvt_e4m3x2(clamp448(v[4 * s] / scale), clamp448(v[4 * s + 1] / scale)) |
                    (cvt_e4m3x2(clamp448(v[4 * s + 2] / scale), clamp448(v[4 * s + 3] / scale)) << 16);
          uint8_t* dst = args.C + m * N_out + cbase;
          static_assert(SNO == 2 || SNO == 4, "fp8 epilogue writes 8 or 16 codes per lane");
          if constexpr (SNO == 4)
            *reinterpret_cast<uint4*>(dst) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
          else
            *reinterpret_cast<uint2*>(dst) = make_uint2(wd[0], wd[1]);
          if (wn == 0 && g == 0) args.c_scales[(long long)(n0 / 128) * args.M_rows + m] = scale;
        }
      } else if constexpr (CT == CType::BF16) {
        if constexpr (SILU) {
          if (args.pre_out != nullptr && row_ok) {
            float* pg = args.pre_out + m * 2 * N_out + cbase;
#pragma unroll
            for (int s = 0; s < SNO; ++s)
              if (cbase + 4 * s + 4 <= N_out) {
                *reinterpret_cast<float4*>(pg + 4 * s) = make_float4(acc[t][s][0], acc[t][s][1], acc[t][s][2], acc[t][s][3]);
                *reinterpret_cast<float4*>(pg + N_out + 4 * s) =
                    make_float4(acc[t][SNO + s][0], acc[t][SNO + s][1], acc[t][SNO + s][2], acc[t][SNO + s][3]);
              }
          }
        }
        if (row_ok) {
          uint16_t* dst = reinterpret_cast<uint16_t*>(args.C) + m * N_out + cbase;
          // 4*SNO contiguous columns, written as 8-column (16-byte) stores where
          // all 8 columns exist, else as 4-column (8-byte) stores; N_out is a
          // multiple of 8 and cbase of 4, so every 4-column unit is whole.
#pragma unroll
          for (int u = 0; u < SNO / 2; ++u) {
            const int c = cbase + 8 * u;
            const uint2 lo = make_uint2(pack_bf16x2(v[8 * u], v[8 * u + 1]), pack_bf16x2(v[8 * u + 2], v[8 * u + 3]));
            const uint2 hi = make_uint2(pack_bf16x2(v[8 * u + 4], v[8 * u + 5]),
                                        pack_bf16x2(v[8 * u + 6], v[8 * u + 7]));
            if (c + 8 <= N_out)
              *reinterpret_cast<uint4*>(dst + 8 * u) = make_uint4(lo.x, lo.y, hi.x, hi.y);
            else if (c + 4 <= N_out)
              *reinterpret_cast<uint2*>(dst + 8 * u) = lo;
          }
          if constexpr (SNO % 2 == 1) {
            constexpr int u = SNO / 2;
            if (cbase + 8 * u + 4 <= N_out)
              *reinterpret_cast<uint2*>(dst + 8 * u) =
                  make_uint2(pack_bf16x2(v[8 * u], v[8 * u + 1]), pack_bf16x2(v[8 * u + 2], v[8 * u + 3]));
          }
        }
      } else {
        if (row_ok) {
          float* dst = reinterpret_cast<float*>(args.C) + m * N_out + cbase;
#pragma unroll
          for (int s = 0; s < SNO; ++s)
            if (cbase + 4 * s + 4 <= N_out)
              *reinterpret_cast<float4*>(dst + 4 * s) =
                  make_float4(v[4 * s], v[4 * s + 1], v[4 * s + 2], v[4 * s + 3]);
        }
      }
    }
    }
  }

  // ---- sentinel rows [offsets[E], M_rows) of C: exact zeros (fp8 scales: 1.0)
  if (!kg) {
    constexpr int kCEsize = (CT == CType::F32) ? 4 : (CT == CType::BF16 ? 2 : 1);
    const long long V = off_at(E);
    const long long rows = (long long)args.M_rows - V;
    if (rows > 0) {
      const long long row_bytes = (long long)N_out * kCEsize;
      const long long n16 = rows * row_bytes / 16;
      uint4* base = reinterpret_cast<uint4*>(args.C + V * row_bytes);
      int tz = tid;
      asm volatile("" : "+v"(tz));   // computed here, not held through the tile loop
      for (long long i = (long long)blockIdx.x * THREADS + tz; i < n16; i += (long long)G * THREADS)
        base[i] = make_uint4(0, 0, 0, 0);
      if constexpr (CT == CType::FP8) {
        // block-major scales [N_out/128, M_rows]: rows [V, M_rows) of every block
        const long long ns = rows * (N_out / 128);
        for (long long i = (long long)blockIdx.x * THREADS + tz; i < ns; i += (long long)G * THREADS)
          args.c_scales[(i / rows) * args.M_rows + V + (i % rows)] = 1.0f;
      }
    }
  }
}

// ------------------------------------------------------------------------- host side

namespace {

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <AbType AB, CType CT, bool SILU, int BM, int BNB, int WM, int WN, int PF, int ST, bool BT = false,
          bool STG = false>
hipError_t launch_cfg(const GemmArgs& a0, hipStream_t stream) {
  using Cfg = GemmCfg<AB, CT, SILU, BM, BNB, WM, WN, PF, ST, STG>;
  GemmArgs a = a0;
  a.n_tiles = (a.N_out + Cfg::kBNOut - 1) / Cfg::kBNOut;
  auto kern = grouped_gemm_kernel<AB, CT, SILU, BM, BNB, WM, WN, PF, ST, BT, STG>;
  static const int per_cu = [&] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, Cfg::kThreads, 0) != hipSuccess || n <= 0)
      n = 1;
    return n;
  }();
  const int grid = device_cu_count() * per_cu;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(Cfg::kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

namespace {
template <int BM, int BNB, int WM, int WN, int PF, int ST>
struct TileOf {
  static constexpr int kM = BM, kN = BNB;
};
}  // namespace

bool use_decode_tiles(long long M_rows, int E) {
  return M_rows <= (long long)MOE_DECODE_ROWS_PER_EXPERT * E;
}
bool use_mid_tiles(long long M_rows, int E) {
  return !use_decode_tiles(M_rows, E) && M_rows <= (long long)MOE_MID_ROWS_PER_EXPERT * E;
}
bool use_narrow_decode_tiles(long long M_rows, int E) {
  return M_rows <= (long long)MOE_DECODE_NARROW_ROWS_PER_EXPERT * E;
}

bool grouped_gemm_tile_shape(int ab_dtype, bool silu, int c_dtype, long long M_rows, int E, int* tile_m,
                             int* tile_n, int* k_slice) {
  if (ab_dtype == 1 && use_mid_tiles(M_rows, E)) {
    using M1 = TileOf<MOE_TILE_BF16_SILU_MID>;
    using M0 = TileOf<MOE_TILE_BF16_NONE_MID>;
    *tile_m = silu ? M1::kM : M0::kM;
    *tile_n = silu ? M1::kN : M0::kN;
    *k_slice = kSliceBytes / 2;
  } else if (ab_dtype == 1) {
    const bool dec = use_decode_tiles(M_rows, E);
    const bool narrow = use_narrow_decode_tiles(M_rows, E);
    using T1 = TileOf<MOE_TILE_BF16_SILU>;
    using T0 = TileOf<MOE_TILE_BF16_NONE>;
    using D1 = TileOf<MOE_TILE_BF16_SILU_DEC>;
    using D0 = TileOf<MOE_TILE_BF16_NONE_DEC>;
    using N0 = TileOf<MOE_TILE_BF16_NONE_DEC_NARROW>;
    *tile_m = dec ? (silu ? D1::kM : (narrow ? N0::kM : D0::kM)) : (silu ? T1::kM : T0::kM);
    *tile_n = dec ? (silu ? D1::kN : (narrow ? N0::kN : D0::kN)) : (silu ? T1::kN : T0::kN);
    *k_slice = kSliceBytes / 2;
  } else if (ab_dtype == 0) {
    *tile_m = 64;
    *tile_n = 64;
    *k_slice = kSliceBytes / 4;
  } else if (ab_dtype == 2) {
    const bool dec = c_dtype != 2 && use_decode_tiles(M_rows, E);
    using T1 = TileOf<MOE_TILE_FP8_SILU>;
    using T0 = TileOf<MOE_TILE_FP8_NONE>;
    using D1 = TileOf<MOE_TILE_FP8_SILU_DEC>;
    using D0 = TileOf<MOE_TILE_FP8_NONE_DEC>;
    *tile_m = dec ? (silu ? D1::kM : D0::kM) : (silu ? T1::kM : T0::kM);
    *tile_n = dec ? (silu ? D1::kN : D0::kN) : (silu ? T1::kN : T0::kN);
    *k_slice = kSliceBytes;
  } else {
    return false;
  }
  return true;
}

hipError_t launch_grouped_gemm(const GemmLaunch& p, hipStream_t stream) {
  GemmArgs a{};
  a.A = static_cast<const uint8_t*>(p.A);
  a.a_scales = p.a_scales;
  a.B = static_cast<const uint8_t*>(p.B);
  a.b_scales = p.b_scales;
  a.offsets = p.offsets;
  a.E = p.E;
  a.M_rows = (int)p.M_rows;
  a.N = (int)p.N;
  a.K = (int)p.K;
  a.C = static_cast<uint8_t*>(p.C);
  a.c_scales = p.c_scales;
  a.N_out = p.silu ? (int)(p.N / 2) : (int)p.N;
  a.koff = p.koff;
  a.lda = p.koff ? (int)p.lda : (int)p.K;
  a.ldb = p.koff ? (int)p.ldb : (p.b_kn ? (int)p.N : (int)p.K);
  if (p.koff && (p.ab_dtype != 1 || p.silu || p.c_dtype == 2)) return hipErrorInvalidValue;
  a.pre_out = p.pre_out;
  if (p.pre_out && (p.ab_dtype != 1 || !p.silu || p.c_dtype != 1 || p.koff)) return hipErrorInvalidValue;
  a.a_rows = p.a_rows;
  a.a_div = p.a_rows ? p.a_div : 1;
  a.a_total = p.a_rows ? (int)p.a_total : (int)p.M_rows;
  a.a_scales_by_row = (p.a_rows && p.a_scales_by_row) ? 1 : 0;
  if (p.a_rows && (p.koff || p.a_div < 1 || p.a_total < 1)) return hipErrorInvalidValue;

  if (p.b_kn) {
    // B as [E][K][N], no SiLU, M-grouped: 128x256 tiles at up to 384 rows per expert (an
    // expert of ~256 rows fills two 128-row m-tiles, where 192-row tiles would run one
    // third full), else the 192x192 configuration
    if (p.ab_dtype != 1 || p.silu || p.koff || p.c_dtype == 2 || p.N % 8 != 0 || p.N < 8)
      return hipErrorInvalidValue;
    if (p.M_rows <= (long long)MOE_BT_SHORT_ROWS_PER_EXPERT * p.E) {
      if (p.c_dtype == 1) return launch_cfg<AbType::BF16, CType::BF16, false, MOE_TILE_BF16_BT_SHORT, true, true>(a, stream);
      return launch_cfg<AbType::BF16, CType::F32, false, MOE_TILE_BF16_BT_SHORT, true, true>(a, stream);
    }
    if (p.c_dtype == 1) return launch_cfg<AbType::BF16, CType::BF16, false, MOE_TILE_BF16_NONE, true, true>(a, stream);
    return launch_cfg<AbType::BF16, CType::F32, false, MOE_TILE_BF16_NONE, true, true>(a, stream);
  }
  // rows the tile shape is chosen for: the launch's rows, or fewer when the caller knows
  // that only the first tile_rows can be valid
  const long long trows = (p.tile_rows > 0 && p.tile_rows < p.M_rows) ? p.tile_rows : p.M_rows;
  // dtype: 0 f32, 1 bf16, 2 fp8 (moe_dtype_t values)
  if (p.ab_dtype == 1 && !p.koff && use_mid_tiles(trows, p.E)) {
    if (p.silu) {
      if (p.c_dtype == 1) return launch_cfg<AbType::BF16, CType::BF16, true, MOE_TILE_BF16_SILU_MID>(a, stream);
      return launch_cfg<AbType::BF16, CType::F32, true, MOE_TILE_BF16_SILU_MID>(a, stream);
    }
    if (p.c_dtype == 1) return launch_cfg<AbType::BF16, CType::BF16, false, MOE_TILE_BF16_NONE_MID>(a, stream);
    return launch_cfg<AbType::BF16, CType::F32, false, MOE_TILE_BF16_NONE_MID>(a, stream);
  }
  if (p.ab_dtype == 1 && !p.koff && use_decode_tiles(trows, p.E)) {
    if (p.silu) {
      if (p.c_dtype == 1) return launch_cfg<AbType::BF16, CType::BF16, true, MOE_TILE_BF16_SILU_DEC>(a, stream);
      return launch_cfg<AbType::BF16, CType::F32, true, MOE_TILE_BF16_SILU_DEC>(a, stream);
    }
    if (use_narrow_decode_tiles(trows, p.E)) {
      if (p.c_dtype == 1) return launch_cfg<AbType::BF16, CType::BF16, false, MOE_TILE_BF16_NONE_DEC_NARROW>(a, stream);
      return launch_cfg<AbType::BF16, CType::F32, false, MOE_TILE_BF16_NONE_DEC_NARROW>(a, stream);
    }
    if (p.c_dtype == 1) return launch_cfg<AbType::BF16, CType::BF16, false, MOE_TILE_BF16_NONE_DEC>(a, stream);
    return launch_cfg<AbType::BF16, CType::F32, false, MOE_TILE_BF16_NONE_DEC>(a, stream);
  }
  if (p.ab_dtype == 1) {
    if (p.silu) {
      if (p.c_dtype == 1) return launch_cfg<AbType::BF16, CType::BF16, true, MOE_TILE_BF16_SILU>(a, stream);
      return launch_cfg<AbType::BF16, CType::F32, true, MOE_TILE_BF16_SILU>(a, stream);
    }
    if (p.koff) {   // the backward's weight gradients: staged stores
      if (p.c_dtype == 1) return launch_cfg<AbType::BF16, CType::BF16, false, MOE_TILE_BF16_NONE, false, true>(a, stream);
      return launch_cfg<AbType::BF16, CType::F32, false, MOE_TILE_BF16_NONE, false, true>(a, stream);
    }
    if (p.c_dtype == 1) return launch_cfg<AbType::BF16, CType::BF16, false, MOE_TILE_BF16_NONE>(a, stream);
    return launch_cfg<AbType::BF16, CType::F32, false, MOE_TILE_BF16_NONE>(a, stream);
  }
  if (p.ab_dtype == 0) {
    if (p.silu) {
      if (p.c_dtype == 1) return launch_cfg<AbType::F32, CType::BF16, true, 64, 64, 2, 2, 1, 2>(a, stream);
      return launch_cfg<AbType::F32, CType::F32, true, 64, 64, 2, 2, 1, 2>(a, stream);
    }
    if (p.c_dtype == 1) return launch_cfg<AbType::F32, CType::BF16, false, 64, 64, 2, 2, 1, 2>(a, stream);
    return launch_cfg<AbType::F32, CType::F32, false, 64, 64, 2, 2, 1, 2>(a, stream);
  }
  // fp8 operands
  if (!p.koff && p.c_dtype != 2 && use_decode_tiles(p.M_rows, p.E)) {
    if (p.silu) {
      if (p.c_dtype == 1) return launch_cfg<AbType::FP8, CType::BF16, true, MOE_TILE_FP8_SILU_DEC>(a, stream);
      return launch_cfg<AbType::FP8, CType::F32, true, MOE_TILE_FP8_SILU_DEC>(a, stream);
    }
    if (p.c_dtype == 1) return launch_cfg<AbType::FP8, CType::BF16, false, MOE_TILE_FP8_NONE_DEC>(a, stream);
    return launch_cfg<AbType::FP8, CType::F32, false, MOE_TILE_FP8_NONE_DEC>(a, stream);
  }
  if (p.silu) {
    if (p.c_dtype == 2) return launch_cfg<AbType::FP8, CType::FP8, true, MOE_TILE_FP8_SILU>(a, stream);
    if (p.c_dtype == 1) return launch_cfg<AbType::FP8, CType::BF16, true, MOE_TILE_FP8_SILU>(a, stream);
    return launch_cfg<AbType::FP8, CType::F32, true, MOE_TILE_FP8_SILU>(a, stream);
  }
  if (p.c_dtype == 1) return launch_cfg<AbType::FP8, CType::BF16, false, MOE_TILE_FP8_NONE>(a, stream);
  return launch_cfg<AbType::FP8, CType::F32, false, MOE_TILE_FP8_NONE>(a, stream);
}

}  // namespace moe
