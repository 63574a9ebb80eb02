// G2: int8 x int8 -> int32 GEMM on gfx950 MFMA with fused epilogues.
//
//   acc[m, n] = sum_k A[m, k] * B[n, k]          (A, B int8, both K-contiguous)
//
// Forward ("SDNQ: SD.Next Quantization Engine": INT8 quantized matmul with a
// fused scale epilogue, FP32 dequantization as with dequantize_fp32):
//   y[m, n] = bf16( fp32(acc) * (row_scale[m] * col_scale[n]) + sum_j T[m, j] * R[n, j] )
// (the LoRA scale is folded into T or R by the caller)
// Backward input (the quantized matmul of the training path): B is the
// transposed int8 weight, and
//   dx[m, :] = bf16( rot_g( fp32(acc[m, :]) * row_scale[m] ) + sum_j T[m, j] * R[:, j] )
// where rot_g is the normalized block Walsh-Hadamard rotation along the output
// columns (the same transform as the forward's, which is its own inverse).
//
// FP8 (E4M3 x E4M3, the float8_e4m3fn quantized matmul of the same pages): the
// same tiles and loads, one v_mfma_f32_32x32x64_f8f6f4 per 32 x 32 tile and
// 64 k positions with fp32 accumulation, and the same epilogues (forward scales,
// or the backward's inverse rotation).
// Its A and B fragments pair up 64 k positions of a tile the same way (the
// two 16-byte halves the int8 path reads for its two 32-deep steps), so the
// contraction is the full 64-k dot product.
//
// Tiling.  A workgroup of 8 wavefronts (two per SIMD, so one hides the other's
// waits) computes a 256 x BN output tile; K is consumed 128 bytes at a time (one
// whole 128-byte cache line of every operand row per k-tile) through a 2-stage
// LDS ring filled by buffer loads that write LDS directly, one k-tile ahead.
// Each wavefront owns a (256/WAVES_M) x (BN/WAVES_N) sub-tile of 32 x 32 MFMA
// tiles (v_mfma_i32_32x32x32_i8, 16 int32 accumulators each), four 32-deep
// k-steps per k-tile.  The MFMA "row" operand is the B side (weight rows, output
// column n) and the "column" operand the A side (tokens m), so each lane ends up
// holding, for one token, runs of 4 consecutive output columns.
//
// Why 128-byte k-tiles: each compute unit's vector memory path fills LDS at up
// to about 55-67 GB/s (the same whether one tile or all CUs are active, and the
// same for loads into registers), and whole cache lines per row per k-tile use
// it best: instead of half lines they took the 4096 x 3840 x 10240 GEMM from
// 150 to 136 us, and a 3- or 4-stage ring of 64-byte k-tiles in the same LDS
// ran 9 % slower than this 2-stage ring.
//
// LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at chunk
// c ^ (r & 7), which makes the 16-byte fragment reads (8 consecutive rows, one
// logical chunk) conflict-free.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the block index is
// remapped so that each XCD walks a contiguous run of tiles, ordered in groups
// of 4 tile-rows, which keeps the tiles sharing A and B rows in one L2.
#include <type_traits>

#include "sdnq_internal.hpp"

namespace sdnq {
namespace {

constexpr int BM = 256, BK = 128, STAGES = 2;
constexpr int kKSteps = BK / 32;  // 32-deep MFMA steps per k-tile
constexpr int kThreads = 512;     // 8 wavefronts: two per SIMD
constexpr int kGroupM = 4;
constexpr unsigned kOutOfRange = 0x80000000u;  // any offset past num_records reads as zero

constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;  // fl32(1/sqrt(128))

typedef __attribute__((address_space(3))) void lds_void;

template <int G>
__device__ __forceinline__ float norm_const() {
  if constexpr (G == 64) return 0.125f;
  else if constexpr (G == 128) return kInvSqrt128;
  else if constexpr (G == 256) return 0.0625f;
  else return 1.0f;
}

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int &tm, int &tn) {
  const int nblk = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int q = nblk >> 3, rmd = nblk & 7;
  const int logical = xcd * q + (xcd < rmd ? xcd : rmd) + local;
  const int per_group = kGroupM * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int in = logical - group * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

// LoRA term of all of a wavefront's 32 x 32 output tiles at once:
// o[i][j] += sum_r R[n(j), r] * T[m(i), r] (bf16 MFMA 32x32x16, fp32 accumulate;
// lane l holds row l % 32 of its tile and rank entries 8 * (l / 32) .. + 7 of
// each 16-wide step), from operands staged in LDS like a k-tile: the T rows
// (tokens) where the A tile goes and the R rows (output columns) where the B
// tile goes, up to 64 rank values (128 bytes) per row in the ring's row
// layout.  Rank step s (16 values, 32 bytes) sits where the int8 k-step s
// does: lane l reads 16 bytes of its row at logical chunk 2 s + l / 32, stored
// at chunk ^ (l & 7).  arow[i] / brow[j]: the tile rows of the wavefront's
// 32-row blocks.
template <int SMX, int SN>
__device__ __forceinline__ void lora_staged(const int8_t *stage, int a_bytes, int row_bytes, const int (&arow)[SMX],
                                            const int (&brow)[SN], int rank, int lane, v16f (&o)[SMX][SN]) {
  const int8_t *base = stage + (lane & 31) * row_bytes;
  for (int st = 0; st < rank / 16; ++st) {
    const int col = 16 * ((2 * st + (lane >> 5)) ^ (lane & 7));
    v8bf ta[SMX], rb[SN];
#pragma unroll
    for (int i = 0; i < SMX; ++i) ta[i] = *reinterpret_cast<const v8bf *>(base + arow[i] * row_bytes + col);
#pragma unroll
    for (int j = 0; j < SN; ++j)
      rb[j] = *reinterpret_cast<const v8bf *>(base + a_bytes + brow[j] * row_bytes + col);
#pragma unroll
    for (int i = 0; i < SMX; ++i)
#pragma unroll
      for (int j = 0; j < SN; ++j) o[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[j], ta[i], o[i][j], 0, 0, 0);
  }
}

// s_waitcnt vmcnt(N) then s_barrier, as one compiler barrier.  The direct-to-LDS
// loads are invisible to the compiler's wait tracking, so their completion is
// awaited here explicitly before any wavefront reads what the others loaded.
template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Tile geometry for an output tile of BM x BN_.  A stage holds the A tile then
// the B tile, rows of BK bytes, loaded in groups of 8 rows (1 KB, one
// direct-to-LDS load per wavefront).  The groups are dealt to the 8 wavefronts
// round-robin (the A groups fill the first kASlots slots); when they do not
// divide evenly the spare slots load nothing (an out-of-range offset) into a
// 1 KB dummy area.
template <int BN_>
struct TileCfg {
  static constexpr int kStageBytes = (BM + BN_) * BK;
  static constexpr int kGroups = (BM + BN_) / 8;
  static constexpr int kASlots = (BM / 8) / 8;
  static constexpr int kLoadsPerWave = (kGroups + 7) / 8;
  static constexpr bool kDummy = kGroups % 8 != 0;
  // the forward epilogue's column scales of the tile (BN floats) follow the ring
  static constexpr int kScaleOff = STAGES * kStageBytes + (kDummy ? 1024 : 0);
  static constexpr int kLdsBytes = kScaleOff + BN_ * 4;
  static_assert(BN_ % 32 == 0 && (BM / 8) % 8 == 0, "the A groups fill whole load slots");
};

template <bool FP8>
struct AccOf {
  typedef v16i type;
};
template <>
struct AccOf<true> {
  typedef v16f type;
};
__device__ __forceinline__ float acc_f32(int v) { return (float)v; }
__device__ __forceinline__ float acc_f32(float v) { return v; }
typedef int v8i __attribute__((ext_vector_type(8)));

// DIAG (the ceiling diagnostic; 0 in every product launch): 1 drops the k loop's
// global loads after the first two k-tiles, so every k-tile multiplies what those
// left in LDS; 2 also drops the LDS reads, so every MFMA multiplies the fragments
// of the first k-step, held in registers; 3 is 2 with fragments made of the loop
// indices instead of the codes (few toggling bits).  Prologue and epilogue are
// unchanged.
template <Epilogue EPI, int BN, int WAVES_M, int G, bool LORA, bool FP8, int DIAG = 0>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_kernel(GemmArgs args, int tiles_m, int tiles_n) {
  static_assert(DIAG == 0 || (EPI == Epilogue::kForward && !LORA && !FP8), "diagnostic modes: int8 forward only");
  using Cfg = TileCfg<BN>;
  constexpr int kStageBytes = Cfg::kStageBytes;
  constexpr int LPW = Cfg::kLoadsPerWave;
  constexpr int ASL = Cfg::kASlots;
  constexpr int WAVES_N = 8 / WAVES_M;
  constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  constexpr int SM = TM / 32, SN = TN / 32;
  static_assert(TM % 32 == 0 && TN % 32 == 0 && SM * SN <= 10, "at most 160 int32 accumulators per wavefront");

  __shared__ __attribute__((aligned(1024))) int8_t smem[Cfg::kLdsBytes];

  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t M = args.m, N = args.n, K = args.k;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lets LDS bases live in SGPRs
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;

  // ---- direct global -> LDS loads (buffer_load_dwordx4 ... lds)
  // A stage holds the A tile (256 rows x 128 B) then the B tile (BN rows).  Load
  // slot j of a wavefront fills the 8-row group 8*j + wave of the stage (slots
  // below ASL: A groups; the others: B groups): lane i lands at byte 16*i of that
  // 1 KB group, i.e. row 8*g + i/8, stored chunk i%8.  Rows are XOR-swizzled
  // (stored chunk = logical chunk ^ (row & 7)), so lane i fetches logical chunk
  // c = (i & 7) ^ ((i >> 3) & 7).  Rows past the matrix end lie past the
  // buffer's num_records and read as zero, and so do chunks past K (their offset
  // is pushed out of range).
  const int64_t rows_a = (M - m0) < BM ? (M - m0) : BM;
  const int64_t rows_b = (N - n0) < BN ? (N - n0) : BN;
  const __amdgpu_buffer_rsrc_t rsrc_a =
      __builtin_amdgcn_make_buffer_rsrc((void *)(args.a + m0 * K), 0, (int)(rows_a * K), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_b =
      __builtin_amdgcn_make_buffer_rsrc((void *)(args.b + n0 * K), 0, (int)(rows_b * K), 0x00020000);
  const int lc = (lane & 7) ^ ((lane >> 3) & 7);
  // per slot: row group within its operand, or -1 for a spare slot
  int grp[LPW];
  unsigned voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int g = 8 * j + wave;
    grp[j] = j < ASL ? g : (g - BM / 8 < BN / 8 ? g - BM / 8 : -1);
    voff[j] = (unsigned)((8 * (grp[j] < 0 ? 0 : grp[j]) + (lane >> 3)) * K + 16 * lc);
  }
  int8_t *const dummy = smem + STAGES * kStageBytes;

  const int nk = (int)((K + BK - 1) / BK);
  // Load slot j of k-tile kt into its stage.  The tile's first byte k0 is uniform
  // and rides in the scalar offset; the lane's part (and the out-of-range bit,
  // which keeps any sum past num_records) stays in the vector offset.  Only a
  // k-tile that runs past K needs the per-lane range check.
  auto load_slot = [&](int kt, int j) {
    const unsigned k0 = (unsigned)kt * BK;
    const unsigned oob = ((int64_t)k0 + BK <= K) ? 0u : (((int64_t)k0 + 16 * lc < K) ? 0u : kOutOfRange);
    int8_t *base = smem + (kt & (STAGES - 1)) * kStageBytes;
    // wavefront-uniform selects, no branch: a spare slot loads nothing into the dummy area
    const bool spare = Cfg::kDummy && j >= ASL && grp[j] < 0;
    int8_t *dst = spare ? dummy : base + (j < ASL ? 0 : BM * BK) + grp[j] * 1024;
    const unsigned off = spare ? kOutOfRange : (voff[j] | oob);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(j < ASL ? rsrc_a : rsrc_b, (lds_void *)dst, 16, off, (int)k0, 0, 0);
  };
  auto issue_loads = [&](int kt) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) load_slot(kt, j);
  };

  // ---- LoRA operands of the epilogue (forward and backward with LoRA): the T
  // rows (tokens) and R rows (output columns) of the tile, in chunks of 64 rank
  // values (128 bytes, one stage row), with the same slot layout and swizzle as
  // a k-tile (T rows where the A rows go, R rows where the B rows go).  Chunk 0
  // takes the place of the zero-filled tile nk: it is loaded into the ring's
  // free stage while the last k-tile is multiplied.  Later chunks (rank > 64)
  // are loaded into the same stage once the previous one has been used.
  constexpr bool kLoraStaged = LORA && EPI != Epilogue::kInt32;
  constexpr int kLoraChunk = BK / 2;
  int8_t *const lora_stage = smem + (nk & (STAGES - 1)) * kStageBytes;
  auto issue_lora_loads = [&](int chunk) {
    const int rb = args.rank * 2;
    const __amdgpu_buffer_rsrc_t rsrc_t = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(args.lora_t + m0 * args.rank), 0, (int)(rows_a * rb), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsrc_r = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(args.lora_r + n0 * args.rank), 0, (int)(rows_b * rb), 0x00020000);
    const unsigned cb = (unsigned)(chunk * BK + 16 * lc);
    const unsigned oob = cb < (unsigned)rb ? 0u : kOutOfRange;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const bool spare = Cfg::kDummy && j >= ASL && grp[j] < 0;
      int8_t *dst = spare ? dummy : lora_stage + (j < ASL ? 0 : BM * BK) + grp[j] * 1024;
      const unsigned row = (unsigned)(8 * (grp[j] < 0 ? 0 : grp[j]) + (lane >> 3));
      const unsigned off = spare ? kOutOfRange : ((row * (unsigned)rb + cb) | oob);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(j < ASL ? rsrc_t : rsrc_r, (lds_void *)dst, 16, off, 0, 0, 0);
    }
  };
  // tile t of the loop, or LoRA chunk 0 in place of the first tile past K
  auto issue_next = [&](int t) {
    if constexpr (kLoraStaged) {
      if (t == nk) {
        issue_lora_loads(0);
        return;
      }
    }
    issue_loads(t);
  };
  // o += the LoRA term of the wavefront's blocks arow (tile rows of T) x brow
  // (tile rows of R).  `reload`: chunk 0 is no longer in the stage either (a
  // previous call used more than one chunk).  Every wavefront makes the same
  // calls: chunk loads end in a barrier.
  auto lora_term = [&](const auto &arow, const auto &brow, auto &o, bool reload) {
    const int nch = (args.rank + kLoraChunk - 1) / kLoraChunk;
    for (int c = 0; c < nch; ++c) {
      if (c > 0 || reload) {
        __syncthreads();  // every wavefront is done with the previous chunk
        issue_lora_loads(c);
        wait_loads_and_barrier<0>();
      }
      const int r = args.rank - c * kLoraChunk < kLoraChunk ? args.rank - c * kLoraChunk : kLoraChunk;
      lora_staged(lora_stage, BM * BK, BK, arow, brow, r, lane, o);
    }
  };

  // ---- fragment reads of k-step kk (0..3) of tile kt: lane l reads row (tile
  // row base + l % 32), logical chunk 2*kk + l / 32, stored at chunk ^ (l & 7)
  // (the row base is a multiple of 32).
  const int frow = (lane & 31) * BK;
  int fcol[kKSteps];
#pragma unroll
  for (int kk = 0; kk < kKSteps; ++kk) fcol[kk] = 16 * ((2 * kk + (lane >> 5)) ^ (lane & 7));
  struct Frags {
    v4i a[SM], b[SN];
  };
  Frags fkeep;
  auto read_frags = [&](int kt, int kk, Frags &f) {
    if constexpr (DIAG == 2) {
      if (kt > 0 || kk > 0) {
        f = fkeep;
        return;
      }
    }
    if constexpr (DIAG == 3) {
#pragma unroll
      for (int i = 0; i < SM; ++i) f.a[i] = v4i{kt, kk, i, 1};
#pragma unroll
      for (int j = 0; j < SN; ++j) f.b[j] = v4i{kk, kt, j, 3};
      return;
    }
    const int8_t *base = smem + (kt & (STAGES - 1)) * kStageBytes + frow + fcol[kk];
#pragma unroll
    for (int i = 0; i < SM; ++i) f.a[i] = *reinterpret_cast<const v4i *>(base + (wm * TM + i * 32) * BK);
#pragma unroll
    for (int j = 0; j < SN; ++j) f.b[j] = *reinterpret_cast<const v4i *>(base + BM * BK + (wn * TN + j * 32) * BK);
    if constexpr (DIAG == 2) fkeep = f;
  };

  typedef typename AccOf<FP8>::type AccT;
  AccT acc[SM][SN];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j) acc[i][j] = AccT{};

  // FP8: one MFMA per tile over both 16-byte halves (64 k positions)
  auto mfma8_all = [&](const Frags &f0, const Frags &f1) {
    if constexpr (FP8) {
#pragma unroll
      for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) {
          const v8i bv = __builtin_shufflevector(f0.b[j], f1.b[j], 0, 1, 2, 3, 4, 5, 6, 7);
          const v8i av = __builtin_shufflevector(f0.a[i], f1.a[i], 0, 1, 2, 3, 4, 5, 6, 7);
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[i][j], 0, 0, 0, 0, 0, 0);
        }
    }
  };
  auto mfma_all = [&](const Frags &f) {
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
      for (int j = 0; j < SN; ++j)
        if constexpr (!FP8) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  };

  // ---- pipeline: tile kt+1 lands in the other stage while tile kt is consumed.
  // Both stages are loaded first; at each k-tile's last step every wavefront
  // waits for tile kt+1 and for its own LDS reads of tile kt, meets the others at
  // the barrier, and loads tile kt+2 into the stage tile kt used.  Tiles past the
  // last one are issued too: every lane's offset is then out of range, so they
  // only write zeros into a free stage, and the loop body stays branch-free.
  auto sched = [&](int loads, int reads, int mfmas) {
#pragma unroll
    for (int u = 0; u < mfmas; ++u) {
      if (u < loads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 global->LDS load
      if (u < reads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // 1 MFMA
    }
  };
  auto wait_tile_and_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  issue_loads(0);
  issue_next(1);
  wait_loads_and_barrier<LPW>();
  Frags f0, f1;
  read_frags(0, 0, f0);

  if constexpr (FP8 && (BN == 320 || SM + SN > 6)) {
    // Ten accumulator tiles (or nine fragments per set) leave room for two
    // fragment sets: each FP8 MFMA
    // step (two k-steps, both 16-byte halves of 64 k positions) waits for its
    // own reads, and the other wavefront of the SIMD fills the gap.
    // Iteration kt: MFMA (kt,0..1) | read (kt,2..3), wait, barrier, load tile
    // kt+2 | MFMA (kt,2..3) | read (kt+1,0..1).
    constexpr int T = SM * SN;
    read_frags(0, 1, f1);
    for (int kt = 0; kt < nk; ++kt) {
      mfma8_all(f0, f1);
      sched(0, 0, T);
      read_frags(kt, 2, f0);
      read_frags(kt, 3, f1);
      wait_tile_and_barrier();
      issue_next(kt + 2);
      mfma8_all(f0, f1);
      sched(LPW, 0, T);
      read_frags(kt + 1, 0, f0);
      read_frags(kt + 1, 1, f1);
    }
  } else if constexpr (FP8) {
    // Iteration kt: read (kt,2..3) | MFMA (kt,0..1); wait, barrier, load tile
    // kt+2 | read (kt+1,0..1) | MFMA (kt,2..3).
    read_frags(0, 1, f1);
    constexpr int T = SM * SN, R = 2 * (SM + SN);
    for (int kt = 0; kt < nk; ++kt) {
      Frags g0, g1;
      read_frags(kt, 2, g0);
      read_frags(kt, 3, g1);
      mfma8_all(f0, f1);
#pragma unroll
      for (int u = 0; u < T; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x100, R / T, 0);                  // LDS reads
        if (u < R % T) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      // 1 MFMA
      }
      wait_tile_and_barrier();
      if constexpr (!kLoraStaged) {
        // interleaved by hand, as in the int8 loop: load u | its share of the
        // reads of (kt+1, 0..1) | MFMA u, nothing moved across
        const int8_t *rbase = smem + ((kt + 1) & (STAGES - 1)) * kStageBytes + frow;
        auto read_one = [&](int r) {  // fragment r % (SM + SN) of step r / (SM + SN)
          const int st = r / (SM + SN), q = r % (SM + SN);
          Frags &f = st == 0 ? f0 : f1;
          const int8_t *b = rbase + fcol[st];
          if (q < SM) f.a[q] = *reinterpret_cast<const v4i *>(b + (wm * TM + q * 32) * BK);
          else f.b[q - SM] = *reinterpret_cast<const v4i *>(b + BM * BK + (wn * TN + (q - SM) * 32) * BK);
        };
#pragma unroll
        for (int u = 0; u < T; ++u) {
          if (u < LPW) load_slot(kt + 2, u);
#pragma unroll
          for (int r = u * R / T; r < (u + 1) * R / T; ++r) read_one(r);
          const int i = u / SN, j = u % SN;
          const v8i bv = __builtin_shufflevector(g0.b[j], g1.b[j], 0, 1, 2, 3, 4, 5, 6, 7);
          const v8i av = __builtin_shufflevector(g0.a[i], g1.a[i], 0, 1, 2, 3, 4, 5, 6, 7);
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc[i][j], 0, 0, 0, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int u = T; u < LPW; ++u) load_slot(kt + 2, u);
      } else {
        issue_next(kt + 2);
        read_frags(kt + 1, 0, f0);
        read_frags(kt + 1, 1, f1);
        mfma8_all(g0, g1);
#pragma unroll
        for (int u = 0; u < T; ++u) {
          if (u < LPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);       // 1 global->LDS load
          __builtin_amdgcn_sched_group_barrier(0x100, R / T, 0);                // LDS reads
          if (u < R % T) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // 1 MFMA
        }
      }
    }
  } else {
    // Iteration kt: read (kt,1) | MFMA (kt,0); read (kt,2) | MFMA (kt,1);
    // read (kt,3) | MFMA (kt,2); wait, barrier, load tile kt+2 | read (kt+1,0) |
    // MFMA (kt,3).  Without LoRA operands to stage, the last step is interleaved
    // by hand, load u | read u | MFMA u with nothing moved across: left to the
    // compiler, every load and its address arithmetic came first, ahead of the
    // step's MFMAs (about 1 % on the MLP GEMMs).
    constexpr int T = SM * SN;
    constexpr bool kByHand = !kLoraStaged && DIAG == 0;
    auto ktile = [&](int kt, auto with_loads) {
      constexpr bool kLoads = decltype(with_loads)::value;
      read_frags(kt, 1, f1);
      mfma_all(f0);
      sched(0, SM + SN, T);
      read_frags(kt, 2, f0);
      mfma_all(f1);
      sched(0, SM + SN, T);
      read_frags(kt, 3, f1);
      mfma_all(f0);
      sched(0, SM + SN, T);
      wait_tile_and_barrier();
      if constexpr (kByHand) {
        const int8_t *rbase = smem + ((kt + 1) & (STAGES - 1)) * kStageBytes + frow + fcol[0];
        auto read_one = [&](int u) {  // fragment u of (kt+1, 0) into f0
          if (u < SM) f0.a[u] = *reinterpret_cast<const v4i *>(rbase + (wm * TM + u * 32) * BK);
          else f0.b[u - SM] = *reinterpret_cast<const v4i *>(rbase + BM * BK + (wn * TN + (u - SM) * 32) * BK);
        };
#pragma unroll
        for (int u = 0; u < T; ++u) {
          if (kLoads && u < LPW) load_slot(kt + 2, u);
          if (u < SM + SN) read_one(u);
          const int i = u / SN, j = u % SN;
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f1.b[j], f1.a[i], acc[i][j], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int u = T; u < LPW; ++u)
          if (kLoads) load_slot(kt + 2, u);
#pragma unroll
        for (int u = T; u < SM + SN; ++u) read_one(u);
      } else {
        if constexpr (DIAG == 0) issue_next(kt + 2);
        read_frags(kt + 1, 0, f0);
        mfma_all(f1);
        sched(LPW, SM + SN, T);
      }
    };
    if constexpr (kByHand) {
      // The last two k-tiles would only load zeros past K into the free stage:
      // they run as a copy of the loop body without the loads.
      int kt = 0;
      for (; kt < nk - 2; ++kt) ktile(kt, std::true_type{});
      for (; kt < nk; ++kt) ktile(kt, std::false_type{});
    } else {
      for (int kt = 0; kt < nk; ++kt) ktile(kt, std::true_type{});
    }
  }
  // Forward epilogue without LoRA: the tile's row and column scales are fetched
  // now, while the last MFMAs drain, rather than by each 32 x 32 tile as it is
  // dequantized.  Row scales go to registers; the column scales (BN / 4 lanes,
  // one float4 each) to an LDS area of their own, published by the epilogue's
  // first barrier.
  constexpr bool kScalesAhead = EPI == Epilogue::kForward && !LORA;
  float sxr[SM];
  if constexpr (kScalesAhead) {
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int64_t m = m0 + wm * TM + i * 32 + (lane & 31);
      sxr[i] = args.row_scale[m < M ? m : M - 1];
    }
    if (tid < BN / 4) {
      int64_t n = n0 + 4 * tid;
      n = n < N ? n : N - 4;  // N is a multiple of 16: a float4 is whole or past the end
      *reinterpret_cast<float4 *>(smem + Cfg::kScaleOff + 16 * tid) = *reinterpret_cast<const float4 *>(args.col_scale + n);
    }
  }
  // The zero-fill loads of the last iterations may still be landing in LDS.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ------------------------------------------------------------ epilogues --
  // Accumulator layout (32 x 32 tile, lane l, register r):
  //   token m = l % 32, output column n = 8 * (r / 4) + 4 * (l / 32) + r % 4.
  const int half = lane >> 5;

  // bf16 outputs leave through LDS (free once the k loop has ended), 128 rows at
  // a time, as whole row segments of BN * 2 bytes in 16-byte non-temporal
  // stores.  Written through, the output does not linger dirty in the caches to
  // be written back while the next kernel (the next layer's rotate+quantize)
  // streams its own data.  Rows are padded by 16 bytes, which spreads the 8-byte
  // writes of 16 consecutive rows over the banks.
  constexpr int kPitch = BN * 2 + 16;
  constexpr int kPassRows = BM / 2;
  constexpr int kRowChunks = BN / 8;
  static_assert(kPassRows * kPitch <= STAGES * kStageBytes, "staged half tile fits in the ring");
  static_assert(TM <= kPassRows, "a wavefront's rows lie in one pass");
  int8_t *const stage = smem;
  // stores the staged rows of pass `pass` (N is a multiple of 16, so a 16-byte
  // chunk is whole or past the end); consecutive lanes cover a row contiguously
  // All of a lane's LDS reads are issued before its first store, so their
  // latencies overlap instead of adding up chunk by chunk.
  constexpr int kStoreIters = kPassRows * kRowChunks / kThreads;
  static_assert(kPassRows * kRowChunks % kThreads == 0, "whole store rounds");
  auto store_pass = [&](int pass) {
    v4u v[kStoreIters];
#pragma unroll
    for (int u = 0; u < kStoreIters; ++u) {
      const int c = tid + u * kThreads, r = c / kRowChunks, k = c - r * kRowChunks;
      v[u] = *reinterpret_cast<const v4u *>(stage + r * kPitch + 16 * k);
    }
#pragma unroll
    for (int u = 0; u < kStoreIters; ++u) {
      const int c = tid + u * kThreads, r = c / kRowChunks, k = c - r * kRowChunks;
      const int64_t m = m0 + pass * kPassRows + r, n = n0 + 8 * k;
      if (m < M && n < N) __builtin_nontemporal_store(v[u], reinterpret_cast<v4u *>(args.out_bf16 + m * N + n));
    }
  };
  // a wavefront's packed outputs pk[i][j][q4]: tile row wm*TM + 32 i + lane % 32,
  // columns wn*TN + 32 j + 8 q4 + 4 half .. + 3
  auto stage_and_store = [&](const v2u (&pk)[SM][SN][4]) {
    __syncthreads();  // every wavefront is done with its last fragments
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if ((wm * TM) / kPassRows == pass) {
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
          for (int j = 0; j < SN; ++j)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
              *reinterpret_cast<v2u *>(stage + (wm * TM + i * 32 + (lane & 31) - pass * kPassRows) * kPitch +
                                       (wn * TN + j * 32 + 8 * q4 + 4 * half) * 2) = pk[i][j][q4];
      }
      __syncthreads();
      store_pass(pass);
      if (pass == 0) __syncthreads();  // the second half overwrites the staging area
    }
  };

  if constexpr (EPI == Epilogue::kInt32) {
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int64_t m = m0 + wm * TM + i * 32 + (lane & 31);
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < SN; ++j) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int64_t n = n0 + wn * TN + j * 32 + 8 * q4 + 4 * half;
          if (n < N) {
            v4i o;
            if constexpr (FP8) {  // the fp32 accumulators' bits
              o = v4i{__float_as_int(acc[i][j][4 * q4]), __float_as_int(acc[i][j][4 * q4 + 1]),
                      __float_as_int(acc[i][j][4 * q4 + 2]), __float_as_int(acc[i][j][4 * q4 + 3])};
            } else {
              o = v4i{acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]};
            }
            *reinterpret_cast<v4i *>(args.c_i32 + m * N + n) = o;
          }
        }
      }
    }
  } else if constexpr (EPI == Epilogue::kForward && LORA) {
    // dequantize every tile, add the LoRA term of all tiles together, then store
    v16f o[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int64_t m = m0 + wm * TM + i * 32 + (lane & 31);
      const float sx = args.row_scale[m < M ? m : M - 1];
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        const int64_t nb = n0 + wn * TN + j * 32 + 4 * half;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          int64_t n = nb + 8 * q4;
          n = n < N ? n : N - 4;
          const float4 sw = *reinterpret_cast<const float4 *>(args.col_scale + n);
          o[i][j][4 * q4 + 0] = acc_f32(acc[i][j][4 * q4 + 0]) * (sx * sw.x);
          o[i][j][4 * q4 + 1] = acc_f32(acc[i][j][4 * q4 + 1]) * (sx * sw.y);
          o[i][j][4 * q4 + 2] = acc_f32(acc[i][j][4 * q4 + 2]) * (sx * sw.z);
          o[i][j][4 * q4 + 3] = acc_f32(acc[i][j][4 * q4 + 3]) * (sx * sw.w);
        }
      }
    }
    {
      int arow[SM], brow[SN];
#pragma unroll
      for (int i = 0; i < SM; ++i) arow[i] = wm * TM + i * 32;
#pragma unroll
      for (int j = 0; j < SN; ++j) brow[j] = wn * TN + j * 32;
      lora_term(arow, brow, o, false);
    }
    v2u pk[SM][SN][4];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          pk[i][j][q4] = v2u{pack_bf16x2(o[i][j][4 * q4 + 0], o[i][j][4 * q4 + 1]),
                             pack_bf16x2(o[i][j][4 * q4 + 2], o[i][j][4 * q4 + 3])};
    stage_and_store(pk);
  } else if constexpr (EPI == Epilogue::kForward) {
    // Dequantized straight into the staging area, pass by pass (the wavefronts
    // of the other pass have nothing to keep in registers meanwhile).
    __syncthreads();  // every wavefront is done with its last fragments
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if ((wm * TM) / kPassRows == pass) {
#pragma unroll
        for (int i = 0; i < SM; ++i) {
          const int row = wm * TM + i * 32 + (lane & 31);
          const float sx = sxr[i];
#pragma unroll
          for (int j = 0; j < SN; ++j) {
            const int col = wn * TN + j * 32 + 4 * half;
            v16f o;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const float4 sw = *reinterpret_cast<const float4 *>(smem + Cfg::kScaleOff + 4 * (col + 8 * q4));
              o[4 * q4 + 0] = acc_f32(acc[i][j][4 * q4 + 0]) * (sx * sw.x);
              o[4 * q4 + 1] = acc_f32(acc[i][j][4 * q4 + 1]) * (sx * sw.y);
              o[4 * q4 + 2] = acc_f32(acc[i][j][4 * q4 + 2]) * (sx * sw.z);
              o[4 * q4 + 3] = acc_f32(acc[i][j][4 * q4 + 3]) * (sx * sw.w);
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const v2u packed{pack_bf16x2(o[4 * q4 + 0], o[4 * q4 + 1]), pack_bf16x2(o[4 * q4 + 2], o[4 * q4 + 3])};
              *reinterpret_cast<v2u *>(stage + (row - pass * kPassRows) * kPitch + (col + 8 * q4) * 2) = packed;
            }
            __builtin_amdgcn_sched_barrier(0);  // one 32 x 32 tile at a time: bounds register pressure
          }
        }
      }
      __syncthreads();
      store_pass(pass);
      if (pass == 0) __syncthreads();  // the second half overwrites the staging area
    }
  } else {
    // Backward.  A wavefront holds TN = 256 / WAVES_N consecutive output columns
    // of its tokens: column c = wn*TN + 32*j + 8*(r/4) + 4*half + (r%4) of the
    // tile, i.e. bits 0-1 = r%4, bit 2 = lane half, bits 3-4 = r/4, then j.
    // WAVES_M = 8: all 256 columns.  WAVES_M = 4 (4 x 2 wavefronts, the forward's
    // fragment traffic): 128 columns, enough for g <= 128.  Every stage runs in
    // the wavefront's registers.
    static_assert((WAVES_M == 8 && SN == 8) || (WAVES_M == 4 && SN == 4 && BN == 256 && G <= 128),
                  "backward epilogue: the rotation block lies within a wavefront's columns");
    v2u pk[SM][SN][4];
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int64_t m = m0 + wm * TM + i * 32 + (lane & 31);
      const int64_t mc = m < M ? m : M - 1;
      const float sdy = args.row_scale[mc];
      float z[SN][16];
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) z[j][r] = acc_f32(acc[i][j][r]) * sdy;

      if constexpr (G > 1) {
        // h = 1, 2: register bits 0-1
#pragma unroll
        for (int h = 1; h < 4; h <<= 1)
#pragma unroll
          for (int j = 0; j < SN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if ((r & h) == 0) {
                const float a = z[j][r], b = z[j][r + h];
                z[j][r] = a + b;
                z[j][r + h] = a - b;
              }
        // h = 4 is the lane half.  Swapping the high half of z[j] with the low
        // half of z[j^1] (v_permlane32_swap) puts both members of every h = 4 pair
        // into one lane: z[j] holds column bit 2 = 0 and z[j^1] bit 2 = 1, while
        // the lane half now selects j's bit 0.  Swapping again restores the layout.
#pragma unroll
        for (int j = 0; j < SN; j += 2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(z[j][r]), __float_as_uint(z[j + 1][r]),
                                                      false, false);
            z[j][r] = __uint_as_float(s[0]);
            z[j + 1][r] = __uint_as_float(s[1]);
          }
#pragma unroll
        for (int j = 0; j < SN; j += 2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float a = z[j][r], b = z[j + 1][r];
            z[j][r] = a + b;
            z[j + 1][r] = a - b;
          }
        // h = 8, 16: register bits (r / 4), valid in either layout
#pragma unroll
        for (int h = 4; h < 16; h <<= 1)
#pragma unroll
          for (int j = 0; j < SN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if ((r & h) == 0) {
                const float a = z[j][r], b = z[j][r + h];
                z[j][r] = a + b;
                z[j][r + h] = a - b;
              }
#pragma unroll
        for (int j = 0; j < SN; j += 2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(z[j][r]), __float_as_uint(z[j + 1][r]),
                                                      false, false);
            z[j][r] = __uint_as_float(s[0]);
            z[j + 1][r] = __uint_as_float(s[1]);
          }
        // h = 32, 64, 128: bits of j, up to g/2
#pragma unroll
        for (int hj = 1; hj < SN; hj <<= 1)
          if (32 * hj < G)
#pragma unroll
            for (int j = 0; j < SN; ++j)
              if ((j & hj) == 0)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const float a = z[j][r], b = z[j + hj][r];
                  z[j][r] = a + b;
                  z[j + hj][r] = a - b;
                }
        const float c = norm_const<G>();
#pragma unroll
        for (int j = 0; j < SN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) z[j][r] = z[j][r] * c;
      }

      v16f ot[1][SN];
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) ot[0][j][r] = z[j][r];
      if constexpr (LORA) {
        const int arow[1] = {wm * TM + i * 32};
        int brow[SN];
#pragma unroll
        for (int j = 0; j < SN; ++j) brow[j] = wn * TN + j * 32;
        lora_term(arow, brow, ot, i > 0 && args.rank > kLoraChunk);
      }
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        const v16f &o = ot[0][j];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          pk[i][j][q4] = v2u{pack_bf16x2(o[4 * q4 + 0], o[4 * q4 + 1]), pack_bf16x2(o[4 * q4 + 2], o[4 * q4 + 3])};
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    stage_and_store(pk);
  }
}

template <Epilogue EPI, int BN, int WAVES_M, int G, bool LORA, bool FP8 = false, int DIAG = 0>
hipError_t launch_typed(const GemmArgs &args, hipStream_t stream) {
  const int tiles_m = (int)((args.m + BM - 1) / BM);
  const int tiles_n = (int)((args.n + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_i8_kernel<EPI, BN, WAVES_M, G, LORA, FP8, DIAG>), dim3(tiles_m * tiles_n), dim3(kThreads),
                     0, stream, args, tiles_m, tiles_n);
  return hipGetLastError();
}

// Backward tiles: 4 x 2 wavefronts where the rotation block fits in a
// wavefront's 128 columns, else 8 x 1 (all 256 columns per wavefront).  The
// 4 x 2 layout at g = 256 with the h = 128 stage through LDS measured slower.
template <int G, bool FP8>
hipError_t launch_backward(const GemmArgs &args, hipStream_t stream) {
  constexpr int kWavesM = G <= 128 ? 4 : 8;
  return args.rank > 0 ? launch_typed<Epilogue::kBackward, 256, kWavesM, G, true, FP8>(args, stream)
                       : launch_typed<Epilogue::kBackward, 256, kWavesM, G, false, FP8>(args, stream);
}

template <bool FP8>
hipError_t launch_backward_any(const GemmArgs &args, hipStream_t stream) {
  switch (args.g) {
    case 1: return launch_backward<1, FP8>(args, stream);
    case 64: return launch_backward<64, FP8>(args, stream);
    case 128: return launch_backward<128, FP8>(args, stream);
    case 256: return launch_backward<256, FP8>(args, stream);
    default: return hipErrorInvalidValue;
  }
}

// Output tile width along N for the forward and int32 epilogues.  One workgroup
// fills a compute unit, so a launch runs in ceil(tiles / CUs) rounds, each as
// long as one tile (proportional to its width).  The width with the fewest
// column-rounds wins (ties go to 256): e.g. 4096 x 10240 takes 2 rounds of
// 256 x 320 tiles instead of 2.5 (so 3) of 256 x 256, and 4096 x 3072 one round
// of 256 x 192 instead of 0.75 of 256 x 256.  The same widths serve the FP8
// path (its 320-column tiles keep two fragment sets in flight instead of four).
int gemm_tile_n(int64_t m, int64_t n) {
  const int64_t cus = device_cu_count();
  const int64_t tiles_m = (m + BM - 1) / BM;
  auto cost = [&](int bn) { return (tiles_m * ((n + bn - 1) / bn) + cus - 1) / cus * bn; };
  int best = 256;
  for (int bn : {320, 192})
    if (cost(bn) < cost(best)) best = bn;
  return best;
}

template <Epilogue EPI, bool LORA>
hipError_t launch_forward_like(const GemmArgs &args, hipStream_t stream) {
  if (args.fp8) {
    switch (gemm_tile_n(args.m, args.n)) {
      case 320: return launch_typed<EPI, 320, 4, 1, LORA, true>(args, stream);
      case 192: return launch_typed<EPI, 192, 4, 1, LORA, true>(args, stream);
      default: return launch_typed<EPI, 256, 2, 1, LORA, true>(args, stream);
    }
  }
  switch (gemm_tile_n(args.m, args.n)) {
    case 320: return launch_typed<EPI, 320, 4, 1, LORA>(args, stream);
    case 192: return launch_typed<EPI, 192, 4, 1, LORA>(args, stream);
    default: return launch_typed<EPI, 256, 2, 1, LORA>(args, stream);
  }
}

template <int DIAG>
hipError_t launch_ceiling(const GemmArgs &args, hipStream_t stream) {
  switch (gemm_tile_n(args.m, args.n)) {
    case 320: return launch_typed<Epilogue::kForward, 320, 4, 1, false, false, DIAG>(args, stream);
    case 192: return launch_typed<Epilogue::kForward, 192, 4, 1, false, false, DIAG>(args, stream);
    default: return launch_typed<Epilogue::kForward, 256, 2, 1, false, false, DIAG>(args, stream);
  }
}

}  // namespace

hipError_t launch_gemm_i8_ceiling(const GemmArgs &args, int mode, hipStream_t stream) {
  switch (mode) {
    case 0: return launch_ceiling<0>(args, stream);
    case 1: return launch_ceiling<1>(args, stream);
    case 2: return launch_ceiling<2>(args, stream);
    case 3: return launch_ceiling<3>(args, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_i8(Epilogue epi, const GemmArgs &args, hipStream_t stream) {
  switch (epi) {
    case Epilogue::kInt32: return launch_forward_like<Epilogue::kInt32, false>(args, stream);
    case Epilogue::kForward:
      return args.rank > 0 ? launch_forward_like<Epilogue::kForward, true>(args, stream)
                           : launch_forward_like<Epilogue::kForward, false>(args, stream);
    case Epilogue::kBackward:
      return args.fp8 ? launch_backward_any<true>(args, stream) : launch_backward_any<false>(args, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace sdnq
