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
// 64-byte k-tile with fp32 accumulation, and the forward epilogue's scales.
// Its A and B fragments pair up 64 k positions of a tile the same way (the
// two 16-byte halves the int8 path reads for its two 32-deep steps), so the
// contraction is the full 64-k dot product.
//
// Tiling.  A workgroup of 8 wavefronts (two per SIMD, so one hides the other's
// waits) computes a 256 x 256 output tile; K is consumed 64 bytes at a time
// through a 4-stage LDS ring (4 x 32 KB) filled by buffer loads that write LDS
// directly, three k-tiles ahead.  Each wavefront owns a (256/WAVES_M) x
// (256/WAVES_N) sub-tile of eight 32 x 32 MFMA tiles (v_mfma_i32_32x32x32_i8,
// 128 int32 accumulators).  The MFMA
// "row" operand is the B side (weight rows, output column n) and the "column"
// operand the A side (tokens m), so each lane ends up holding, for one token,
// runs of 4 consecutive output columns: bf16 stores of 8 bytes.
//
// LDS rows are 64 bytes; the 16-byte chunk c of row r is stored at chunk
// c ^ ((r >> 2) & 3), which makes the 16-byte fragment reads (16 rows, one chunk)
// conflict-free (the bank-conflict counter reads zero).
//
// Workgroups are dispatched round-robin over the 8 XCDs; the block index is
// remapped so that each XCD walks a contiguous run of tiles, ordered in groups
// of 4 tile-rows, which keeps the tiles sharing A and B rows in one L2.
#include "sdnq_internal.hpp"

namespace sdnq {
namespace {

constexpr int BM = 256, BK = 64, STAGES = 4;
constexpr int kThreads = 512;  // 8 wavefronts: two per SIMD
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
// o[i][j] += sum_r R[nrow[j], r] * T[mrow[i], r], one 16-wide rank step at a
// time (bf16 MFMA 32x32x16, fp32 accumulate), with the next step's fragments
// loaded while this step's MFMAs run, so the loads of all tiles overlap instead
// of paying one memory round trip per tile.  Lane l holds row l % 32 of its
// tile and rank entries 8 * (l / 32) .. + 7 of each step.
template <int SM, int SN>
__device__ __forceinline__ void lora_all(const uint16_t *__restrict__ T, const uint16_t *__restrict__ R,
                                         const int64_t (&mrow)[SM], const int64_t (&nrow)[SN], int rank, int lane,
                                         v16f (&o)[SM][SN]) {
  const int koff = 8 * (lane >> 5);
  v8bf ta[SM], rb[SN];
#pragma unroll
  for (int i = 0; i < SM; ++i) ta[i] = *reinterpret_cast<const v8bf *>(T + mrow[i] * rank + koff);
#pragma unroll
  for (int j = 0; j < SN; ++j) rb[j] = *reinterpret_cast<const v8bf *>(R + nrow[j] * rank + koff);
  for (int k0 = 0; k0 < rank; k0 += 16) {
    const int kn = k0 + 16 < rank ? k0 + 16 : k0;  // the last step reloads its own fragments
    v8bf tn[SM], rn[SN];
#pragma unroll
    for (int i = 0; i < SM; ++i) tn[i] = *reinterpret_cast<const v8bf *>(T + mrow[i] * rank + kn + koff);
#pragma unroll
    for (int j = 0; j < SN; ++j) rn[j] = *reinterpret_cast<const v8bf *>(R + nrow[j] * rank + kn + koff);
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
      for (int j = 0; j < SN; ++j) o[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[j], ta[i], o[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < SM; ++i) ta[i] = tn[i];
#pragma unroll
    for (int j = 0; j < SN; ++j) rb[j] = rn[j];
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
// the B tile, rows of BK bytes, loaded in groups of 16 rows (1 KB, one
// direct-to-LDS load per wavefront).  The groups are dealt to the 8 wavefronts
// round-robin; when they do not divide evenly the spare slots load nothing (an
// out-of-range offset) into a 1 KB dummy area, so every wavefront issues the same
// number of loads and one vmcnt value fits all.
template <int BN_>
struct TileCfg {
  static constexpr int kStageBytes = (BM + BN_) * BK;
  static constexpr int kGroups = (BM + BN_) / 16;
  static constexpr int kLoadsPerWave = (kGroups + 7) / 8;
  static constexpr bool kDummy = kGroups % 8 != 0;
  static constexpr int kLdsBytes = STAGES * kStageBytes + (kDummy ? 1024 : 0);
  static_assert(BN_ % 32 == 0 && BM / 16 == 16, "A groups fill load slots 0 and 1");
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

template <Epilogue EPI, int BN, int WAVES_M, int G, bool LORA, bool FP8>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_kernel(GemmArgs args, int tiles_m, int tiles_n) {
  static_assert(!FP8 || EPI != Epilogue::kBackward, "FP8 runs the forward only");
  using Cfg = TileCfg<BN>;
  constexpr int kStageBytes = Cfg::kStageBytes;
  constexpr int LPW = Cfg::kLoadsPerWave;
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
  // A stage holds the A tile (256 rows x 64 B) then the B tile (BN rows).  Load
  // slot j of a wavefront fills the 16-row group 8*j + wave of the stage (slots
  // 0, 1: A groups; slots 2..: B groups): lane i lands at byte 16*i of that 1 KB
  // group, i.e. row 16*g + i/4, stored chunk i%4.  Rows are XOR-swizzled (stored
  // chunk = logical chunk ^ ((row >> 2) & 3)), so lane i fetches logical chunk
  // c = (i & 3) ^ ((i >> 4) & 3).  Rows past the matrix end lie past the
  // buffer's num_records and read as zero, and so do chunks past K (their offset
  // is pushed out of range).
  const int64_t rows_a = (M - m0) < BM ? (M - m0) : BM;
  const int64_t rows_b = (N - n0) < BN ? (N - n0) : BN;
  const __amdgpu_buffer_rsrc_t rsrc_a =
      __builtin_amdgcn_make_buffer_rsrc((void *)(args.a + m0 * K), 0, (int)(rows_a * K), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_b =
      __builtin_amdgcn_make_buffer_rsrc((void *)(args.b + n0 * K), 0, (int)(rows_b * K), 0x00020000);
  const int lc = (lane & 3) ^ ((lane >> 4) & 3);
  // per slot: row group within its operand, or -1 for a spare slot
  int grp[LPW];
  unsigned voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int g = 8 * j + wave;
    grp[j] = j < 2 ? g : (g - BM / 16 < BN / 16 ? g - BM / 16 : -1);
    voff[j] = (unsigned)((16 * (grp[j] < 0 ? 0 : grp[j]) + (lane >> 2)) * K + 16 * lc);
  }
  int8_t *const dummy = smem + STAGES * kStageBytes;

  const int nk = (int)((K + BK - 1) / BK);
  auto issue_loads = [&](int kt) {
    const int st = kt & (STAGES - 1);
    const unsigned k0 = (unsigned)kt * BK;
    // Only a k-tile that runs past K needs the per-lane range check.
    const unsigned oob = ((int64_t)k0 + BK <= K) ? 0u : (((int64_t)k0 + 16 * lc < K) ? 0u : kOutOfRange);
    int8_t *base = smem + st * kStageBytes;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      // wavefront-uniform selects, no branch: a spare slot loads nothing into the dummy area
      const bool spare = Cfg::kDummy && j >= 2 && grp[j] < 0;
      int8_t *dst = spare ? dummy : base + (j < 2 ? 0 : BM * BK) + grp[j] * 1024;
      const unsigned off = spare ? kOutOfRange : ((voff[j] + k0) | oob);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(j < 2 ? rsrc_a : rsrc_b, (lds_void *)dst, 16, off, 0, 0, 0);
    }
  };

  // ---- fragment reads: lane l reads row (tile row base + l % 32), logical chunk
  // 2*kk + l / 32, stored at chunk ^ ((l >> 2) & 3).
  const int frow = (lane & 31) * BK;
  const int fcol0 = 16 * ((0 + (lane >> 5)) ^ ((lane >> 2) & 3));
  const int fcol1 = 16 * ((2 + (lane >> 5)) ^ ((lane >> 2) & 3));
  struct Frags {
    v4i a[SM], b[SN];
  };
  auto read_frags = [&](int kt, int kk, Frags &f) {
    const int8_t *base = smem + (kt & (STAGES - 1)) * kStageBytes + frow + (kk ? fcol1 : fcol0);
#pragma unroll
    for (int i = 0; i < SM; ++i) f.a[i] = *reinterpret_cast<const v4i *>(base + (wm * TM + i * 32) * BK);
#pragma unroll
    for (int j = 0; j < SN; ++j) f.b[j] = *reinterpret_cast<const v4i *>(base + BM * BK + (wn * TN + j * 32) * BK);
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

  // ---- pipeline: tiles kt+1..kt+3 are in flight while tile kt is consumed.
  // Iteration kt: read (kt, kk=1) | MFMA (kt, kk=0) | wait for tile kt+1, barrier |
  // load tile kt+3 into the stage tile kt-1 used | read (kt+1, kk=0) | MFMA (kt, kk=1).
  // Tiles past the last one are issued too: every lane's offset is then out of
  // range, so they only write zeros into a free stage.  This keeps the loop body
  // branch-free and the number of loads in flight constant (4 per tile).
  for (int t = 0; t < STAGES - 1; ++t) issue_loads(t);
  wait_loads_and_barrier<2 * LPW>();
  Frags f0, f1;
  read_frags(0, 0, f0);

  if constexpr (FP8 && BN == 320) {
    // Ten accumulator tiles leave room for three fragment sets only.  Iteration
    // kt: read the second half of tile kt | wait for tile kt+1, barrier | load
    // tile kt+3 | read the first half of tile kt+1 | MFMA tile kt.
    for (int kt = 0; kt < nk; ++kt) {
      read_frags(kt, 1, f1);
      wait_loads_and_barrier<LPW>();
      issue_loads(kt + 3);
      Frags g0;
      read_frags(kt + 1, 0, g0);
      mfma8_all(f0, f1);
#pragma unroll
      for (int u = 0; u < SM * SN; ++u) {
        if (u < LPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // 1 global->LDS load
        if (u < SM + SN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // 1 MFMA
      }
      f0 = g0;
    }
  } else if constexpr (FP8) {
    // Iteration kt: wait for tile kt+1, barrier | load tile kt+3 | read both
    // halves of tile kt+1 | MFMA tile kt (both halves, read one iteration ago).
    read_frags(0, 1, f1);
    constexpr int R = 2 * (SM + SN);
    for (int kt = 0; kt < nk; ++kt) {
      wait_loads_and_barrier<LPW>();
      issue_loads(kt + 3);
      Frags g0, g1;
      read_frags(kt + 1, 0, g0);
      read_frags(kt + 1, 1, g1);
      mfma8_all(f0, f1);
#pragma unroll
      for (int u = 0; u < SM * SN; ++u) {
        if (u < LPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                      // 1 global->LDS load
        __builtin_amdgcn_sched_group_barrier(0x100, R / (SM * SN), 0);                    // LDS reads
        if (u < R % (SM * SN)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                   // 1 MFMA
      }
      f0 = g0;
      f1 = g1;
    }
  } else
  for (int kt = 0; kt < nk; ++kt) {
    read_frags(kt, 1, f1);
    mfma_all(f0);
#pragma unroll
    for (int u = 0; u < SM * SN; ++u) {
      if (u < SM + SN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // 1 MFMA
    }
    wait_loads_and_barrier<LPW>();
    issue_loads(kt + 3);
    read_frags(kt + 1, 0, f0);
    mfma_all(f1);
#pragma unroll
    for (int u = 0; u < SM * SN; ++u) {
      if (u < LPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // 1 global->LDS load
      if (u < SM + SN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // 1 MFMA
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
  auto store_pass = [&](int pass) {
    for (int c = tid; c < kPassRows * kRowChunks; c += kThreads) {
      const int r = c / kRowChunks, k = c - r * kRowChunks;
      const int64_t m = m0 + pass * kPassRows + r, n = n0 + 8 * k;
      if (m < M && n < N)
        __builtin_nontemporal_store(*reinterpret_cast<const v4u *>(stage + r * kPitch + 16 * k),
                                    reinterpret_cast<v4u *>(args.out_bf16 + m * N + n));
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
    int64_t mrow[SM], nrow[SN];
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int64_t m = m0 + wm * TM + i * 32 + (lane & 31);
      mrow[i] = m < M ? m : M - 1;
      const float sx = args.row_scale[mrow[i]];
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
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int64_t nr = n0 + wn * TN + j * 32 + (lane & 31);
      nrow[j] = nr < N ? nr : N - 1;
    }
    lora_all<SM, SN>(args.lora_t, args.lora_r, mrow, nrow, args.rank, lane, o);
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
          const int64_t m = m0 + row;
          const int64_t mc = m < M ? m : M - 1;
          const float sx = args.row_scale[mc];
#pragma unroll
          for (int j = 0; j < SN; ++j) {
            const int col = wn * TN + j * 32 + 4 * half;
            v16f o;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              int64_t n = n0 + col + 8 * q4;
              n = n < N ? n : N - 4;
              const float4 sw = *reinterpret_cast<const float4 *>(args.col_scale + n);
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
        const int64_t mrow[1] = {mc};
        int64_t nrow[SN];
#pragma unroll
        for (int j = 0; j < SN; ++j) {
          const int64_t nr = n0 + wn * TN + j * 32 + (lane & 31);
          nrow[j] = nr < N ? nr : N - 1;
        }
        lora_all<1, SN>(args.lora_t, args.lora_r, mrow, nrow, args.rank, lane, ot);
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

template <Epilogue EPI, int BN, int WAVES_M, int G, bool LORA, bool FP8 = false>
hipError_t launch_typed(const GemmArgs &args, hipStream_t stream) {
  const int tiles_m = (int)((args.m + BM - 1) / BM);
  const int tiles_n = (int)((args.n + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_i8_kernel<EPI, BN, WAVES_M, G, LORA, FP8>), dim3(tiles_m * tiles_n), dim3(kThreads), 0,
                     stream, args, tiles_m, tiles_n);
  return hipGetLastError();
}

// Backward tiles: 4 x 2 wavefronts where the rotation block fits in a
// wavefront's 128 columns, else 8 x 1 (all 256 columns per wavefront).  The
// 4 x 2 layout at g = 256 with the h = 128 stage through LDS measured slower.
template <int G>
hipError_t launch_backward(const GemmArgs &args, hipStream_t stream) {
  constexpr int kWavesM = G <= 128 ? 4 : 8;
  return args.rank > 0 ? launch_typed<Epilogue::kBackward, 256, kWavesM, G, true>(args, stream)
                       : launch_typed<Epilogue::kBackward, 256, kWavesM, G, false>(args, stream);
}

// Output tile width along N for the forward and int32 epilogues.  One workgroup
// fills a compute unit, so a launch runs in ceil(tiles / CUs) rounds, each as
// long as one tile (proportional to its width).  The width with the fewest
// column-rounds wins (ties go to 256): e.g. 4096 x 10240 takes 2 rounds of
// 256 x 320 tiles instead of 2.5 (so 3) of 256 x 256, and 4096 x 3072 one round
// of 256 x 192 instead of 0.75 of 256 x 256.
// (FP8 keeps two fragment sets of both halves live, which 320 columns do not fit.)
int gemm_tile_n(int64_t m, int64_t n, bool fp8) {
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
    switch (gemm_tile_n(args.m, args.n, true)) {
      case 320: return launch_typed<EPI, 320, 4, 1, LORA, true>(args, stream);
      case 192: return launch_typed<EPI, 192, 4, 1, LORA, true>(args, stream);
      default: return launch_typed<EPI, 256, 2, 1, LORA, true>(args, stream);
    }
  }
  switch (gemm_tile_n(args.m, args.n, false)) {
    case 320: return launch_typed<EPI, 320, 4, 1, LORA>(args, stream);
    case 192: return launch_typed<EPI, 192, 4, 1, LORA>(args, stream);
    default: return launch_typed<EPI, 256, 2, 1, LORA>(args, stream);
  }
}

}  // namespace

hipError_t launch_gemm_i8(Epilogue epi, const GemmArgs &args, hipStream_t stream) {
  switch (epi) {
    case Epilogue::kInt32: return launch_forward_like<Epilogue::kInt32, false>(args, stream);
    case Epilogue::kForward:
      return args.rank > 0 ? launch_forward_like<Epilogue::kForward, true>(args, stream)
                           : launch_forward_like<Epilogue::kForward, false>(args, stream);
    case Epilogue::kBackward:
      if (args.fp8) return hipErrorInvalidValue;
      switch (args.g) {
        case 1: return launch_backward<1>(args, stream);
        case 64: return launch_backward<64>(args, stream);
        case 128: return launch_backward<128>(args, stream);
        case 256: return launch_backward<256>(args, stream);
        default: return hipErrorInvalidValue;
      }
  }
  return hipErrorInvalidValue;
}

}  // namespace sdnq
