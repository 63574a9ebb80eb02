// G3: the bf16 LoRA side path of the quantized linear layer ("ConvRot / Hadamard
// SDNQ", "PEFT Behavior": the adapter is trained in bf16 on top of the frozen
// int8 base) and small layout transposes.
//
//  - lora_down:  out[m, r] = bf16(scale * sum_c x[m, c] * R[r, c])
//                (t = x A with R = A^T, and g_r = scale * dY B^T with R = B);
//  - lora_grad:  out[a, b] = bf16(scale * sum_t P[t, a] * Q[t, b])
//                (dA = x^T g_r and dB = scale * t^T dY), reduced over tokens in
//                equal splits whose fp32 partials are summed in split order.
// All products run on bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation.
#include "sdnq_internal.hpp"

namespace sdnq {
namespace {

// ----------------------------------------------------------- lora_down --
// A workgroup of 4 wavefronts handles 16*TT tokens; each wavefront takes a
// quarter of the contraction and keeps 16*TT x rank fp32 partial sums, which are
// added in wavefront order through LDS.
// MFMA 16x16x32: row operand = R rows (rank index), column operand = x rows
// (token), so lane l owns token l % 16 and the four consecutive rank indices
// 4 * (l / 16) + 0..3 of each 16 x 16 tile.  The contraction is walked in batches
// of 4 steps of 32 whose loads are all issued before the batch's MFMAs, so
// several steps of loads stay in flight.
constexpr int kMaxRank = 128;
constexpr int kDownBatch = 4;
typedef __attribute__((address_space(3))) void lds_void;

// One down-projection of a launch: out[m, r] = bf16(scale * x[m, :] . rmat[r, :]).
struct DownJob {
  const uint16_t *x;     // [m, cols]
  int64_t cols;
  const uint16_t *rmat;  // [rank, cols]
  float scale;
  uint16_t *out;         // row stride out_stride
  int64_t blocks;        // workgroups of this job
};

template <int RT, int TT>  // RT = rank / 16, TT = tokens / 16
__global__ __launch_bounds__(256) void lora_down_kernel(DownJob j0, DownJob j1, int64_t m, int64_t out_stride) {
  constexpr int TG = TT;  // 16-token subtiles
  __shared__ v4f red[4][TG][RT][64];
  // the first j0.blocks workgroups compute job 0, the others job 1
  const bool second = (int64_t)blockIdx.x >= j0.blocks;
  const uint16_t *__restrict__ x = second ? j1.x : j0.x;
  const int64_t cols = second ? j1.cols : j0.cols;
  const uint16_t *__restrict__ rmat = second ? j1.rmat : j0.rmat;
  const float scale = second ? j1.scale : j0.scale;
  uint16_t *__restrict__ out = second ? j1.out : j0.out;
  const int64_t blk = second ? blockIdx.x - j0.blocks : blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wq = wave;  // contraction quarter
  const int64_t t0 = blk * (16 * TT);

  // contraction range of this wavefront, in steps of 32
  const int64_t steps = (cols + 31) / 32;
  const int64_t per = (steps + 3) / 4;
  const int64_t c_begin = wq * per * 32;
  int64_t c_end = (wq + 1) * per * 32;
  c_end = c_end < cols ? c_end : cols;

  const int koff = 8 * (lane >> 4);
  const uint16_t *xr[TG];
#pragma unroll
  for (int s = 0; s < TG; ++s) {
    int64_t t = t0 + s * 16 + (lane & 15);
    t = t < m ? t : m - 1;
    xr[s] = x + t * cols + koff;
  }
  const uint16_t *rr[RT];
#pragma unroll
  for (int u = 0; u < RT; ++u) rr[u] = rmat + (int64_t)(u * 16 + (lane & 15)) * cols + koff;

  v4f acc[TG][RT];
#pragma unroll
  for (int s = 0; s < TG; ++s)
#pragma unroll
    for (int u = 0; u < RT; ++u) acc[s][u] = v4f{};

  for (int64_t cb = c_begin; cb < c_end; cb += 32 * kDownBatch) {
    v8bf bx[kDownBatch][TG], br[kDownBatch][RT];
#pragma unroll
    for (int b = 0; b < kDownBatch; ++b) {
      const int64_t c0 = cb + 32 * b;
      const bool ok = c0 < c_end && c0 + koff < cols;
#pragma unroll
      for (int s = 0; s < TG; ++s) bx[b][s] = ok ? *reinterpret_cast<const v8bf *>(xr[s] + c0) : v8bf{};
#pragma unroll
      for (int u = 0; u < RT; ++u) br[b][u] = ok ? *reinterpret_cast<const v8bf *>(rr[u] + c0) : v8bf{};
    }
#pragma unroll
    for (int b = 0; b < kDownBatch; ++b)
#pragma unroll
      for (int s = 0; s < TG; ++s)
#pragma unroll
        for (int u = 0; u < RT; ++u)
          acc[s][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(br[b][u], bx[b][s], acc[s][u], 0, 0, 0);
  }

#pragma unroll
  for (int s = 0; s < TG; ++s)
#pragma unroll
    for (int u = 0; u < RT; ++u) red[wq][s][u][lane] = acc[s][u];
  __syncthreads();
  // wavefront wq writes token subtiles s = wq, wq + 4, ... (sums in wavefront order)
  for (int s = wq; s < TG; s += 4) {
    const int64_t t = t0 + s * 16 + (lane & 15);
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      v4f sum = red[0][s][u][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) sum = sum + red[w][s][u][lane];
      if (t < m) {
        const int r0 = u * 16 + 4 * (lane >> 4);
        uint2 packed;
        packed.x = pack_bf16x2(scale * sum[0], scale * sum[1]);
        packed.y = pack_bf16x2(scale * sum[2], scale * sum[3]);
        *reinterpret_cast<uint2 *>(out + t * out_stride + r0) = packed;
      }
    }
  }
}

// ------------------------------------------------------ lora_down (staged) --
// The same projection with the contraction staged through LDS like the int8
// GEMM's: a workgroup of W wavefronts computes 32 W tokens x the whole rank
// slice (each wavefront 32 tokens x rank), 64 columns (128 bytes of every row)
// per k-tile.  A stage holds the x rows, then the rank rows of rmat, 128 bytes
// each, filled by direct-to-LDS buffer loads of 1 KB (8 rows) in a 3-stage
// ring; 16-byte chunk c of row r is stored at c ^ (r & 7).  Every load moves
// whole 128-byte lines.  W = 4 (the factor read once per 128 tokens) when that
// still gives every CU a workgroup, else W = 2.  With fewer tokens the
// register-loading kernel is used: one wavefront per workgroup could not hide
// the load latency (8192 x 3072, rank 32: 15.4 against 14.2 us), while at 16384
// tokens two wavefronts already win (rank 64: 20.3 against 28.6 us).
// MFMA 32x32x16 bf16: row operand = rmat rows (rank), column operand = x rows
// (tokens); lane l ends up with token l % 32 and ranks 8 (r / 4) + 4 (l / 32) +
// r % 4 of each 32-rank block.
constexpr int kStagedStages = 3;

// one 16-byte direct-to-LDS load per lane (a plain function: issued from the
// kernel template's lambda, the builtin kept the host pass from emitting the
// kernel's launch stub)
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, uint8_t *dst, unsigned off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, off, 0, 0, 0);
}

// RB = ceil(rank / 32) of the slice (1 .. 4; ranks past `rank` read zeros and are
// not stored); W = wavefronts, each 32 tokens
template <int RB, int W>
__global__ __launch_bounds__(64 * W) void lora_down_staged_kernel(DownJob j0, DownJob j1, int64_t m, int rank,
                                                                  int64_t out_stride) {
  constexpr int kStagedTokens = 32 * W;
  constexpr int kRows = kStagedTokens + 32 * RB;  // staged rows per k-tile
  constexpr int kStage = kRows * 128;
  constexpr int kLpw = kRows / 8 / W;             // 1 KB loads per wavefront per k-tile
  static_assert(kRows % (8 * W) == 0, "every wavefront issues the same number of loads");
  constexpr int kXGroups = kStagedTokens / 8;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStagedStages * kStage];
  const bool second = (int64_t)blockIdx.x >= j0.blocks;
  const uint16_t *x = second ? j1.x : j0.x;
  const int64_t cols = second ? j1.cols : j0.cols;
  const uint16_t *rmat = second ? j1.rmat : j0.rmat;
  const float scale = second ? j1.scale : j0.scale;
  uint16_t *__restrict__ out = second ? j1.out : j0.out;
  const int64_t blk = second ? blockIdx.x - j0.blocks : blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t t0 = blk * kStagedTokens;
  const int64_t rows_x = (m - t0) < kStagedTokens ? (m - t0) : kStagedTokens;
  const int64_t row_bytes = cols * 2;

  // slot j of wavefront w loads group g = W j + w: x rows 8 g .. (g < kXGroups),
  // else rmat rows 8 (g - kXGroups) ..; lane i lands at byte 16 i of the group:
  // row 8 g + i / 8, stored chunk i % 8, holding logical chunk (i & 7) ^ (i >> 3)
  const __amdgpu_buffer_rsrc_t rs_x =
      __builtin_amdgcn_make_buffer_rsrc((void *)(x + t0 * cols), 0, (int)(rows_x * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_r =
      __builtin_amdgcn_make_buffer_rsrc((void *)rmat, 0, (int)(rank * row_bytes), 0x00020000);
  const int lc = (lane & 7) ^ ((lane >> 3) & 7);
  unsigned voff[kLpw];
#pragma unroll
  for (int j = 0; j < kLpw; ++j) {
    const int g = W * j + wave;
    const int row = 8 * (g < kXGroups ? g : g - kXGroups) + (lane >> 3);
    voff[j] = (unsigned)(row * row_bytes + 16 * lc);
  }
  const int nk = (int)((row_bytes + 127) / 128);
  auto issue = [&](int kt) {
    const unsigned k0 = (unsigned)kt * 128;
    const unsigned oob = (int64_t)k0 + 16 * lc < row_bytes ? 0u : 0x80000000u;
    uint8_t *base = smem + (kt % kStagedStages) * kStage;
#pragma unroll
    for (int j = 0; j < kLpw; ++j) {
      const int g = W * j + wave;
      load_lds16(g < kXGroups ? rs_x : rs_r, base + g * 1024, (voff[j] + k0) | oob);
    }
  };

  // fragments of k-step kk (0..3): row (block base + l % 32), logical chunk
  // 2 kk + l / 32, stored at that ^ (l & 7)
  const int frow = (lane & 31) * 128;
  v16f acc[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) acc[j] = v16f{};
  issue(0);
  issue(1);
  for (int kt = 0; kt < nk; ++kt) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kLpw) : "memory");  // tile kt has landed
    __builtin_amdgcn_sched_barrier(0);
    issue(kt + 2);  // into the stage of tile kt - 1, which every wavefront has finished
    const uint8_t *base = smem + (kt % kStagedStages) * kStage + frow;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int col = 16 * ((2 * kk + (lane >> 5)) ^ (lane & 7));
      const v8bf xa = *reinterpret_cast<const v8bf *>(base + (32 * wave) * 128 + col);
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const v8bf rv = *reinterpret_cast<const v8bf *>(base + (kStagedTokens + 32 * j) * 128 + col);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rv, xa, acc[j], 0, 0, 0);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the zero-fill loads past the last tile

  const int64_t t = t0 + 32 * wave + (lane & 31);
  if (t < m) {
#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r0 = 32 * j + 8 * q + 4 * (lane >> 5);
        if (r0 < rank) {  // rank is a multiple of 16, so 4 ranks are all in or all out
          uint2 packed;
          packed.x = pack_bf16x2(scale * acc[j][4 * q], scale * acc[j][4 * q + 1]);
          packed.y = pack_bf16x2(scale * acc[j][4 * q + 2], scale * acc[j][4 * q + 3]);
          *reinterpret_cast<uint2 *>(out + t * out_stride + r0) = packed;
        }
      }
  }
}

// ----------------------------------------------------------- lora_grad --
// partial[split][a][b] = sum over the split's tokens t of P[t, a] * Q[t, b], with
// P the wide operand (x or dY: a over 3072-ish features) and Q the narrow one
// (g_r or t: b over the rank).  Workgroup tile: 128 (a) x 64 (b), 4 wavefronts
// of 32 (a) x 64 (b) (two v_mfma_f32_32x32x16_bf16 accumulators each), over one
// token split (lora_grad_splits), 64 tokens per step.
// The contraction runs over tokens, the slow index of both P and Q, so the
// tiles are staged row-major in LDS (direct-to-LDS buffer loads, a 3-stage
// ring) and the MFMA operands are read with ds_read_b64_tr_b16: within each group of
// 16 lanes, lane j supplies the address of 4 consecutive bf16 of token row
// (j / 4), column quad (j % 4), and lane l receives column (l % 16) of those 4
// token rows.  So lane l gets 4 consecutive tokens of one column, which is the
// operand layout (two reads give the 8 tokens of a 16-token MFMA step).
// LDS sub-tiles are 64 token rows x 64 columns (128-byte rows); 16-byte chunk c
// of row t is stored at chunk c ^ (t & 7) so the transposing reads spread over
// the banks.  The P tile is two such sub-tiles side by side (256 contiguous
// bytes of each token row), the Q tile one.
constexpr int kGradA = 128;  // P columns per workgroup
constexpr int kGradB = 64;   // Q columns per workgroup
constexpr int kGradTokens = 64;
constexpr int kGradStages = 3;
constexpr int kGradSub = kGradTokens * 64 * 2;               // one 64 x 64 bf16 sub-tile, 8 KB
constexpr int kGradStageBytes = (kGradA / 64 + 1) * kGradSub;  // P sub-tiles then the Q sub-tile
constexpr int kGradBlocks = kGradStageBytes / 1024;          // 1 KB direct loads per stage
constexpr int kMaxSplits = 16;
// Splits per launch: enough for about this many workgroups (1.5 per CU of a
// 256-CU chip).  On the 16384-token PEFT backward (48 column tiles) that is 8
// splits of 2048 tokens: 298 us for the whole backward against 313 us with 16
// splits of 1024 (a second, half-empty round of workgroups) and 302-314 us with
// 6, 5 or 4 longer splits.
constexpr int64_t kGradTargetBlocks = 384;
static_assert(kGradBlocks % 4 == 0, "every wavefront issues the same number of loads");

// One token reduction of a launch (P [m, pa], Q [m, qb], partials [splits, pa, qb]).
struct GradJob {
  const uint16_t *p;
  int64_t pa;
  const uint16_t *q;
  float *partials;
  int64_t tiles;  // column tiles of kGradA of this job
};
// and its final sum: out = bf16(scale * sum of the partials), [pa, qb] or transposed
struct ReduceJob {
  const float *partials;
  int64_t pa;
  float scale;
  int transposed;
  uint16_t *out;
  int64_t count;  // pa * qb
};

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

__global__ __launch_bounds__(256) void lora_grad_partial_kernel(GradJob j0, GradJob j1, int64_t qb, int64_t m,
                                                                int64_t tokens_per_split) {
  constexpr int LPW = kGradBlocks / 4;  // loads per wavefront per step
  constexpr int PSUB = kGradA / 64;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kGradStages * kGradStageBytes];
  // the first j0.tiles column tiles of the grid compute job 0, the others job 1
  const bool second = (int64_t)blockIdx.x >= j0.tiles;
  const uint16_t *__restrict__ p = second ? j1.p : j0.p;
  const int64_t pa = second ? j1.pa : j0.pa;
  const uint16_t *__restrict__ q = second ? j1.q : j0.q;
  float *__restrict__ partials = second ? j1.partials : j0.partials;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t a0 = (second ? blockIdx.x - j0.tiles : (int64_t)blockIdx.x) * kGradA;
  const int64_t b0 = (int64_t)blockIdx.y * kGradB;
  const int split = blockIdx.z;
  const int64_t tb = split * tokens_per_split;
  int64_t te = tb + tokens_per_split;
  te = te < m ? te : m;
  te = te > tb ? te : tb;  // an empty split reads nothing (num_records 0) and writes zeros
  const int nsteps = (int)((te - tb + kGradTokens - 1) / kGradTokens);

  // Loads: block B of a stage (1 KB = 8 token rows x 128 B of one sub-tile) is
  // issued by wavefront B % 4.  Blocks 0 .. 8*PSUB-1 are P (sub-tile B / 8), the
  // rest Q.  Lane i of a block lands in LDS slot i: row 8 * (B % 8) + i / 8,
  // stored chunk i % 8, which holds logical chunk (i % 8) ^ (row & 7).  Rows past
  // the split and columns past the matrix read as zero.
  const __amdgpu_buffer_rsrc_t rs_p = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(p + tb * pa), 0, (int)((te - tb) * pa * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_q = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(q + tb * qb), 0, (int)((te - tb) * qb * 2), 0x00020000);
  unsigned off[LPW];
  bool ok[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int blk = 4 * u + wave;
    const bool isp = blk < 8 * PSUB;
    const int row = 8 * (blk % 8) + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);
    const int64_t col = isp ? a0 + 64 * (blk / 8) + 8 * chunk : b0 + 8 * chunk;
    const int64_t width = isp ? pa : qb;
    ok[u] = col < width;
    off[u] = (unsigned)((row * width + col) * 2);
  }
  auto issue = [&](int step) {
    uint8_t *base = smem + (step % kGradStages) * kGradStageBytes;
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int blk = 4 * u + wave;
      const bool isp = blk < 8 * PSUB;
      const int64_t width = isp ? pa : qb;
      const unsigned step_off = (unsigned)((int64_t)step * kGradTokens * width * 2);
      const unsigned o = ok[u] ? off[u] + step_off : 0x80000000u;
      uint8_t *dst = base + blk * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isp ? rs_p : rs_q, (lds_void *)dst, 16, o, 0, 0, 0);
    }
  };

  // Transposing operand reads.  Wavefront w multiplies P columns 32 w .. 32 w + 31
  // (sub-tile w / 2) by all 64 Q columns.  Lane l, group G = l / 16, j = l % 16:
  // token row 8 * (G / 2) + 4 * h + j / 4 of the 16-token step, column quad
  // j % 4 of the 16 columns 16 * (G % 2) of a 32-column block.
  const int G = lane >> 4, jl = lane & 15;
  const int trow = 8 * (G >> 1) + (jl >> 2);
  const int qcol = 16 * (G & 1) + 4 * (jl & 3);
  const int pbyte = 2 * (32 * (wave & 1) + qcol);  // in the wavefront's P sub-tile
  const int psub = (wave >> 1) * kGradSub;
  auto tr_read = [&](const uint8_t *tile, int row, int cb) {
    const int addr = row * 128 + ((((cb >> 4) ^ (row & 7)) << 4) | (cb & 15));
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(tile + addr));
  };
  auto cat = [](v4s lo, v4s hi) {
    return __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  v16f acc[2] = {v16f{}, v16f{}};
#pragma unroll
  for (int t = 0; t < kGradStages - 1; ++t) issue(t);
  for (int step = 0; step < nsteps; ++step) {
    __builtin_amdgcn_sched_barrier(0);
    // the loads of the kGradStages - 2 later steps may still be in flight
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((kGradStages - 2) * LPW) : "memory");
    __builtin_amdgcn_sched_barrier(0);
    issue(step + kGradStages - 1);
    const uint8_t *tile = smem + (step % kGradStages) * kGradStageBytes;
    const uint8_t *tp = tile + psub;
    const uint8_t *tq = tile + PSUB * kGradSub;
#pragma unroll
    for (int kk = 0; kk < kGradTokens / 16; ++kk) {
      const int r0 = 16 * kk + trow;
      const v8bf av = cat(tr_read(tp, r0, pbyte), tr_read(tp, r0 + 4, pbyte));
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int qb2 = 2 * (32 * jb + qcol);
        const v8bf bv = cat(tr_read(tq, r0, qb2), tr_read(tq, r0 + 4, qb2));
        acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[jb], 0, 0, 0);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the zero-fill loads past the last step

  // acc[jb] element r: a = 32 w + 8*(r/4) + 4*(l/32) + r%4, b = 32 jb + l%32
  float *dst = partials + (int64_t)split * pa * qb;
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
    const int64_t b = b0 + 32 * jb + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t a = a0 + 32 * wave + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (a < pa && b < qb) dst[a * qb + b] = acc[jb][r];
    }
  }
}

// out = bf16(scale * sum over splits of partial), in split order; the partials
// are [pa][qb]; out is [pa][qb], or [qb][pa] when transposed.  Threads past job
// 0's count sum job 1.
__global__ void lora_grad_reduce_kernel(ReduceJob j0, ReduceJob j1, int splits, int64_t qb) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // index into the partials
  const bool second = i >= j0.count;
  if (second) i -= j0.count;
  const ReduceJob &j = second ? j1 : j0;
  const float *__restrict__ partials = j.partials;
  const int64_t pa = j.pa, count = j.count;
  const float scale = j.scale;
  const int transposed = j.transposed;
  uint16_t *__restrict__ out = j.out;
  if (i >= count) return;
  // all splits' loads in flight first (splits <= kMaxSplits, the same for every
  // lane), then the sum in split order
  float t[kMaxSplits];
#pragma unroll
  for (int k = 0; k < kMaxSplits; ++k) t[k] = k < splits ? partials[(int64_t)k * count + i] : 0.0f;
  float s = t[0];
#pragma unroll
  for (int k = 1; k < kMaxSplits; ++k)
    if (k < splits) s += t[k];
  const __bf16 b = (__bf16)(scale * s);
  out[transposed ? (i % qb) * pa + i / qb : i] = __builtin_bit_cast(uint16_t, b);
}

__global__ void fill_zero_u16_kernel(uint16_t *__restrict__ out, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) out[i] = 0;
}

// out[i, j] = in[i, j] inside in's [in_rows, in_cols], else 0, for out [out_rows, out_cols]:
// pads a LoRA factor with zero rows or columns, or crops a padded result.
__global__ void copy2d_u16_kernel(const uint16_t *__restrict__ in, int64_t in_rows, int64_t in_cols,
                                  uint16_t *__restrict__ out, int64_t out_rows, int64_t out_cols) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= out_rows * out_cols) return;
  const int64_t i = idx / out_cols, j = idx - i * out_cols;
  out[idx] = (i < in_rows && j < in_cols) ? in[i * in_cols + j] : (uint16_t)0;
}

// ---------------------------------------------------------- transposes --
// bf16 transpose of a rows x cols matrix whose sides are multiples of 8, in
// 64 x 64 tiles: 16-byte row chunks in, LDS with an 8-byte row pad, 16-byte
// column chunks (gathered 2 bytes at a time from LDS) out.
constexpr int kT16 = 64;
constexpr int kT16Pitch = kT16 + 4;  // in uint16

// One transpose of a launch (tiles = its 64 x 64 tiles, tiles_c of them per tile row).
struct TJob {
  const uint16_t *in;
  int64_t rows, cols;
  uint16_t *out;
  int64_t tiles_c, tiles;
};

// The first j0.tiles workgroups transpose job 0, the others job 1.
__global__ __launch_bounds__(256) void transpose_u16_kernel(TJob j0, TJob j1) {
  __shared__ __align__(16) uint16_t tile[kT16 * kT16Pitch];
  const bool second = (int64_t)blockIdx.x >= j0.tiles;
  const uint16_t *__restrict__ in = second ? j1.in : j0.in;
  uint16_t *__restrict__ out = second ? j1.out : j0.out;
  const int64_t rows = second ? j1.rows : j0.rows, cols = second ? j1.cols : j0.cols;
  const int64_t tiles_c = second ? j1.tiles_c : j0.tiles_c;
  const int64_t t = second ? blockIdx.x - j0.tiles : blockIdx.x;
  const int64_t r0 = (t / tiles_c) * kT16, c0 = (t % tiles_c) * kT16;
  const int tid = threadIdx.x;
  v4u v[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // item = (row, chunk of 8 columns)
    const int item = tid + 256 * i, r = item >> 3, ch = item & 7;
    const bool ok = r0 + r < rows && c0 + 8 * ch < cols;
    v[i] = ok ? *reinterpret_cast<const v4u *>(in + (r0 + r) * cols + c0 + 8 * ch) : v4u{};
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int item = tid + 256 * i, r = item >> 3, ch = item & 7;
    uint32_t *d = reinterpret_cast<uint32_t *>(tile + r * kT16Pitch + 8 * ch);
    d[0] = v[i][0];
    d[1] = v[i][1];
    d[2] = v[i][2];
    d[3] = v[i][3];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // item = (output row = input column c, chunk of 8 input rows)
    const int item = tid + 256 * i, c = item >> 3, ch = item & 7;
    if (c0 + c < cols && r0 + 8 * ch < rows) {
      v4u o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint16_t *src = tile + (8 * ch + 2 * w) * kT16Pitch + c;
        o[w] = (uint32_t)src[0] | ((uint32_t)src[kT16Pitch] << 16);
      }
      *reinterpret_cast<v4u *>(out + (c0 + c) * rows + r0 + 8 * ch) = o;
    }
  }
}

template <typename T, int TILE>
__global__ __launch_bounds__(256) void transpose_kernel(const T *__restrict__ in, int64_t rows, int64_t cols,
                                                        T *__restrict__ out) {
  __shared__ T tile[TILE][TILE + 1];
  const int64_t r0 = (int64_t)blockIdx.y * TILE, c0 = (int64_t)blockIdx.x * TILE;
  for (int idx = threadIdx.x; idx < TILE * TILE; idx += 256) {
    const int r = idx / TILE, c = idx % TILE;
    if (r0 + r < rows && c0 + c < cols) tile[r][c] = in[(r0 + r) * cols + c0 + c];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < TILE * TILE; idx += 256) {
    const int c = idx / TILE, r = idx % TILE;
    if (r0 + r < rows && c0 + c < cols) out[(c0 + c) * rows + r0 + r] = tile[r][c];
  }
}

// int8 transpose of a rows x cols matrix whose sides are multiples of 16, in
// 128 x 128 tiles: 16-byte row chunks in, LDS with a 4-byte row pad, 16-byte
// column chunks (gathered byte by byte from LDS) out.
constexpr int kT8 = 128;
constexpr int kT8Pitch = kT8 + 4;

__global__ __launch_bounds__(256) void transpose_i8_kernel(const int8_t *__restrict__ in, int64_t rows,
                                                           int64_t cols, int8_t *__restrict__ out) {
  __shared__ __align__(16) uint8_t tile[kT8 * kT8Pitch];
  const int64_t r0 = (int64_t)blockIdx.y * kT8, c0 = (int64_t)blockIdx.x * kT8;
  const int tid = threadIdx.x;
  v4u v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // item = (row, chunk of 16 columns)
    const int item = tid + 256 * i, r = item >> 3, ch = item & 7;
    const bool ok = r0 + r < rows && c0 + 16 * ch < cols;
    v[i] = ok ? *reinterpret_cast<const v4u *>(in + (r0 + r) * cols + c0 + 16 * ch) : v4u{};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int item = tid + 256 * i, r = item >> 3, ch = item & 7;
    uint32_t *d = reinterpret_cast<uint32_t *>(tile + r * kT8Pitch + 16 * ch);
    d[0] = v[i][0];
    d[1] = v[i][1];
    d[2] = v[i][2];
    d[3] = v[i][3];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // item = (output row = input column c, chunk of 16 input rows)
    const int item = tid + 256 * i, c = item >> 3, ch = item & 7;
    if (c0 + c < cols && r0 + 16 * ch < rows) {
      v4u o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint8_t *src = tile + (16 * ch + 4 * w) * kT8Pitch + c;
        o[w] = (uint32_t)src[0] | ((uint32_t)src[kT8Pitch] << 8) | ((uint32_t)src[2 * kT8Pitch] << 16) |
               ((uint32_t)src[3 * kT8Pitch] << 24);
      }
      *reinterpret_cast<v4u *>(out + (c0 + c) * rows + r0 + 16 * ch) = o;
    }
  }
}

__global__ __launch_bounds__(256) void transpose_scale_bf16_kernel(const uint16_t *__restrict__ in, int64_t rows,
                                                                   int64_t cols, float scale,
                                                                   uint16_t *__restrict__ out) {
  __shared__ uint16_t tile[32][33];
  const int64_t r0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 32;
  for (int idx = threadIdx.x; idx < 32 * 32; idx += 256) {
    const int r = idx / 32, c = idx % 32;
    if (r0 + r < rows && c0 + c < cols) {
      const float v = __uint_as_float((uint32_t)in[(r0 + r) * cols + c0 + c] << 16) * scale;
      tile[r][c] = __builtin_bit_cast(uint16_t, (__bf16)v);
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 32 * 32; idx += 256) {
    const int c = idx / 32, r = idx % 32;
    if (r0 + r < rows && c0 + c < cols) out[(c0 + c) * rows + r0 + r] = tile[r][c];
  }
}

}  // namespace

hipError_t launch_transpose_scale_bf16(const uint16_t *in, int64_t rows, int64_t cols, float scale, uint16_t *out,
                                       hipStream_t stream) {
  const dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
  hipLaunchKernelGGL(transpose_scale_bf16_kernel, grid, dim3(256), 0, stream, in, rows, cols, scale, out);
  return hipGetLastError();
}

template <int RB, int W>
hipError_t launch_lora_down_staged_t(DownJob j0, DownJob j1, int64_t m, int rank, int64_t out_stride,
                                     hipStream_t stream) {
  const int64_t per_job = (m + 32 * W - 1) / (32 * W);
  j0.blocks = per_job;
  j1.blocks = j1.x ? per_job : 0;
  hipLaunchKernelGGL((lora_down_staged_kernel<RB, W>), dim3((unsigned)(j0.blocks + j1.blocks)), dim3(64 * W), 0,
                     stream, j0, j1, m, rank, out_stride);
  return hipGetLastError();
}

template <int W>
hipError_t launch_lora_down_staged_w(DownJob j0, DownJob j1, int64_t m, int rank, int64_t out_stride,
                                     hipStream_t stream) {
  switch ((rank + 31) / 32) {
    case 1: return launch_lora_down_staged_t<1, W>(j0, j1, m, rank, out_stride, stream);
    case 2: return launch_lora_down_staged_t<2, W>(j0, j1, m, rank, out_stride, stream);
    case 3: return launch_lora_down_staged_t<3, W>(j0, j1, m, rank, out_stride, stream);
    case 4: return launch_lora_down_staged_t<4, W>(j0, j1, m, rank, out_stride, stream);
    default: return hipErrorInvalidValue;
  }
}

// Wavefronts per workgroup of the staged kernel: the most (4 or 2) that still
// give every CU a workgroup, or 0 when even 2 would not (the register kernel then).
int staged_waves(int64_t m, int64_t jobs) {
  const int64_t cus = device_cu_count();
  if (jobs * ((m + 127) / 128) >= cus) return 4;
  if (jobs * ((m + 63) / 64) >= cus) return 2;
  return 0;
}

template <int TT>
hipError_t launch_lora_down_t(DownJob j0, DownJob j1, int64_t m, int rank, int64_t out_stride, hipStream_t stream) {
  const int64_t per_job = (m + 16 * TT - 1) / (16 * TT);
  j0.blocks = per_job;
  j1.blocks = j1.x ? per_job : 0;
  const dim3 grid((unsigned)(j0.blocks + j1.blocks));
  switch (rank / 16) {
#define SDNQ_DOWN(RT)                                                                                        \
  case RT:                                                                                                   \
    hipLaunchKernelGGL((lora_down_kernel<RT, TT>), grid, dim3(256), 0, stream, j0, j1, m, out_stride);         \
    break;
    SDNQ_DOWN(1) SDNQ_DOWN(2) SDNQ_DOWN(3) SDNQ_DOWN(4) SDNQ_DOWN(5) SDNQ_DOWN(6) SDNQ_DOWN(7) SDNQ_DOWN(8)
#undef SDNQ_DOWN
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The staged kernel when its workgroups of 2 or 4 wavefronts fill the chip,
// else the register-loading one with 64 tokens per workgroup when that fills it
// (the rank x cols factor is then re-read from L2 half as often) or 32.  Ranks
// above kMaxRank run as launches over consecutive slices of at most kMaxRank
// rows of rmat, each writing its columns of out.
hipError_t launch_lora_down2(const uint16_t *x0, int64_t cols0, const uint16_t *rmat0, float scale0, uint16_t *out0,
                             const uint16_t *x1, int64_t cols1, const uint16_t *rmat1, float scale1, uint16_t *out1,
                             int64_t m, int rank, hipStream_t stream) {
  if (rank <= 0 || rank % 16) return hipErrorInvalidValue;
  for (int r0 = 0; r0 < rank; r0 += kMaxRank) {
    const int rr = rank - r0 < kMaxRank ? rank - r0 : kMaxRank;
    const DownJob j0{x0, cols0, rmat0 + (int64_t)r0 * cols0, scale0, out0 + r0, 0};
    const DownJob j1{x1, cols1, x1 ? rmat1 + (int64_t)r0 * cols1 : nullptr, scale1, x1 ? out1 + r0 : nullptr, 0};
    const int w = staged_waves(m, x1 ? 2 : 1);
    const hipError_t e = w == 4       ? launch_lora_down_staged_w<4>(j0, j1, m, rr, rank, stream)
                         : w == 2     ? launch_lora_down_staged_w<2>(j0, j1, m, rr, rank, stream)
                         : m >= 16384 ? launch_lora_down_t<4>(j0, j1, m, rr, rank, stream)
                                      : launch_lora_down_t<2>(j0, j1, m, rr, rank, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_lora_down(const uint16_t *x, int64_t m, int64_t cols, const uint16_t *rmat, int rank,
                            float scale, uint16_t *out, hipStream_t stream) {
  return launch_lora_down2(x, cols, rmat, scale, out, nullptr, 0, nullptr, 0.0f, nullptr, m, rank, stream);
}

int64_t lora_grad_tiles(int64_t pa0, int64_t pa1, int64_t qb) {
  return ((pa0 + kGradA - 1) / kGradA + (pa1 + kGradA - 1) / kGradA) * ((qb + kGradB - 1) / kGradB);
}

int lora_grad_splits(int64_t m, int64_t tiles) {
  int64_t s = tiles > 0 ? (kGradTargetBlocks + tiles - 1) / tiles : 1;
  const int64_t steps = (m + kGradTokens - 1) / kGradTokens;  // at least one 64-token step per split
  if (s > steps) s = steps;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_lora_grad2(const uint16_t *p0, int64_t pa0, const uint16_t *q0, float scale0, bool transposed0,
                             float *partials0, uint16_t *out0, const uint16_t *p1, int64_t pa1, const uint16_t *q1,
                             float scale1, bool transposed1, float *partials1, uint16_t *out1, int64_t qb, int64_t m,
                             int splits, hipStream_t stream) {
  if (splits < 1 || splits > kMaxSplits) return hipErrorInvalidValue;
  int64_t per = (m + splits - 1) / splits;
  per = (per + kGradTokens - 1) / kGradTokens * kGradTokens;
  const GradJob g0{p0, pa0, q0, partials0, (pa0 + kGradA - 1) / kGradA};
  const GradJob g1{p1, pa1, q1, partials1, p1 ? (pa1 + kGradA - 1) / kGradA : 0};
  const dim3 grid((unsigned)(g0.tiles + g1.tiles), (unsigned)((qb + kGradB - 1) / kGradB), (unsigned)splits);
  hipLaunchKernelGGL(lora_grad_partial_kernel, grid, dim3(256), 0, stream, g0, g1, qb, m, per);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const ReduceJob r0{partials0, pa0, scale0, transposed0 ? 1 : 0, out0, pa0 * qb};
  const ReduceJob r1{partials1, pa1, scale1, transposed1 ? 1 : 0, out1, p1 ? pa1 * qb : 0};
  const int64_t count = r0.count + r1.count;
  hipLaunchKernelGGL(lora_grad_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, r0, r1,
                     splits, qb);
  return hipGetLastError();
}

hipError_t launch_lora_grad(const uint16_t *p, int64_t pa, const uint16_t *q, int64_t qb, int64_t m, float scale,
                            bool transposed, float *partials, uint16_t *out, int splits, hipStream_t stream) {
  return launch_lora_grad2(p, pa, q, scale, transposed, partials, out, nullptr, 0, nullptr, 0.0f, false, nullptr,
                           nullptr, qb, m, splits, stream);
}

hipError_t launch_copy2d_u16(const uint16_t *in, int64_t in_rows, int64_t in_cols, uint16_t *out, int64_t out_rows,
                             int64_t out_cols, hipStream_t stream) {
  const int64_t count = out_rows * out_cols;
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy2d_u16_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, in, in_rows,
                     in_cols, out, out_rows, out_cols);
  return hipGetLastError();
}

hipError_t launch_fill_zero_u16(uint16_t *out, int64_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_u16_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, out, count);
  return hipGetLastError();
}

hipError_t launch_transpose_i8(const int8_t *in, int64_t rows, int64_t cols, int8_t *out, hipStream_t stream) {
  if (rows % 16 || cols % 16) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((cols + kT8 - 1) / kT8), (unsigned)((rows + kT8 - 1) / kT8));
  hipLaunchKernelGGL(transpose_i8_kernel, grid, dim3(256), 0, stream, in, rows, cols, out);
  return hipGetLastError();
}

hipError_t launch_transpose_u16_pair(const uint16_t *in0, int64_t rows0, int64_t cols0, uint16_t *out0,
                                     const uint16_t *in1, int64_t rows1, int64_t cols1, uint16_t *out1,
                                     hipStream_t stream) {
  if (rows0 % 8 || cols0 % 8 || (in1 && (rows1 % 8 || cols1 % 8))) return hipErrorInvalidValue;
  TJob j0{in0, rows0, cols0, out0, (cols0 + kT16 - 1) / kT16, 0};
  j0.tiles = j0.tiles_c * ((rows0 + kT16 - 1) / kT16);
  TJob j1{in1, rows1, cols1, out1, in1 ? (cols1 + kT16 - 1) / kT16 : 1, 0};
  j1.tiles = in1 ? j1.tiles_c * ((rows1 + kT16 - 1) / kT16) : 0;
  if (j0.tiles + j1.tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_u16_kernel, dim3((unsigned)(j0.tiles + j1.tiles)), dim3(256), 0, stream, j0, j1);
  return hipGetLastError();
}

hipError_t launch_transpose_u16(const uint16_t *in, int64_t rows, int64_t cols, uint16_t *out, hipStream_t stream) {
  if (rows % 8 == 0 && cols % 8 == 0)
    return launch_transpose_u16_pair(in, rows, cols, out, nullptr, 0, 0, nullptr, stream);
  const dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
  hipLaunchKernelGGL((transpose_kernel<uint16_t, 32>), grid, dim3(256), 0, stream, in, rows, cols, out);
  return hipGetLastError();
}

}  // namespace sdnq
