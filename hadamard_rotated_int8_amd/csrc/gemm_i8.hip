// G2: int8 x int8 -> int32 GEMM on gfx950 MFMA with fused epilogues.
//
//   acc[m, n] = sum_k A[m, k] * B[n, k]          (A, B int8, both K-contiguous)
//
// Forward ("SDNQ: SD.Next Quantization Engine": INT8 quantized matmul with a
// fused scale epilogue, FP32 dequantization as with dequantize_fp32):
//   y[m, n] = bf16( fp32(acc) * (row_scale[m] * col_scale[n])
//                   + lora_scale * sum_j T[m, j] * R[n, j] )
// Backward input (the quantized matmul of the training path): B is the
// transposed int8 weight, and
//   dx[m, :] = bf16( rot_g( fp32(acc[m, :]) * row_scale[m] ) + sum_j T[m, j] * R[:, j] )
// where rot_g is the normalized block Walsh-Hadamard rotation along the output
// columns (the same transform as the forward's, which is its own inverse).
//
// Tiling.  A workgroup of 4 wavefronts computes a 256 x 256 output tile; K is
// consumed 128 bytes at a time through a two-stage LDS ring (2 x 64 KB).  Each
// wavefront owns a (256/WAVES_M) x (256/WAVES_N) sub-tile made of 32 x 32 MFMA
// tiles (v_mfma_i32_32x32x32_i8, int32 accumulators in registers).  The MFMA
// "row" operand is the B side (weight rows, output column n) and the "column"
// operand the A side (tokens m), so each lane ends up holding, for one token,
// runs of 4 consecutive output columns: bf16 stores of 8 bytes.
//
// LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at chunk
// c ^ ((r >> 1) & 7), which makes both the 16-byte fragment reads (16 rows, one
// chunk) and the stores (2 rows, 8 chunks) conflict-free.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the block index is
// remapped so that each XCD walks a contiguous run of tiles, ordered in groups
// of 4 tile-rows, which keeps the tiles sharing A and B rows in one L2.
#include "sdnq_internal.hpp"

namespace sdnq {
namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kThreads = 256;
constexpr int kGroupM = 4;

constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;  // fl32(1/sqrt(128))

template <int G>
__device__ __forceinline__ float norm_const() {
  if constexpr (G == 64) return 0.125f;
  else if constexpr (G == 128) return kInvSqrt128;
  else if constexpr (G == 256) return 0.0625f;
  else return 1.0f;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + 16 * (chunk ^ ((row >> 1) & 7)); }

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

// One LoRA 32 x 32 output tile: out[i = n][j = m] = sum_r R[n, r] * T[m, r]
// (bf16 MFMA, fp32 accumulate).  Rows beyond the matrix are clamped (their
// results are never stored).
__device__ __forceinline__ v16f lora_tile(const uint16_t *__restrict__ T, const uint16_t *__restrict__ R,
                                          int64_t m, int64_t n, int rank, int lane) {
  v16f acc = {};
  const int koff = 8 * (lane >> 5);
  const uint16_t *tr = T + m * rank + koff;
  const uint16_t *rr = R + n * rank + koff;
  for (int k0 = 0; k0 < rank; k0 += 16) {
    const v8bf a = *reinterpret_cast<const v8bf *>(rr + k0);
    const v8bf b = *reinterpret_cast<const v8bf *>(tr + k0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
  return acc;
}

template <Epilogue EPI, int WAVES_M, int G>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_kernel(GemmArgs args, int tiles_m, int tiles_n) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  constexpr int SM = TM / 32, SN = TN / 32;
  static_assert(SM * SN == 16, "16 MFMA tiles per wavefront");

  __shared__ __attribute__((aligned(16))) int8_t smem[2][2][BM * BK];

  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int64_t M = args.m, N = args.n, K = args.k;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;

  // Global -> LDS assignment: 8 chunks of 16 B per operand per thread;
  // chunk id = it * 256 + tid -> tile row it * 32 + (tid >> 3), 16-byte column tid & 7.
  const int lrow = tid >> 3, lc = tid & 7;
  // Row offsets relative to the tile's first row (tail rows clamped to the last one;
  // their results are never stored).
  const int8_t *a_tile = args.a + m0 * K + 16 * lc;
  const int8_t *b_tile = args.b + n0 * K + 16 * lc;
  int a_off[8], b_off[8];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    int64_t ra = m0 + it * 32 + lrow;
    int64_t rb = n0 + it * 32 + lrow;
    ra = ra < M ? ra : M - 1;
    rb = rb < N ? rb : N - 1;
    a_off[it] = (int)((ra - m0) * K);
    b_off[it] = (int)((rb - n0) * K);
  }

  v4i ra[8], rb[8];
  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
    const bool ok = k0 + 16 * lc < K;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      ra[it] = ok ? *reinterpret_cast<const v4i *>(a_tile + a_off[it] + k0) : v4i{0, 0, 0, 0};
      rb[it] = ok ? *reinterpret_cast<const v4i *>(b_tile + b_off[it] + k0) : v4i{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int stage) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int off = swz(it * 32 + lrow, lc);
      *reinterpret_cast<v4i *>(&smem[stage][0][off]) = ra[it];
      *reinterpret_cast<v4i *>(&smem[stage][1][off]) = rb[it];
    }
  };

  v16i acc[SM][SN];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j) acc[i][j] = v16i{};

  const int nk = (int)((K + BK - 1) / BK);
  gload(0);
  sstore(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1);
    const int8_t *As = smem[kt & 1][0];
    const int8_t *Bs = smem[kt & 1][1];
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      const int ch = 2 * kk + (lane >> 5);
      v4i fa[SM], fb[SN];
#pragma unroll
      for (int i = 0; i < SM; ++i)
        fa[i] = *reinterpret_cast<const v4i *>(As + swz(wm * TM + i * 32 + (lane & 31), ch));
#pragma unroll
      for (int j = 0; j < SN; ++j)
        fb[j] = *reinterpret_cast<const v4i *>(Bs + swz(wn * TN + j * 32 + (lane & 31), ch));
#pragma unroll
      for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
    if (more) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogues --
  // Accumulator layout (32 x 32 tile, lane l, register r):
  //   token m = l % 32, output column n = 8 * (r / 4) + 4 * (l / 32) + r % 4.
  const int half = lane >> 5;
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
            v4i o = {acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]};
            *reinterpret_cast<v4i *>(args.c_i32 + m * N + n) = o;
          }
        }
      }
    }
  } else if constexpr (EPI == Epilogue::kForward) {
    const bool lora = args.rank > 0;
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int64_t m = m0 + wm * TM + i * 32 + (lane & 31);
      const int64_t mc = m < M ? m : M - 1;
      const float sx = args.row_scale[mc];
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        v16f l = {};
        if (lora) {
          int64_t nr = n0 + wn * TN + j * 32 + (lane & 31);
          nr = nr < N ? nr : N - 1;
          l = lora_tile(args.lora_t, args.lora_r, mc, nr, args.rank, lane);
        }
        if (m >= M) continue;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int64_t n = n0 + wn * TN + j * 32 + 8 * q4 + 4 * half;
          if (n < N) {
            const float4 sw = *reinterpret_cast<const float4 *>(args.col_scale + n);
            float o[4];
            o[0] = (float)acc[i][j][4 * q4 + 0] * (sx * sw.x);
            o[1] = (float)acc[i][j][4 * q4 + 1] * (sx * sw.y);
            o[2] = (float)acc[i][j][4 * q4 + 2] * (sx * sw.z);
            o[3] = (float)acc[i][j][4 * q4 + 3] * (sx * sw.w);
            if (lora) {
#pragma unroll
              for (int t = 0; t < 4; ++t) o[t] = __builtin_fmaf(args.lora_scale, l[4 * q4 + t], o[t]);
            }
            uint2 packed;
            packed.x = pack_bf16x2(o[0], o[1]);
            packed.y = pack_bf16x2(o[2], o[3]);
            *reinterpret_cast<uint2 *>(args.out_bf16 + m * N + n) = packed;
          }
        }
      }
    }
  } else {
    // Backward: WAVES_M = 4, so one wavefront holds all 256 output columns of
    // its 64 tokens: column c = 32*j + 8*(r/4) + 4*half + (r%4) of the tile,
    // i.e. bits 0-1 = r%4, bit 2 = lane half, bits 3-4 = r/4, bits 5-7 = j.
    static_assert(WAVES_M == 4 && SN == 8, "backward epilogue needs full-width wavefront tiles");
    const bool lora = args.rank > 0;
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int64_t m = m0 + wm * TM + i * 32 + (lane & 31);
      const int64_t mc = m < M ? m : M - 1;
      const float sdy = args.row_scale[mc];
      float z[SN][16];
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) z[j][r] = (float)acc[i][j][r] * sdy;

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

#pragma unroll
      for (int j = 0; j < SN; ++j) {
        v16f l = {};
        if (lora) {
          int64_t nr = n0 + j * 32 + (lane & 31);
          nr = nr < N ? nr : N - 1;
          l = lora_tile(args.lora_t, args.lora_r, mc, nr, args.rank, lane);
        }
        if (m >= M) continue;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int64_t n = n0 + j * 32 + 8 * q4 + 4 * half;
          if (n < N) {
            float o[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              o[t] = z[j][4 * q4 + t];
              if (lora) o[t] = __builtin_fmaf(args.lora_scale, l[4 * q4 + t], o[t]);
            }
            uint2 packed;
            packed.x = pack_bf16x2(o[0], o[1]);
            packed.y = pack_bf16x2(o[2], o[3]);
            *reinterpret_cast<uint2 *>(args.out_bf16 + m * N + n) = packed;
          }
        }
      }
    }
  }
}

template <Epilogue EPI, int WAVES_M, int G>
hipError_t launch_typed(const GemmArgs &args, hipStream_t stream) {
  const int tiles_m = (int)((args.m + BM - 1) / BM);
  const int tiles_n = (int)((args.n + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_i8_kernel<EPI, WAVES_M, G>), dim3(tiles_m * tiles_n), dim3(kThreads), 0, stream,
                     args, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_i8(Epilogue epi, const GemmArgs &args, hipStream_t stream) {
  switch (epi) {
    case Epilogue::kInt32: return launch_typed<Epilogue::kInt32, 2, 1>(args, stream);
    case Epilogue::kForward: return launch_typed<Epilogue::kForward, 2, 1>(args, stream);
    case Epilogue::kBackward:
      switch (args.g) {
        case 1: return launch_typed<Epilogue::kBackward, 4, 1>(args, stream);
        case 64: return launch_typed<Epilogue::kBackward, 4, 64>(args, stream);
        case 128: return launch_typed<Epilogue::kBackward, 4, 128>(args, stream);
        case 256: return launch_typed<Epilogue::kBackward, 4, 256>(args, stream);
        default: return hipErrorInvalidValue;
      }
  }
  return hipErrorInvalidValue;
}

}  // namespace sdnq
