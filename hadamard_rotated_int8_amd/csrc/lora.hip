// G3: the bf16 LoRA side path of the quantized linear layer ("ConvRot / Hadamard
// SDNQ", "PEFT Behavior": the adapter is trained in bf16 on top of the frozen
// int8 base) and small layout transposes.
//
//  - lora_down:  out[m, r] = bf16(scale * sum_c x[m, c] * R[r, c])
//                (t = x A with R = A^T, and g_r = scale * dY B^T with R = B);
//  - lora_grad:  out[a, b] = bf16(scale * sum_t P[t, a] * Q[t, b])
//                (dA = x^T g_r and dB = scale * t^T dY), reduced over tokens in
//                fixed-size splits whose fp32 partials are summed in split order.
// All products run on bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation.
#include "sdnq_internal.hpp"

namespace sdnq {
namespace {

// ----------------------------------------------------------- lora_down --
// A workgroup of 4 wavefronts handles 16*TT tokens; each wavefront takes a
// quarter of the contraction and keeps 16*TT x rank fp32 partial sums, which are
// added in wavefront order through LDS.  MFMA 16x16x32: row operand = R rows
// (rank index), column operand = x rows (token), so lane l owns token l % 16 and
// the four consecutive rank indices 4 * (l / 16) + 0..3 of each 16 x 16 tile.
// The contraction is walked in batches of 4 steps of 32 whose loads are all
// issued before the batch's MFMAs, so several steps of loads stay in flight.
constexpr int kMaxRank = 128;
constexpr int kDownBatch = 4;

template <int RT, int TT>  // RT = rank / 16, TT = tokens / 16
__global__ __launch_bounds__(256) void lora_down_kernel(const uint16_t *__restrict__ x, int64_t m, int64_t cols,
                                                        const uint16_t *__restrict__ rmat, float scale,
                                                        uint16_t *__restrict__ out) {
  __shared__ v4f red[4][TT][RT][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * (16 * TT);
  const int rank = RT * 16;

  // contraction range of this wavefront, in steps of 32
  const int64_t steps = (cols + 31) / 32;
  const int64_t per = (steps + 3) / 4;
  const int64_t c_begin = wave * per * 32;
  int64_t c_end = (wave + 1) * per * 32;
  c_end = c_end < cols ? c_end : cols;

  const int koff = 8 * (lane >> 4);
  const uint16_t *xr[TT];
#pragma unroll
  for (int s = 0; s < TT; ++s) {
    int64_t t = t0 + s * 16 + (lane & 15);
    t = t < m ? t : m - 1;
    xr[s] = x + t * cols + koff;
  }
  const uint16_t *rr[RT];
#pragma unroll
  for (int u = 0; u < RT; ++u) rr[u] = rmat + (int64_t)(u * 16 + (lane & 15)) * cols + koff;

  v4f acc[TT][RT];
#pragma unroll
  for (int s = 0; s < TT; ++s)
#pragma unroll
    for (int u = 0; u < RT; ++u) acc[s][u] = v4f{};

  for (int64_t cb = c_begin; cb < c_end; cb += 32 * kDownBatch) {
    v8bf bx[kDownBatch][TT], br[kDownBatch][RT];
#pragma unroll
    for (int b = 0; b < kDownBatch; ++b) {
      const int64_t c0 = cb + 32 * b;
      const bool ok = c0 < c_end && c0 + koff < cols;
#pragma unroll
      for (int s = 0; s < TT; ++s) bx[b][s] = ok ? *reinterpret_cast<const v8bf *>(xr[s] + c0) : v8bf{};
#pragma unroll
      for (int u = 0; u < RT; ++u) br[b][u] = ok ? *reinterpret_cast<const v8bf *>(rr[u] + c0) : v8bf{};
    }
#pragma unroll
    for (int b = 0; b < kDownBatch; ++b)
#pragma unroll
      for (int s = 0; s < TT; ++s)
#pragma unroll
        for (int u = 0; u < RT; ++u)
          acc[s][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(br[b][u], bx[b][s], acc[s][u], 0, 0, 0);
  }

#pragma unroll
  for (int s = 0; s < TT; ++s)
#pragma unroll
    for (int u = 0; u < RT; ++u) red[wave][s][u][lane] = acc[s][u];
  __syncthreads();
  // wavefront w writes token subtiles s = w, w + 4, ... (sums in wavefront order)
  for (int s = wave; s < TT; s += 4) {
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
        *reinterpret_cast<uint2 *>(out + t * rank + r0) = packed;
      }
    }
  }
}

// ----------------------------------------------------------- lora_grad --
// partial[split][a][b] = sum over the split's tokens t of P[t, a] * Q[t, b], with
// P the wide operand (x or dY: a over 3072-ish features) and Q the narrow one
// (g_r or t: b over the rank).  Workgroup tile: 128 (a) x 64 (b), 4 wavefronts
// of 32 (a) x 64 (b) (two v_mfma_f32_32x32x16_bf16 accumulators each), over one
// split of at most 1024 tokens, 64 tokens per step.
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
constexpr int64_t kTokensPerSplit = 1024;
static_assert(kGradBlocks % 4 == 0, "every wavefront issues the same number of loads");

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

__global__ __launch_bounds__(256) void lora_grad_partial_kernel(const uint16_t *__restrict__ p, int64_t pa,
                                                                const uint16_t *__restrict__ q, int64_t qb,
                                                                int64_t m, int64_t tokens_per_split,
                                                                float *__restrict__ partials) {
  constexpr int LPW = kGradBlocks / 4;  // loads per wavefront per step
  constexpr int PSUB = kGradA / 64;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kGradStages * kGradStageBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t a0 = (int64_t)blockIdx.x * kGradA;
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
// are [pa][qb]; out is [pa][qb], or [qb][pa] when transposed.
__global__ void lora_grad_reduce_kernel(const float *__restrict__ partials, int splits, int64_t pa, int64_t qb,
                                        float scale, int transposed, uint16_t *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // index into the partials
  const int64_t count = pa * qb;
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

// ---------------------------------------------------------- transposes --
// bf16 transpose of a rows x cols matrix whose sides are multiples of 8, in
// 64 x 64 tiles: 16-byte row chunks in, LDS with an 8-byte row pad, 16-byte
// column chunks (gathered 2 bytes at a time from LDS) out.
constexpr int kT16 = 64;
constexpr int kT16Pitch = kT16 + 4;  // in uint16

__global__ __launch_bounds__(256) void transpose_u16_kernel(const uint16_t *__restrict__ in, int64_t rows,
                                                            int64_t cols, uint16_t *__restrict__ out) {
  __shared__ __align__(16) uint16_t tile[kT16 * kT16Pitch];
  const int64_t r0 = (int64_t)blockIdx.y * kT16, c0 = (int64_t)blockIdx.x * kT16;
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

template <int TT>
hipError_t launch_lora_down_t(const uint16_t *x, int64_t m, int64_t cols, const uint16_t *rmat, int rank,
                              float scale, uint16_t *out, hipStream_t stream) {
  const dim3 grid((unsigned)((m + 16 * TT - 1) / (16 * TT)));
  switch (rank / 16) {
#define SDNQ_DOWN(RT)                                                                                         \
  case RT:                                                                                                    \
    hipLaunchKernelGGL((lora_down_kernel<RT, TT>), grid, dim3(256), 0, stream, x, m, cols, rmat, scale, out); \
    break;
    SDNQ_DOWN(1) SDNQ_DOWN(2) SDNQ_DOWN(3) SDNQ_DOWN(4) SDNQ_DOWN(5) SDNQ_DOWN(6) SDNQ_DOWN(7) SDNQ_DOWN(8)
#undef SDNQ_DOWN
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 64 tokens per workgroup when there are enough tokens to fill the chip that way
// (the rank x cols factor is then re-read from L2 half as often), else 32.
hipError_t launch_lora_down(const uint16_t *x, int64_t m, int64_t cols, const uint16_t *rmat, int rank,
                            float scale, uint16_t *out, hipStream_t stream) {
  if (m >= 16384) return launch_lora_down_t<4>(x, m, cols, rmat, rank, scale, out, stream);
  return launch_lora_down_t<2>(x, m, cols, rmat, rank, scale, out, stream);
}

int lora_grad_splits(int64_t m) {
  int64_t s = (m + kTokensPerSplit - 1) / kTokensPerSplit;
  if (s < 1) s = 1;
  if (s > kMaxSplits) s = kMaxSplits;
  return (int)s;
}

hipError_t launch_lora_grad(const uint16_t *p, int64_t pa, const uint16_t *q, int64_t qb, int64_t m, float scale,
                            bool transposed, float *partials, uint16_t *out, hipStream_t stream) {
  const int splits = lora_grad_splits(m);
  int64_t per = (m + splits - 1) / splits;
  per = (per + kGradTokens - 1) / kGradTokens * kGradTokens;
  const dim3 grid((unsigned)((pa + kGradA - 1) / kGradA), (unsigned)((qb + kGradB - 1) / kGradB), (unsigned)splits);
  hipLaunchKernelGGL(lora_grad_partial_kernel, grid, dim3(256), 0, stream, p, pa, q, qb, m, per, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t count = pa * qb;
  hipLaunchKernelGGL(lora_grad_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream,
                     partials, splits, pa, qb, scale, transposed ? 1 : 0, out);
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

hipError_t launch_transpose_u16(const uint16_t *in, int64_t rows, int64_t cols, uint16_t *out, hipStream_t stream) {
  if (rows % 8 == 0 && cols % 8 == 0) {
    const dim3 grid((unsigned)((cols + kT16 - 1) / kT16), (unsigned)((rows + kT16 - 1) / kT16));
    hipLaunchKernelGGL(transpose_u16_kernel, grid, dim3(256), 0, stream, in, rows, cols, out);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
  hipLaunchKernelGGL((transpose_kernel<uint16_t, 32>), grid, dim3(256), 0, stream, in, rows, cols, out);
  return hipGetLastError();
}

}  // namespace sdnq
