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
// Workgroup tile: 64 (a) x 64 (b) outputs, 4 wavefronts of 32 x 32 (2 x 2 MFMA
// 16x16 tiles); tokens are consumed 32 at a time through LDS.  The contraction
// runs over tokens, which are the slow index of both P and Q, so the MFMA
// operands (8 consecutive tokens of one column per lane) are gathered from the
// row-major LDS tiles with 16-bit reads.
constexpr int kGradTile = 64;
constexpr int kGradTokens = 32;
constexpr int kGradPad = 68;  // LDS row stride in bf16: 136 B keeps 8-byte stores aligned and puts rows 8 apart 16 banks apart
constexpr int kMaxSplits = 16;
constexpr int64_t kTokensPerSplit = 1024;

__global__ __launch_bounds__(256) void lora_grad_partial_kernel(const uint16_t *__restrict__ p, int64_t pa,
                                                                const uint16_t *__restrict__ q, int64_t qb,
                                                                int64_t m, int64_t tokens_per_split,
                                                                float *__restrict__ partials) {
  __shared__ uint16_t ps[kGradTokens][kGradPad];
  __shared__ uint16_t qs[kGradTokens][kGradPad];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t a0 = (int64_t)blockIdx.x * kGradTile;
  const int64_t b0 = (int64_t)blockIdx.y * kGradTile;
  const int split = blockIdx.z;
  const int64_t tb = split * tokens_per_split;
  int64_t te = tb + tokens_per_split;
  te = te < m ? te : m;

  // loader: each thread moves 8 bf16 of one token row of each tile
  const int lt = tid >> 3;        // token within the step, 0..31
  const int lcol = 8 * (tid & 7); // column within the tile, 0..56

  const int wa = wave & 1, wb = wave >> 1;
  v4f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v4f{};

  for (int64_t t0 = tb; t0 < te; t0 += kGradTokens) {
    const int64_t t = t0 + lt;
    uint4 pv = make_uint4(0u, 0u, 0u, 0u), qv = make_uint4(0u, 0u, 0u, 0u);
    if (t < te) {
      if (a0 + lcol < pa) pv = *reinterpret_cast<const uint4 *>(p + t * pa + a0 + lcol);
      if (b0 + lcol < qb) qv = *reinterpret_cast<const uint4 *>(q + t * qb + b0 + lcol);
    }
    __syncthreads();
    *reinterpret_cast<uint2 *>(&ps[lt][lcol]) = make_uint2(pv.x, pv.y);
    *reinterpret_cast<uint2 *>(&ps[lt][lcol + 4]) = make_uint2(pv.z, pv.w);
    *reinterpret_cast<uint2 *>(&qs[lt][lcol]) = make_uint2(qv.x, qv.y);
    *reinterpret_cast<uint2 *>(&qs[lt][lcol + 4]) = make_uint2(qv.z, qv.w);
    __syncthreads();
    // operands: lane l -> column (l % 16) of its 16-wide tile, tokens 8*(l/16) + 0..7
    const int tk = 8 * (lane >> 4);
    v8bf fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ca = wa * 32 + i * 16 + (lane & 15);
      const int cb = wb * 32 + i * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        fa[i][e] = __builtin_bit_cast(__bf16, ps[tk + e][ca]);
        fb[i][e] = __builtin_bit_cast(__bf16, qs[tk + e][cb]);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  }

  // acc[i][j] element e: a = a0 + wa*32 + i*16 + 4*(lane/16) + e, b = b0 + wb*32 + j*16 + lane%16
  float *dst = partials + (int64_t)split * pa * qb;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t b = b0 + wb * 32 + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t a = a0 + wa * 32 + i * 16 + 4 * (lane >> 4) + e;
        if (a < pa && b < qb) dst[a * qb + b] = acc[i][j][e];
      }
    }
}

__global__ void lora_grad_reduce_kernel(const float *__restrict__ partials, int splits, int64_t count, float scale,
                                        uint16_t *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float s = partials[i];
  for (int k = 1; k < splits; ++k) s += partials[(int64_t)k * count + i];
  const __bf16 b = (__bf16)(scale * s);
  out[i] = __builtin_bit_cast(uint16_t, b);
}

__global__ void fill_zero_u16_kernel(uint16_t *__restrict__ out, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) out[i] = 0;
}

// ---------------------------------------------------------- transposes --
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
                            float *partials, uint16_t *out, hipStream_t stream) {
  const int splits = lora_grad_splits(m);
  int64_t per = (m + splits - 1) / splits;
  per = (per + kGradTokens - 1) / kGradTokens * kGradTokens;
  const dim3 grid((unsigned)((pa + kGradTile - 1) / kGradTile), (unsigned)((qb + kGradTile - 1) / kGradTile),
                  (unsigned)splits);
  hipLaunchKernelGGL(lora_grad_partial_kernel, grid, dim3(256), 0, stream, p, pa, q, qb, m, per, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t count = pa * qb;
  hipLaunchKernelGGL(lora_grad_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream,
                     partials, splits, count, scale, out);
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
  const dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
  hipLaunchKernelGGL((transpose_kernel<uint16_t, 32>), grid, dim3(256), 0, stream, in, rows, cols, out);
  return hipGetLastError();
}

}  // namespace sdnq
