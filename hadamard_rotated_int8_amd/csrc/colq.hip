// Rotate + quantize along the tokens, reading the tokens-major matrix directly.
//
// The weight gradient dW = dY^T x contracts over the tokens, so each operand is
// quantized per feature with the rotation block g running along the tokens: the
// rows of X^T [f, m] go through the same steps as any activation row (butterfly
// stages h = 1 .. g/2 with (a+b, a-b) in binary32, a multiply by fl32(1/sqrt(g)),
// a = max |y| over the row, s = fl32(a/127), r = fl32(127/a) with rows below
// 2^-100 first scaled by 2^100, code = round-half-even(fl32(y*r)) clamped to
// +-127).  These kernels read X [m, f] as it is and write the codes transposed,
// [f, m], without materializing X^T: pass 1 forms each feature's rotated absmax
// (an atomic max on the binary32 bits), pass 2 recomputes the same rotated
// values and writes codes and scales.
//
// A workgroup owns a tile of 256 tokens x 64 features (256 rows of 128 bytes).
// Each thread reads an 8-token x 8-feature block (eight 16-byte loads; eight
// neighbouring lanes read one row's whole 128 bytes), transposes it in registers
// and writes it as eight 16-byte units of a feature-major [64][256] LDS tile.
// Lane l of wavefront w then reads feature 16 w + l / 4, tokens 64 (l % 4) .. + 63,
// as eight 16-byte LDS reads: butterfly stages h = 1 .. 32 run inside the lane's
// registers, h = 64 and 128 pair lanes l ^ 1 and l ^ 2 (one DPP move each).  The
// tile's 16-byte units are XOR-swizzled so that the writes and the reads of eight
// neighbouring lanes land on distinct LDS banks.  In pass 2 each lane writes its
// 64 codes as four 16-byte stores.
#include "sdnq_internal.hpp"

namespace sdnq {
namespace {

constexpr int kTok = 256;    // tokens per tile
constexpr int kFeat = 64;    // features per tile
constexpr int kVals = 64;    // rotated values per lane (one feature, 64 tokens)
constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;  // fl32(1/sqrt(128))

template <int G>
__device__ __forceinline__ float norm_const() {
  if constexpr (G == 64) return 0.125f;
  else if constexpr (G == 128) return kInvSqrt128;
  else if constexpr (G == 256) return 0.0625f;
  else return 1.0f;
}

// Physical 16-byte unit (8 tokens) of logical unit u in feature row fl of the tile.
__device__ __forceinline__ int tile_unit(int u, int fl) {
  const int swz = (fl ^ (fl >> 3)) & 7;
  return u ^ ((((u >> 3) << 1) ^ swz) & 7);
}

// quad_perm lane swaps: [1,0,3,2] (lane ^ 1) and [2,3,0,1] (lane ^ 2)
template <int CTRL>
__device__ __forceinline__ float dpp_swap(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// One butterfly stage across lane pairs (lane ^ 1 or lane ^ 2).  Each lane keeps
// acc with y = sigma * acc, sigma = +-1 per lane.  The lower lane of a pair needs
// y + y_p = sigma (acc + sigma sigma_p acc_p), the upper one y_p - y =
// -sigma (acc - sigma sigma_p acc_p): one multiply-add of the partner's acc by
// +-1 (rounded once, as the sum or difference), and a sign that the lane carries.
template <int CTRL, int BIT>
__device__ __forceinline__ void pair_stage(float (&v)[kVals], float &sigma, int b) {
  const float partner_sigma = dpp_swap<CTRL>(sigma);
  const bool upper = (b & BIT) != 0;
  const float mul = upper ? -(sigma * partner_sigma) : sigma * partner_sigma;
#pragma unroll
  for (int i = 0; i < kVals; ++i) v[i] = fmaf(dpp_swap<CTRL>(v[i]), mul, v[i]);
  if (upper) sigma = -sigma;
}

// The lane's values before the normalization: y = sigma * v[i] is the butterfly
// output of feature f0 + 16 w + l/4, token t0 + 64 (l%4) + i.  Tokens past m and
// features past f read as zero.  Every thread reaches the barrier.
template <int G>
__device__ __forceinline__ void load_rotate(const uint16_t *__restrict__ x, int64_t m, int64_t f, int64_t t0,
                                            int64_t f0, uint16_t *tile, float (&v)[kVals], float &sigma) {
  const int t = threadIdx.x;
  {
    // Thread t: tokens 8 (t/8) .. + 7 (one 16-byte unit of every feature row of the
    // tile) and features 8 (t%8) .. + 7; the eight lanes of one row read its whole
    // 128 bytes.  The 8 x 8 block is transposed in registers and leaves as eight
    // 16-byte LDS writes.
    const int chunk = t & 7, u = t >> 3;
    const int64_t rows = m - t0 < kTok ? m - t0 : kTok;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(x + t0 * f + f0), 0, (int)(rows * f * 2), 0x00020000);
    const bool feat_ok = f0 + 8 * chunk < f;  // f is a multiple of 16: a chunk is whole or absent
    v4u raw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const unsigned off = feat_ok ? (unsigned)(((8 * u + j) * f + 8 * chunk) * 2) : 0x80000000u;
      raw[j] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // tokens (2p, 2p+1) of feature 8 chunk + e: halves e%2 of dword e/2 of rows 2p, 2p+1
      const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
      v4u out;
#pragma unroll
      for (int p = 0; p < 4; ++p) out[p] = __builtin_amdgcn_perm(raw[2 * p + 1][e >> 1], raw[2 * p][e >> 1], sel);
      const int fl = 8 * chunk + e;
      *reinterpret_cast<v4u *>(tile + fl * kTok + 8 * tile_unit(u, fl)) = out;
    }
  }
  __syncthreads();
  const int lane = t & 63, fl = 16 * (t >> 6) + (lane >> 2), b = lane & 3;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const v4u r = *reinterpret_cast<const v4u *>(tile + fl * kTok + 8 * tile_unit(8 * b + j, fl));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * j + 2 * i] = bf16_lo(r[i]);
      v[8 * j + 2 * i + 1] = bf16_hi(r[i]);
    }
  }
  sigma = 1.0f;
#pragma unroll
  for (int h = 1; h < (G < kVals ? G : kVals); h <<= 1)
#pragma unroll
    for (int i = 0; i < kVals; ++i)
      if (!(i & h)) {
        const float a = v[i], c = v[i + h];
        v[i] = a + c;
        v[i + h] = a - c;
      }
  if constexpr (G >= 128) pair_stage<0xB1, 1>(v, sigma, b);  // h = 64
  if constexpr (G >= 256) pair_stage<0x4E, 2>(v, sigma, b);  // h = 128
}

struct ColqOperand {
  const uint16_t *x;  // [m, f] bf16
  int64_t f;
  int64_t blocks;     // feature tiles of this operand
  uint32_t *colmax;   // [f] binary32 bits, zero before pass 1
  int8_t *q;          // [f, m]
  float *scale;       // [f]
};

// Pass 1: a = max over the tokens of |y| = |fl32(sigma acc c)|.  Rounding is
// monotone, so max fl32(|acc| c) = fl32(max |acc| * c): one multiply per lane.
template <int G>
__global__ __launch_bounds__(256) void colq_absmax_kernel(ColqOperand op0, ColqOperand op1, int64_t m) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kFeat * kTok];
  const bool second = blockIdx.x >= op0.blocks;
  const ColqOperand &op = second ? op1 : op0;
  const int64_t f0 = ((int64_t)blockIdx.x - (second ? op0.blocks : 0)) * kFeat, t0 = (int64_t)blockIdx.y * kTok;
  float v[kVals], sigma;
  load_rotate<G>(op.x, m, op.f, t0, f0, tile, v, sigma);
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < kVals; ++i) a = fmaxf(a, fabsf(v[i]));
  if constexpr (G > 1) a = a * norm_const<G>();
  a = fmaxf(a, dpp_swap<0xB1>(a));
  a = fmaxf(a, dpp_swap<0x4E>(a));
  const int lane = threadIdx.x & 63;
  const int64_t feat = f0 + 16 * (threadIdx.x >> 6) + (lane >> 2);
  if ((lane & 3) == 0 && feat < op.f) atomicMax(op.colmax + feat, __float_as_uint(a));
}

// Pass 2: codes.  fl32(y * r) + 1.5 * 2^23 rounds to the nearest integer, ties to
// even, and |fl32(y * r)| < 127.5 (y <= a, r <= 127/a rounded up by half an ulp),
// so the low byte of the sum's bits is the code, already within +-127.
template <int G>
__global__ __launch_bounds__(256) void colq_quantize_kernel(ColqOperand op0, ColqOperand op1, int64_t m) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kFeat * kTok];
  const bool second = blockIdx.x >= op0.blocks;
  const ColqOperand &op = second ? op1 : op0;
  const int64_t f0 = ((int64_t)blockIdx.x - (second ? op0.blocks : 0)) * kFeat, t0 = (int64_t)blockIdx.y * kTok;
  const int lane = threadIdx.x & 63, b = lane & 3;
  const int64_t feat = f0 + 16 * (threadIdx.x >> 6) + (lane >> 2);
  const bool feat_ok = feat < op.f;
  const float a = feat_ok ? __uint_as_float(op.colmax[feat]) : 0.0f;
  const bool tiny = a < 0x1p-100f;
  const float up = tiny ? 0x1p100f : 1.0f;
  const float as = a * up;
  const float r = as > 0.0f ? 127.0f / as : 0.0f;
  if (feat_ok && blockIdx.y == 0 && b == 0) op.scale[feat] = a / 127.0f;
  float v[kVals], sigma;
  load_rotate<G>(op.x, m, op.f, t0, f0, tile, v, sigma);
  if constexpr (G > 1) {
    const float nc = sigma * norm_const<G>();  // y = fl32(acc * nc): sigma only flips the sign
#pragma unroll
    for (int i = 0; i < kVals; ++i) v[i] = v[i] * nc;
  }
  if (tiny) {
#pragma unroll
    for (int i = 0; i < kVals; ++i) v[i] = v[i] * up;
  }
  constexpr float kRound = 0x1.8p23f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    v4u pk;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t c[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = __float_as_uint(__fadd_rn(__fmul_rn(v[16 * s + 4 * w + e], r), kRound));
      pk[w] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(c[3], c[2], 0x0C0C0400u),
                                    __builtin_amdgcn_perm(c[1], c[0], 0x0C0C0400u), 0x05040100u);
    }
    const int64_t tok = t0 + 64 * b + 16 * s;  // m is a multiple of 16: a piece is whole or absent
    if (feat_ok && tok < m) *reinterpret_cast<v4u *>(op.q + feat * m + tok) = pk;
  }
}

template <int G>
hipError_t launch_colq_g(const ColqOperand &a, const ColqOperand &b, int64_t m, hipStream_t s) {
  const dim3 grid((unsigned)(a.blocks + b.blocks), (unsigned)((m + kTok - 1) / kTok));
  hipLaunchKernelGGL(colq_absmax_kernel<G>, grid, dim3(256), 0, s, a, b, m);
  hipLaunchKernelGGL(colq_quantize_kernel<G>, grid, dim3(256), 0, s, a, b, m);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_colq_pair(const uint16_t *x0, int64_t f0, int8_t *q0, float *s0, const uint16_t *x1, int64_t f1,
                            int8_t *q1, float *s1, int64_t m, int g, uint32_t *colmax, hipStream_t stream) {
  if (f0 <= 0 || f0 % 16 != 0 || f1 < 0 || f1 % 16 != 0 || m <= 0 || m % 16 != 0) return hipErrorInvalidValue;
  if (g > 1 && m % g != 0) return hipErrorInvalidValue;
  if ((m + kTok - 1) / kTok > 65535) return hipErrorInvalidValue;
  const ColqOperand a{x0, f0, (f0 + kFeat - 1) / kFeat, colmax, q0, s0};
  const ColqOperand b{x1, f1, (f1 + kFeat - 1) / kFeat, colmax + f0, q1, s1};
  switch (g) {
    case 1: return launch_colq_g<1>(a, b, m, stream);
    case 64: return launch_colq_g<64>(a, b, m, stream);
    case 128: return launch_colq_g<128>(a, b, m, stream);
    case 256: return launch_colq_g<256>(a, b, m, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdnq
