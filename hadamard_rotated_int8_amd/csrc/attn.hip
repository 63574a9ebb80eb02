// Int8 Q K^T attention with K smoothing and a Hadamard rotation of the head rows.
//
// What it computes ("SDNQ: SD.Next Quantization Engine", the SDPA-replacement
// example: matmul_dtype int8 for Q K^T, pv_matmul_dtype disabled, smooth_k,
// use_hadamard with hadamard_group_size, quantize_fp32; SDPA's is_causal, scale
// and enable_gqa).  Readings, the pages giving the options only:
//   q [B, Hq, Sq, D], k and v [B, Hkv, Sk, D]; query head h reads head
//   h / (Hq / Hkv) of k and v.
//   smooth_k: mean[b, h, c] = fl32(sum_j k[b, h, j, c] / Sk), the sum in fp64 over
//   blocks of 64 tokens (each block in token order, then the block sums in
//   block order); K' = fl32(k - mean).
//   Q and K' rows are rotated with block min(g, D) (the linear layer's butterfly
//   and normalization) and quantized per token with its int8 quantizer.
//   scores s_ij = fp32(int32 q_i . k_j) * s_q[i] * s_k[j] * scale, keys j > i
//   masked when causal (top-left aligned); softmax; P V with P rounded to bf16 and
//   fp32 accumulation (online, flash-attention style); bf16 output.
//
// Kernels:
//  - attn_kmean_kernel (with smoothing): the K-mean block sums in fp64, one lane
//    per head, block and 4 channels;
//  - attn_prep_kernel: one launch for the rest of the prep: the K prep (with
//    smoothing each workgroup first finishes its head's mean from the block sums
//    into LDS), V^T with the keys of each 16-key group reordered, the Q prep,
//    and the split-tile flags cleared;
//  - the prep itself: four lanes per row of D values, the butterfly in
//    registers and, for the two stages that cross lanes, as multiply-adds with
//    DPP reads; the absmax by DPP reads; the int8 quantizer;
//  - attn_fwd_kernel: 128 query rows per workgroup (4 wavefronts x 32), 64 keys
//    per step, K codes and V^T double-buffered in LDS.  S = K Q^T per wavefront
//    with v_mfma_i32_32x32x32_i8 (lane l: query l % 32, keys 8 (r / 4) +
//    4 (l / 32) + r % 4 in register r); P V with v_mfma_f32_32x32x16_bf16, whose
//    contraction index is mapped to the keys so that each lane's own registers
//    8c .. 8c + 7 form its P operand: lane group g = l / 32 takes keys
//    16c + 4g + {0..3} and 16c + 8 + 4g + {0..3}, read from V^T as two 8-byte
//    runs.  exp2 with the log2(e) folded into the query scale; the softmax offset
//    is lazy (it moves only when a row maximum grows by more than 2^8).
#include <float.h>
#include <math.h>

#include <atomic>
#include <type_traits>

#include "sdnq_internal.hpp"

namespace sdnq {
namespace {

// The maximum and the sum of a value over lanes l and l ^ 32 (the two halves of a
// score row), with one v_permlane32_swap instead of an LDS-routed shuffle: the
// swap of (v, v) gives s[0] = v of lane l % 32 and s[1] = v of lane l % 32 + 32.
// The sum adds the lane's own value first, as own + partner.
__device__ __forceinline__ float xhalf_max(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float lo = __uint_as_float(s[0]), hi = __uint_as_float(s[1]);
  return (threadIdx.x & 32) ? hi + lo : lo + hi;
}

constexpr int kMeanBlock = 64;       // tokens per block of the K-mean sum
constexpr int kBM = 128;             // query rows per workgroup
constexpr int kBN = 64;              // keys per step
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.0f;    // the softmax offset moves when the maximum grows past 2^8
constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;  // fl32(1/sqrt(128))

// ---- Prep ----------------------------------------------------------------
// Rows of D values are handled by groups of 4 lanes: lane j of a group holds
// elements 32a + 8j + b (a < D/32, b < 8), loaded as D/32 runs of 8 bf16.  The
// butterfly stages h = 1, 2, 4 (bits of b) and h = 32, 64 (bits of a) pair
// elements inside a lane; h = 8 and 16 pair lane j with lane j ^ 1 and j ^ 2,
// read with DPP quad permutations.  A workgroup of 256 lanes takes 128 rows, two
// per group, both loaded (buffer loads: rows past the end read as zero) before
// either is processed.
constexpr int kPrepRows = 128;
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23

template <int G>
__device__ __forceinline__ float norm_const() {
  if constexpr (G == 64) return 0.125f;
  else if constexpr (G == 128) return kInvSqrt128;
  else return 1.0f;
}

template <int CTRL>
__device__ __forceinline__ float quad_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;

// One cross-lane butterfly stage on 8 registers: v = fma(v[partner lane], m, v)
// as one v_fmac_f32 with a quad_perm DPP source; m = +-1, so the product is exact
// and the result is fl(a + b) or -fl(a - b).  The s_nop gives the two wait states
// a DPP read needs after a VALU write of its source; inside the block no
// instruction reads a register that the one before it wrote.
#define ATTN_FMAC_DPP8(PERM)                                                                    \
  "s_nop 1\n\t"                                                                                \
  "v_fmac_f32_dpp %0, %0, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %1, %1, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %2, %2, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %3, %3, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %4, %4, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %5, %5, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %6, %6, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %7, %7, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf"

__device__ __forceinline__ void fmac_dpp_xor1(float (&r)[8], float m) {
  asm volatile(ATTN_FMAC_DPP8("[1,0,3,2]")
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7])
               : "v"(m));
}
__device__ __forceinline__ void fmac_dpp_xor2(float (&r)[8], float m) {
  asm volatile(ATTN_FMAC_DPP8("[2,3,0,1]")
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7])
               : "v"(m));
}

// Rows [first, first + kPrepRows) of x clipped to `valid` rows: lane group
// threadIdx.x / 4 reads rows first + g and first + g + 64.
template <int D>
__device__ __forceinline__ void prep_load2(const uint16_t *__restrict__ x, int64_t first, int64_t valid,
                                           v4u (&raw0)[D / 32], v4u (&raw1)[D / 32]) {
  const int64_t n = valid < kPrepRows ? valid : kPrepRows;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(x + first * D), 0, (int)(n * D * 2), 0x00020000);
  const int j = threadIdx.x & 3, g = threadIdx.x >> 2;
#pragma unroll
  for (int a = 0; a < D / 32; ++a) {
    raw0[a] = __builtin_bit_cast(
        v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, (unsigned)((g * D + 32 * a + 8 * j) * 2), 0, 0));
    raw1[a] = __builtin_bit_cast(
        v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, (unsigned)(((g + kPrepRows / 2) * D + 32 * a + 8 * j) * 2),
                                                   0, 0));
  }
}

// One row: minus the offset (K smoothing) when given, the rotation with block G,
// the row absmax across the group's lanes and the int8 quantizer.  Every lane of
// a group runs this, also for a missing row, so that the DPP reads see live lanes.
// The cross-lane stages leave y = sigma * v with sigma = +-1 per lane (the lower
// lane of a pair adds, the upper one takes the difference with a flipped sign);
// the normalization multiplies by sigma * norm, exactly y * norm.  Codes: rounding
// to nearest even by adding 1.5 * 2^23 (exact for |t| < 2^22), the code is the low
// byte; |t| <= 127 (1 + 2^-23) since r = fl(127 / absmax), so no clamp is needed.
template <int D, int G>
__device__ __forceinline__ void prep_row(const v4u (&raw)[D / 32], const float *offset, int j, bool ok, int64_t row,
                                         int8_t *__restrict__ codes, float *__restrict__ scale) {
  constexpr int NA = D / 32;
  float v[NA][8];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      v[a][2 * w] = bf16_lo(raw[a][w]);
      v[a][2 * w + 1] = bf16_hi(raw[a][w]);
    }
  if (offset) {
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      const float4 m0 = *reinterpret_cast<const float4 *>(offset + 32 * a + 8 * j);
      const float4 m1 = *reinterpret_cast<const float4 *>(offset + 32 * a + 8 * j + 4);
      v[a][0] = v[a][0] - m0.x; v[a][1] = v[a][1] - m0.y; v[a][2] = v[a][2] - m0.z; v[a][3] = v[a][3] - m0.w;
      v[a][4] = v[a][4] - m1.x; v[a][5] = v[a][5] - m1.y; v[a][6] = v[a][6] - m1.z; v[a][7] = v[a][7] - m1.w;
    }
  }
  if constexpr (G > 1) {
    static_assert(G >= 32, "the cross-lane stages are taken whole");
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b)
          if ((b & h) == 0) {
            const float lo = v[a][b], hi = v[a][b + h];
            v[a][b] = lo + hi;
            v[a][b + h] = lo - hi;
          }
    const float m1 = (j & 1) ? -1.0f : 1.0f, m2 = (j & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int a = 0; a < NA; ++a) fmac_dpp_xor1(v[a], m1);
#pragma unroll
    for (int a = 0; a < NA; ++a) fmac_dpp_xor2(v[a], m2);
#pragma unroll
    for (int h = 1; h < NA && 32 * h < G; h <<= 1)
#pragma unroll
      for (int a = 0; a < NA; ++a)
        if ((a & h) == 0)
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const float lo = v[a][b], hi = v[a + h][b];
            v[a][b] = lo + hi;
            v[a + h][b] = lo - hi;
          }
    const float sn = (m1 * m2) * norm_const<G>();
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int b = 0; b < 8; ++b) v[a][b] = v[a][b] * sn;
  }
  float am = 0.0f;
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) am = fmaxf(am, fabsf(v[a][b]));
  am = fmaxf(am, quad_dpp<kQuadXor1>(am));
  am = fmaxf(am, quad_dpp<kQuadXor2>(am));
  const float up = am < 0x1p-100f ? 0x1p100f : 1.0f;
  const float as = am * up;
  const float r = as > 0.0f ? 127.0f / as : 0.0f;
  if (!ok) return;
  if (j == 0) scale[row] = am / 127.0f;
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    uint32_t c[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) c[b] = __float_as_uint(__fadd_rn(__fmul_rn(v[a][b] * up, r), kRoundMagic));
    // v_perm_b32: selector bytes 0-3 pick the second operand's bytes, 4-7 the first's
    const uint32_t w0 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(c[3], c[2], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(c[1], c[0], 0x0c0c0400u), 0x05040100u);
    const uint32_t w1 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(c[7], c[6], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(c[5], c[4], 0x0c0c0400u), 0x05040100u);
    *reinterpret_cast<v2u *>(codes + row * D + 32 * a + 8 * j) = v2u{w0, w1};
  }
}

// kPrepRows consecutive rows from `first` of which `valid` exist, with an offset
// row of D values (LDS or global) or none.
template <int D, int G>
__device__ __forceinline__ void prep_rows(const uint16_t *__restrict__ x, int64_t first, int64_t valid,
                                          const float *offset, int8_t *__restrict__ codes,
                                          float *__restrict__ scale) {
  const int j = threadIdx.x & 3, g = threadIdx.x >> 2;
  v4u raw0[D / 32], raw1[D / 32];
  prep_load2<D>(x, first, valid, raw0, raw1);
  prep_row<D, G>(raw0, offset, j, g < valid, first + g, codes, scale);
  prep_row<D, G>(raw1, offset, j, g + kPrepRows / 2 < valid, first + g + kPrepRows / 2, codes, scale);
}

// K-mean partial sums: part[bh, blk, c] = sum of k[bh, j, c] over the tokens j of
// block blk (kMeanBlock tokens, the last one shorter), in token order, in fp64.
// One lane per (head, block, 4 channels); a whole block's tokens are loaded at
// once (8 bytes each), then added in order.  A short last block (16, 32 or 48
// tokens, as sk is a multiple of 16) goes 16 at a time.  The launch has few
// wavefronts, so registers go to loads in flight rather than occupancy.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 3))) void attn_kmean_kernel(const uint16_t *__restrict__ k, int64_t bhk, int64_t sk,
                                                         double *__restrict__ part) {
  constexpr int CG = D / 4;
  const int64_t nblk = (sk + kMeanBlock - 1) / kMeanBlock;
  const int64_t unit = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (unit >= bhk * nblk * CG) return;
  const int cg = (int)(unit % CG);
  const int64_t hb = unit / CG;  // bh * nblk + blk
  const int64_t bh = hb / nblk, blk = hb % nblk;
  const int64_t j0 = blk * kMeanBlock;
  const int n = (int)(sk - j0 < kMeanBlock ? sk - j0 : kMeanBlock);
  const uint16_t *p = k + (bh * sk + j0) * D + 4 * cg;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  auto run = [&](int t0, auto nb) {
    constexpr int NB = decltype(nb)::value;
    v2u w[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) w[i] = *reinterpret_cast<const v2u *>(p + (int64_t)(t0 + i) * D);
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        acc[2 * e] += (double)bf16_lo(w[i][e]);
        acc[2 * e + 1] += (double)bf16_hi(w[i][e]);
      }
  };
  if (n == kMeanBlock) {
    run(0, std::integral_constant<int, kMeanBlock>{});
  } else {
    for (int t0 = 0; t0 < n; t0 += 16) run(t0, std::integral_constant<int, 16>{});
  }
  double *o = part + hb * D + 4 * cg;
  *reinterpret_cast<double2 *>(o) = double2{acc[0], acc[1]};
  *reinterpret_cast<double2 *>(o + 2) = double2{acc[2], acc[3]};
}

// vt[bh, c, p] = v[bh, key(p), c]: V^T with the keys of every 16-key group stored
// in the order 0-3, 8-11, 4-7, 12-15, so that the 8 keys one lane feeds to the
// P V product are 16 contiguous bytes.  A lane moves 8 keys x 8 channels: eight
// 16-byte row loads, an 8 x 8 transpose of 16-bit values with byte permutes,
// eight 16-byte stores.  Lane l of a wavefront takes positions 8 (l / 8) .. + 7
// and channels 8 (l % 8) .. + 7 of a 64 x 64 block; a workgroup covers
// 256 / (D / 64) positions of all D channels.  sk is a multiple of 16, so a
// lane's 8 positions are all below sk or all past it.
template <int D>
__device__ __forceinline__ void vt_block(const uint16_t *__restrict__ v, int64_t sk, int64_t unit,
                                         uint16_t *__restrict__ vt) {
  constexpr int CW = D / 64;           // wavefronts across the channels
  constexpr int PPW = 64 * (4 / CW);   // positions per workgroup
  const int64_t npb = (sk + PPW - 1) / PPW;
  const int64_t bh = unit / npb;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t p0 = (unit % npb) * PPW + 64 * (wave / CW) + 8 * (lane >> 3);
  if (p0 >= sk) return;
  const int c0 = 64 * (wave % CW) + 8 * (lane & 7);
  const int64_t kb = (p0 & ~(int64_t)15) + ((p0 & 8) >> 1);
  const uint16_t *src = v + (bh * sk + kb) * D + c0;
  v4u r[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = *reinterpret_cast<const v4u *>(src + (int64_t)((i & 3) + ((i & 4) << 1)) * D);
  uint16_t *dst = vt + (bh * D + c0) * sk + p0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    v4u o;
#pragma unroll
    for (int w = 0; w < 4; ++w) o[w] = __builtin_amdgcn_perm(r[2 * w + 1][c >> 1], r[2 * w][c >> 1], sel);
    *reinterpret_cast<v4u *>(dst + (int64_t)c * sk) = o;
  }
}

// K prep with smoothing for kPrepRows keys of head bh from chunk `chunk`: the
// rows are loaded first; then the head's mean is finished from the partial sums
// into LDS: the block sums added in block order (32 loads in flight at a time;
// those past the last block read as +0, which leaves a sum that started at +0
// unchanged), then one division and one rounding to binary32.  The chunk-0
// workgroup also stores the mean.
template <int D, int G>
__device__ __forceinline__ void prep_k_smooth(const uint16_t *__restrict__ k, int64_t sk, int64_t bh, int64_t chunk,
                                              const double *__restrict__ kpart, float *__restrict__ kmean,
                                              int8_t *__restrict__ kc, float *__restrict__ ks, float *smean) {
  constexpr int kBatch = 32;
  const int j = threadIdx.x & 3, g = threadIdx.x >> 2;
  const int64_t first = bh * sk + chunk * kPrepRows, valid = sk - chunk * kPrepRows;
  v4u raw0[D / 32], raw1[D / 32];
  prep_load2<D>(k, first, valid, raw0, raw1);
  if (threadIdx.x < D) {
    const int64_t nblk = (sk + kMeanBlock - 1) / kMeanBlock;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(kpart + bh * nblk * D), 0, (int)(nblk * D * 8), 0x00020000);
    double s = 0.0;
    for (int64_t b0 = 0; b0 < nblk; b0 += kBatch) {
      double t[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int64_t b = b0 + i;
        const unsigned off = b < nblk ? (unsigned)((b * D + threadIdx.x) * 8) : 0x80000000u;
        t[i] = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0));
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) s += t[i];
    }
    const float m = (float)(s / (double)sk);
    smean[threadIdx.x] = m;
    if (chunk == 0) kmean[bh * D + threadIdx.x] = m;
  }
  __syncthreads();
  prep_row<D, G>(raw0, smean, j, g < valid, first + g, kc, ks);
  prep_row<D, G>(raw1, smean, j, g + kPrepRows / 2 < valid, first + g + kPrepRows / 2, kc, ks);
}

// Everything after the K-mean partial sums, in one launch; workgroups by range:
// [0, wg_k) the K prep (with smoothing: workgroup (bh, chunk), the mean finished
// first; these come first so that their wait overlaps the others' work), then
// wg_vt for V^T, then the Q prep.  The first lanes also clear the split-tile
// flags of the forward launch.
struct PrepArgs {
  const uint16_t *q, *k, *v;
  int64_t rows_q, bhk, sk;
  int8_t *qc, *kc;
  float *qs, *ks;
  const double *kpart;  // null: no smoothing
  float *kmean;
  uint16_t *vt;
  uint32_t *flags;
  int64_t nflags;
  int64_t wg_k, wg_vt;
};

template <int D, int G>
__global__ __launch_bounds__(256) void attn_prep_kernel(PrepArgs p) {
  __shared__ float smean[D];
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < p.nflags; i += (int64_t)gridDim.x * 256)
    p.flags[i] = 0u;
  int64_t b = blockIdx.x;
  if (b < p.wg_k) {
    if (p.kpart) {
      const int64_t nchunk = (p.sk + kPrepRows - 1) / kPrepRows;
      prep_k_smooth<D, G>(p.k, p.sk, b / nchunk, b % nchunk, p.kpart, p.kmean, p.kc, p.ks, smean);
    } else {
      prep_rows<D, G>(p.k, b * kPrepRows, p.bhk * p.sk - b * kPrepRows, nullptr, p.kc, p.ks);
    }
    return;
  }
  b -= p.wg_k;
  if (b < p.wg_vt) {
    vt_block<D>(p.v, p.sk, b, p.vt);
    return;
  }
  b -= p.wg_vt;
  prep_rows<D, G>(p.q, b * kPrepRows, p.rows_q - b * kPrepRows, nullptr, p.qc, p.qs);
}

// Block index -> (head, query tile): each XCD takes a contiguous run of the
// logical order (heads outermost), so the K and V of a head stay in one L2.
__device__ __forceinline__ void attn_coords(int nq, int &bh, int &qt) {
  const int nblk = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int q = nblk >> 3, rmd = nblk & 7;
  const int logical = xcd * q + (xcd < rmd ? xcd : rmd) + local;
  bh = logical / nq;
  qt = logical % nq;
}

typedef __attribute__((address_space(3))) void lds_void;
constexpr unsigned kOutOfRange = 0x80000000u;  // any offset past num_records reads as zero

// Split tiles: partial state of each tile whose key tiles two workgroups share.
// flags (zero before the launch): word 0 is the call's hand-over status, then
// per tile an arrival count and a published flag.
struct AttnSplit {
  float *part_o;      // [tiles][4 wavefronts][D/32][64 lanes][16] fp32 (in register order)
  float *part_ml;     // [tiles][128 rows][2]: offset, row sum
  uint32_t *flags;    // [1 + 2 tiles]
  int64_t tiles;      // query tiles x heads x batch
  int64_t per;        // key tiles per workgroup
  uint32_t polls;     // bound of the hand-over wait (polls of about 64 clocks); 0: give up at once
};
constexpr uint32_t kSpinLimit = SDNQ_ATTENTION_HANDOVER_POLLS;  // about a second
// The hand-over wait's bound for the launches that follow; a test lowers it to
// make the wait give up, so that the status word's path runs with every kernel
// still exiting normally.
std::atomic<uint32_t> handover_polls{kSpinLimit};
constexpr int kSegFull = 0, kSegHead = 1, kSegTail = 2;

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(256, 3) void attn_fwd_kernel(const int8_t *__restrict__ qc, const float *__restrict__ qs,
                                                       const int8_t *__restrict__ kc, const float *__restrict__ ks,
                                                       const uint16_t *__restrict__ vt, int hq, int hkv, int64_t sq,
                                                       int64_t sk, float scale_log2, uint16_t *__restrict__ out,
                                                       AttnSplit split) {
  static_assert(!SPLIT || !CAUSAL, "split tiles: non-causal only (equal key ranges)");
  // LDS tiles, filled by direct global -> LDS loads (16 bytes per lane, 1 KB per
  // wavefront instruction), 16-byte chunks XOR-swizzled by row instead of padded:
  //   K codes [64 keys][D bytes]: chunk c of row r stored at c ^ (r % CPR);
  //   V^T     [D rows][64 key positions] bf16 (128-byte rows, keys permuted within
  //           16-key groups as the prep stores them): chunk c of row d at
  //           c ^ (d % 8).
  constexpr int CPR = D / 16;                 // 16-byte chunks per K row
  constexpr int KB = kBN * D;                 // K tile bytes
  constexpr int VB = D * kBN * 2;             // V^T tile bytes
  constexpr int KSLOTS = KB / 1024 / 4;       // K loads per wavefront per tile
  constexpr int VSLOTS = VB / 1024 / 4;       // V^T loads per wavefront per tile
  constexpr int KS = D / 32;                  // 32-deep k-steps of Q K^T
  constexpr int DT = D / 32;                  // 32-wide output column tiles of P V
  __shared__ __attribute__((aligned(1024))) int8_t k_lds[2][KB];
  __shared__ __attribute__((aligned(1024))) int8_t v_lds[2][VB];
  __shared__ __attribute__((aligned(16))) float ks_lds[2][kBN];
  __shared__ uint32_t first_owner;

  const int nq = (int)((sq + kBM - 1) / kBM);
  const int64_t nkt = (sk + kBN - 1) / kBN;  // key tiles of a full row
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sk32 = (int)sk;  // below 2^20

  // per-lane parts of the load offsets (independent of the head)
  unsigned koff[KSLOTS], voff[VSLOTS];
  int vkey[VSLOTS];
#pragma unroll
  for (int j = 0; j < KSLOTS; ++j) {
    const int slot = j * 4 + wave;
    const int row = slot * (64 / CPR) + lane / CPR;
    const int lc = (lane % CPR) ^ (row % CPR);
    koff[j] = (unsigned)(row * D + 16 * lc);
  }
#pragma unroll
  for (int j = 0; j < VSLOTS; ++j) {
    const int slot = j * 4 + wave;
    const int d = slot * 8 + lane / 8;
    const int lc = (lane % 8) ^ (d % 8);
    vkey[j] = 8 * lc;
    voff[j] = (unsigned)((d * sk32 + 8 * lc) * 2);
  }

  // One segment: query tile qt of head bh against key tiles [kb, ke).
  // kSegFull writes the output.  The two owners of a split tile (kSegHead runs
  // its first key tiles, kSegTail the rest) meet at the tile's arrival count:
  // the first to arrive publishes (o, offset, row sum), the second merges them
  // with its own and writes the output.
  auto segment = [&](int bh, int qt, int64_t kb, int64_t ke, int mode) {
    const int b = bh / hq, h = bh % hq;
    const int64_t bhk = (int64_t)b * hkv + h / (hq / hkv);
    const int64_t q0 = (int64_t)qt * kBM;
    const int64_t my_row = q0 + 32 * wave + (lane & 31);
    const int my_row32 = (int)my_row;  // below 2^20

    // Q fragments: lane holds row my_row, bytes 32 s + 16 g .. + 15
    v4i qf[KS];
    const bool row_ok = my_row < sq;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = row_ok ? *reinterpret_cast<const v4i *>(qc + (bh * sq + my_row) * D + 32 * s + 16 * g)
                     : v4i{0, 0, 0, 0};
    // The row's factor s_q * scale * log2 e, at least FLT_MIN: a zero (or flushed
    // subnormal) factor would make a masked key's -inf * 0 a NaN; with FLT_MIN the
    // row's valid scores stay within 2^-126 of zero and masked keys stay at -inf.
    const float qscale = row_ok ? fmaxf(qs[bh * sq + my_row] * scale_log2, FLT_MIN) : FLT_MIN;

    // buffer resources over this head's K codes, K scales and V^T: rows past sk
    // lie past num_records and read as zero; V^T chunks past sk get an
    // out-of-range offset (the next row would follow otherwise)
    const __amdgpu_buffer_rsrc_t rs_k =
        __builtin_amdgcn_make_buffer_rsrc((void *)(kc + bhk * sk * D), 0, (int)(sk * D), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_s =
        __builtin_amdgcn_make_buffer_rsrc((void *)(ks + bhk * sk), 0, (int)(sk * 4), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_v =
        __builtin_amdgcn_make_buffer_rsrc((void *)(vt + bhk * (int64_t)D * sk), 0, (int)(D * sk * 2), 0x00020000);
    auto issue = [&](int64_t t, int buf) {
      const int k0 = (int)(t * kBN);
#pragma unroll
      for (int j = 0; j < KSLOTS; ++j) {
        const unsigned off = koff[j] + (unsigned)(k0 * D);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_k, (lds_void *)(k_lds[buf] + 1024 * (j * 4 + wave)), 16, off, 0,
                                                 0, 0);
      }
#pragma unroll
      for (int j = 0; j < VSLOTS; ++j) {
        const unsigned off = (k0 + vkey[j] < sk32) ? voff[j] + (unsigned)(k0 * 2) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_v, (lds_void *)(v_lds[buf] + 1024 * (j * 4 + wave)), 16, off, 0,
                                                 0, 0);
      }
      if (wave == 0) {
        const unsigned off = (unsigned)((k0 + lane) * 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_s, (lds_void *)ks_lds[buf], 4, off, 0, 0, 0);
      }
    };

    v16f o[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) o[i] = v16f{};
    float m_run = -INFINITY, l_run = 0.0f;

    if (CAUSAL) {
      const int64_t last = (q0 + kBM - 1) / kBN + 1;
      if (last < ke) ke = last;
    }
    issue(kb, (int)(kb & 1));
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    for (int64_t t = kb; t < ke; ++t) {
      const int buf = (int)(t & 1);
      if (t + 1 < ke) issue(t + 1, buf ^ 1);  // buf ^ 1 was released by the last barrier
      const int k032 = (int)(t * kBN);
      const int8_t *kt = k_lds[buf];
      const int8_t *vtile = v_lds[buf];
      // two 32-key halves, each with its own online-softmax update
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // S = K Q^T: lane: query l % 32, key 32 u + 8 (r / 4) + 4 g + r % 4 in register r
        v16i sacc = v16i{};
        const int krow = 32 * u + (lane & 31);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const int lc = (2 * s + g) ^ (krow % CPR);
          const v4i kf = *reinterpret_cast<const v4i *>(kt + krow * D + 16 * lc);
          sacc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[s], sacc, 0, 0, 0);
        }
        float sv[16];
        const bool edge = (k032 + 32 * u + 32 > sk32) || (CAUSAL && k032 + 32 * u + 31 > (int)q0 + 32 * wave);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int kk = 32 * u + 8 * r4 + 4 * g;
          const float4 kq = *reinterpret_cast<const float4 *>(&ks_lds[buf][kk]);
          const float kv[4] = {kq.x, kq.y, kq.z, kq.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[4 * r4 + e] = (float)sacc[4 * r4 + e] * kv[e];
          if (edge) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = k032 + kk + e;
              if (key >= sk32 || (CAUSAL && key > my_row32)) sv[4 * r4 + e] = -INFINITY;
            }
          }
        }
        // sv holds acc * s_k (the row's positive factor s_q * scale * log2 e is
        // applied inside the exponent, after the max)
        float mx = sv[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sv[r]);
        mx = xhalf_max(mx) * qscale;
        // Lazy reference: the exponent's offset m_run moves only when the row's
        // maximum exceeds it by more than kLazyLog2, so p <= 2^kLazyLog2 and the
        // running output is rescaled rarely.  softmax is unchanged: numerator and
        // denominator share the offset.  The first half moves it (key 0 is valid
        // for every row, so it is finite from then on).
        const float m_new = mx > m_run + kLazyLog2 ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        const float neg_m = -m_new;
        // The exponent is one fma of the exact product against the rounded offset.
        // Once offsets pass 2^14 (a logit of about 10^4) half an ulp of the offset
        // is no longer small in the exponent, and past 2^31 it would exceed 128 and
        // turn the row maximum's term into inf or 0; such wavefronts (never with
        // ordinary inputs) take the rounded product minus the offset, which is
        // exactly 0 for the maximum.  The vote is a compare on the offset, so the
        // exponents do not wait for alpha.
        const bool big = __ballot(fabsf(m_new) > 0x1p14f) != 0;
        float qf = qscale;
        if (big) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[r] = __fmul_rn(sv[r], qscale);
          qf = 1.0f;  // fma(t, 1, -m) = t - m, rounded once
        }
        float psum2[2] = {0.0f, 0.0f};
        v8bf pf[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[8 * c + e], qf, neg_m));
            psum2[c] += p[e];
          }
          v4u packed;
#pragma unroll
          for (int w = 0; w < 4; ++w) packed[w] = pack_bf16x2(p[2 * w], p[2 * w + 1]);
          pf[c] = __builtin_bit_cast(v8bf, packed);
        }
        float psum = psum2[0] + psum2[1];
        psum = xhalf_sum(psum);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        // rescale the running output only when some row's offset moved (alpha is
        // exactly 1 otherwise)
        if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
          for (int i = 0; i < DT; ++i) o[i] = o[i] * alpha;
        }
        // O += P V: V^T operand of lane l: row d = 32 dt + l % 32, keys 32 u + 16 c +
        // 4 g + {0..3, 8..11}, i.e. stored positions 32 u + 16 c + 8 g .. + 7, one
        // logical 16-byte chunk 4 u + 2 c + g
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int d = 32 * dt + (lane & 31);
          const int8_t *vrow = vtile + d * (kBN * 2);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const v8bf vv = *reinterpret_cast<const v8bf *>(vrow + 16 * ((4 * u + 2 * c + g) ^ (d % 8)));
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pf[c], o[dt], 0, 0, 0);
          }
        }
      }
      // tile t + 1 has landed and every wavefront is done with tile t: its own
      // LDS reads of tile t too (lgkmcnt), since the compiler may leave the last
      // fragment reads in flight here and wait for them only at their MFMAs,
      // while the next step's loads already refill this buffer
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    if (mode == kSegHead || mode == kSegTail) {
      // A share of a tile (o, the offset and the row sum) goes through
      // agent-coherent (sc1) stores and loads: written through, read past any
      // cached copy.  No cache-wide write-back or invalidation is needed, which
      // would otherwise empty the XCD's L2 under every other workgroup.
      const int64_t tile = (int64_t)bh * nq + qt;
      uint32_t *const arrivals = split.flags + 1 + 2 * tile;
      uint32_t *const published = arrivals + 1;
      const __amdgpu_buffer_rsrc_t rs_o = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(split.part_o + tile * (int64_t)kBM * D), 0, kBM * D * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t rs_ml = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(split.part_ml + tile * (int64_t)kBM * 2), 0, kBM * 2 * 4, 0x00020000);
      // o of (wave, dt): 64 lanes x 64 bytes, lane-contiguous; (m, l) of row 32 wave + lane % 32
      const unsigned o_off = (unsigned)((wave * DT * 64 + lane) * 64);
      const unsigned ml_off = (unsigned)((32 * wave + (lane & 31)) * 8);
      constexpr int kSc1 = 16;  // cache policy: agent-coherent
      if (tid == 0)
        first_owner = __hip_atomic_fetch_add(arrivals, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u;
      __syncthreads();
      if (first_owner) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(v4u, v4f{o[dt][4 * c], o[dt][4 * c + 1], o[dt][4 * c + 2], o[dt][4 * c + 3]}),
                rs_o, o_off + (unsigned)(dt * 64 * 64 + 16 * c), 0, kSc1);
        if (g == 0) __builtin_amdgcn_raw_buffer_store_b64(v2u{__float_as_uint(m_run), __float_as_uint(l_run)}, rs_ml,
                                                          ml_off, 0, kSc1);
        // every wavefront's stores have completed (vmcnt), then one flag store
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (tid == 0) __hip_atomic_store(published, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
      // Second to arrive: the first owner counted itself in after its key tiles,
      // so it is running and only its stores remain; it depends on no other
      // workgroup.  The wait is bounded all the same, so no wavefront can spin
      // forever; running out marks the call's status word.
      if (tid == 0) {
        bool ok = split.polls > 0;
        for (uint32_t spin = 0; ok && __hip_atomic_load(published, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u;) {
          if (++spin >= split.polls)
            ok = false;
          else
            __builtin_amdgcn_s_sleep(2);
        }
        if (!ok) __hip_atomic_store(split.flags, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      const v2u ml = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(rs_ml, ml_off, 0, kSc1));
      const float m_h = __uint_as_float(ml[0]), l_h = __uint_as_float(ml[1]);
      const float m_new = fmaxf(m_run, m_h);
      const float a_t = __builtin_amdgcn_exp2f(m_run - m_new), a_h = __builtin_amdgcn_exp2f(m_h - m_new);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const v4f hd = __builtin_bit_cast(
              v4f, __builtin_amdgcn_raw_buffer_load_b128(rs_o, o_off + (unsigned)(dt * 64 * 64 + 16 * c), 0, kSc1));
#pragma unroll
          for (int e = 0; e < 4; ++e) o[dt][4 * c + e] = o[dt][4 * c + e] * a_t + hd[e] * a_h;
        }
        __builtin_amdgcn_sched_barrier(0);  // one tile of the other share at a time: bounds registers
      }
      l_run = l_run * a_t + l_h * a_h;
    }

    // out[bh, row, d] = bf16(o / l); lane holds d = 32 dt + 8 (r / 4) + 4 g + r % 4
    if (!row_ok) return;
    const float inv = 1.0f / l_run;
    uint16_t *orow = out + (bh * sq + my_row) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        v2u pk = {pack_bf16x2(o[dt][4 * r4] * inv, o[dt][4 * r4 + 1] * inv),
                  pack_bf16x2(o[dt][4 * r4 + 2] * inv, o[dt][4 * r4 + 3] * inv)};
        *reinterpret_cast<v2u *>(orow + 32 * dt + 8 * r4 + 4 * g) = pk;
      }
  };

  // The segments this workgroup runs, through one call site (inlined once).
  int nseg = 1;
  [[maybe_unused]] int64_t s0 = 0, e0 = 0, tf = 0, tl = 0;
  [[maybe_unused]] bool has_head = false, has_tail = false;
  if constexpr (SPLIT) {
    // Split tiles (non-causal): the tiles' key tiles laid end to end (tiles in
    // the XCD-contiguous order of attn_coords, heads outermost), and workgroup p
    // in that order takes the run [p * per, (p + 1) * per), per >= nkt.  A tile
    // then has at most two owners, one running its head key tiles and one its
    // tail; whichever finishes second merges the two shares.  Each workgroup
    // runs its head segment first, then whole tiles, then its tail segment, so
    // the head share is usually the one published.
    const int64_t total = split.tiles * nkt;
    const int nblk = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, local = bid >> 3;
    const int qd = nblk >> 3, rmd = nblk & 7;
    const int64_t p = xcd * qd + (xcd < rmd ? xcd : rmd) + local;
    s0 = p * split.per;
    e0 = s0 + split.per < total ? s0 + split.per : total;
    if (s0 >= e0) return;
    tf = s0 / nkt;
    tl = (e0 - 1) / nkt;
    has_tail = s0 > tf * nkt;       // the range starts inside tile tf
    has_head = e0 < (tl + 1) * nkt;  // the range ends inside tile tl (tl > tf: per >= nkt)
    nseg = (int)(tl - tf + 1);
  }
  for (int i = 0; i < nseg; ++i) {
    int bh, qt, mode = kSegFull;
    int64_t kb = 0, ke = nkt;
    if constexpr (SPLIT) {
      int64_t t;
      if (has_head && i == 0) {
        t = tl;
        ke = e0 - tl * nkt;
        mode = kSegHead;
      } else if (has_tail && i == nseg - 1) {
        t = tf;
        kb = s0 - tf * nkt;
        mode = kSegTail;
      } else {
        t = (has_tail ? tf + 1 : tf) + (i - (has_head ? 1 : 0));
      }
      bh = (int)(t / nq);
      qt = (int)(t - (int64_t)bh * nq);
      if (i > 0) __syncthreads();  // the previous segment is done with the LDS tiles
    } else {
      attn_coords(nq, bh, qt);
      if (CAUSAL) qt = nq - 1 - qt;  // the longest rows first
    }
    segment(bh, qt, kb, ke, mode);
  }
}

struct AttnLayout {
  size_t qc, qs, kc, ks, kmean, kpart, vt, part_o, part_ml, flags, total;
};

// Split tiles are used for at most this many query tiles (about five rounds of
// workgroups), which bounds their scratch (64 KB per tile at head_dim 128).
constexpr int64_t kMaxSplitTiles = 4096;

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

AttnLayout attn_layout(int64_t bsz, int64_t hq, int64_t hkv, int64_t sq, int64_t sk, int64_t d) {
  AttnLayout L{};
  const int64_t nblk = (sk + kMeanBlock - 1) / kMeanBlock;
  size_t off = 0;
  L.qc = off; off += align256((size_t)(bsz * hq * sq * d));
  L.qs = off; off += align256((size_t)(bsz * hq * sq) * 4);
  L.kc = off; off += align256((size_t)(bsz * hkv * sk * d));
  L.ks = off; off += align256((size_t)(bsz * hkv * sk) * 4);
  L.kmean = off; off += align256((size_t)(bsz * hkv * d) * 4);
  L.kpart = off; off += align256((size_t)(bsz * hkv * nblk * d) * 8);
  L.vt = off; off += align256((size_t)(bsz * hkv * sk * d) * 2);
  const int64_t tiles = bsz * hq * ((sq + kBM - 1) / kBM);
  const int64_t split_tiles = tiles <= kMaxSplitTiles ? tiles : 0;
  L.part_o = off; off += align256((size_t)split_tiles * kBM * d * 4);
  L.part_ml = off; off += align256((size_t)split_tiles * kBM * 2 * 4);
  L.flags = off; off += align256((size_t)(1 + 2 * split_tiles) * 4);  // status word, then 2 per split tile
  L.total = off;
  return L;
}

// The prep launches: with smoothing the K-mean partial sums, then the fused one.
template <int D, int G>
hipError_t launch_prep(const PrepArgs &p, hipStream_t s) {
  if (p.kpart) {
    const int64_t nblk = (p.sk + kMeanBlock - 1) / kMeanBlock;
    const int64_t lanes = p.bhk * nblk * (D / 4);
    hipLaunchKernelGGL((attn_kmean_kernel<D>), dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s, p.k, p.bhk,
                       p.sk, const_cast<double *>(p.kpart));
  }
  const int64_t wg_q = (p.rows_q + kPrepRows - 1) / kPrepRows;
  hipLaunchKernelGGL((attn_prep_kernel<D, G>), dim3((unsigned)(p.wg_k + p.wg_vt + wg_q)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t prep_any(int block, const PrepArgs &p, hipStream_t s) {
  switch (block) {
    case 1: return launch_prep<D, 1>(p, s);
    case 64: return launch_prep<D, 64>(p, s);
    case 128:
      if constexpr (D >= 128) return launch_prep<D, 128>(p, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

// Resident split-tile workgroups per CU (the split deals the key tiles to
// exactly the workgroups that fit at once; correctness does not depend on it).
template <int D>
int split_blocks_per_cu() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void *)attn_fwd_kernel<D, false, true>, 256, 0) !=
            hipSuccess ||
        n < 1)
      n = 1;
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D>
hipError_t attention_d(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t bsz, int64_t hq, int64_t hkv,
                       int64_t sq, int64_t sk, bool causal, float scale, bool smooth_k, int g, uint16_t *out,
                       void *ws, hipStream_t s) {
  const AttnLayout L = attn_layout(bsz, hq, hkv, sq, sk, D);
  char *base = static_cast<char *>(ws);
  int8_t *qc = reinterpret_cast<int8_t *>(base + L.qc);
  float *qs = reinterpret_cast<float *>(base + L.qs);
  int8_t *kc = reinterpret_cast<int8_t *>(base + L.kc);
  float *ks = reinterpret_cast<float *>(base + L.ks);
  float *kmean = reinterpret_cast<float *>(base + L.kmean);
  double *kpart = reinterpret_cast<double *>(base + L.kpart);
  uint16_t *vt = reinterpret_cast<uint16_t *>(base + L.vt);
  const int block = g <= 1 ? 1 : (g < D ? g : D);
  const int64_t bhk = bsz * hkv;
  const int64_t nq = (sq + kBM - 1) / kBM;
  const int64_t tiles = nq * bsz * hq;
  const float sl = scale * kLog2e;
  // Non-causal: when the tiles overfill the resident workgroups by a little, a
  // last round runs almost empty for nearly a full workgroup's time; split tiles
  // spread the key tiles evenly over exactly the resident workgroups instead.
  // Splitting costs about 7 % per tile (segment starts, the head's hand-over),
  // so it is used only while the leftover is at most a sixth of a round (flux.1,
  // 864 tiles on 768 workgroups: 357 -> 329 us; 1008 tiles would lose 3 %).
  const int64_t nkt = (sk + kBN - 1) / kBN;
  bool split = false;
  int64_t slots = 0;
  if (!causal) {
    slots = (int64_t)device_cu_count() * split_blocks_per_cu<D>();
    const int64_t leftover = tiles % slots;
    split = tiles > slots && leftover != 0 && 6 * leftover <= slots && tiles <= kMaxSplitTiles && nkt >= 8;
  }
  PrepArgs pa{};
  pa.q = q;
  pa.k = k;
  pa.v = v;
  pa.rows_q = bsz * hq * sq;
  pa.bhk = bhk;
  pa.sk = sk;
  pa.qc = qc;
  pa.kc = kc;
  pa.qs = qs;
  pa.ks = ks;
  pa.kpart = smooth_k ? kpart : nullptr;
  pa.kmean = kmean;
  pa.vt = vt;
  pa.flags = reinterpret_cast<uint32_t *>(base + L.flags);
  pa.nflags = split ? 1 + 2 * tiles : 1;  // the status word is cleared on every call
  pa.wg_k = smooth_k ? bhk * ((sk + kPrepRows - 1) / kPrepRows) : (bhk * sk + kPrepRows - 1) / kPrepRows;
  const int64_t ppw = 64 * (4 / (D / 64));
  pa.wg_vt = bhk * ((sk + ppw - 1) / ppw);
  hipError_t e;
  if ((e = prep_any<D>(block, pa, s)) != hipSuccess) return e;
  if (causal) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, true, false>), dim3((unsigned)tiles), dim3(256), 0, s, qc, qs, kc, ks, vt,
                       (int)hq, (int)hkv, sq, sk, sl, out, AttnSplit{});
    return hipGetLastError();
  }
  if (split) {
    AttnSplit sp{};
    sp.part_o = reinterpret_cast<float *>(base + L.part_o);
    sp.part_ml = reinterpret_cast<float *>(base + L.part_ml);
    sp.flags = pa.flags;
    sp.tiles = tiles;
    sp.per = (tiles * nkt + slots - 1) / slots;  // >= nkt since tiles > slots
    sp.polls = handover_polls.load(std::memory_order_relaxed);
    hipLaunchKernelGGL((attn_fwd_kernel<D, false, true>), dim3((unsigned)slots), dim3(256), 0, s, qc, qs, kc, ks, vt,
                       (int)hq, (int)hkv, sq, sk, sl, out, sp);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((attn_fwd_kernel<D, false, false>), dim3((unsigned)tiles), dim3(256), 0, s, qc, qs, kc, ks, vt,
                     (int)hq, (int)hkv, sq, sk, sl, out, AttnSplit{});
  return hipGetLastError();
}

}  // namespace

void set_attention_handover_polls(uint32_t polls) { handover_polls.store(polls, std::memory_order_relaxed); }

size_t attention_workspace_bytes(int64_t bsz, int64_t hq, int64_t hkv, int64_t sq, int64_t sk, int64_t d) {
  return attn_layout(bsz, hq, hkv, sq, sk, d).total;
}

void attention_workspace_offsets(int64_t bsz, int64_t hq, int64_t hkv, int64_t sq, int64_t sk, int64_t d,
                                 size_t *offsets) {
  const AttnLayout L = attn_layout(bsz, hq, hkv, sq, sk, d);
  offsets[0] = L.qc;
  offsets[1] = L.qs;
  offsets[2] = L.kc;
  offsets[3] = L.ks;
  offsets[4] = L.kmean;
  offsets[5] = L.flags;
}

hipError_t launch_attention_int8(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t bsz, int64_t hq,
                                 int64_t hkv, int64_t sq, int64_t sk, int64_t d, bool causal, float scale,
                                 bool smooth_k, int g, uint16_t *out, void *workspace, hipStream_t stream) {
  if (d == 64) return attention_d<64>(q, k, v, bsz, hq, hkv, sq, sk, causal, scale, smooth_k, g, out, workspace, stream);
  if (d == 128)
    return attention_d<128>(q, k, v, bsz, hq, hkv, sq, sk, causal, scale, smooth_k, g, out, workspace, stream);
  return hipErrorInvalidValue;
}

}  // namespace sdnq
