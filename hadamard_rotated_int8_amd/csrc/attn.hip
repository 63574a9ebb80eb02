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
//  - attn_kmean_partial / attn_kmean_finish: the blocked fp64 sum, then the mean;
//  - attn_prep_kernel: sixteen lanes per row of D values (D/16 per lane), the
//    butterfly in registers and across the row's lanes with shuffles, absmax by
//    a 16-lane reduction;
//  - attn_vt_kernel: V [BH, Sk, D] -> V^T [BH, D, Sk] (64 x 64 LDS tiles);
//  - attn_fwd_kernel: 128 query rows per workgroup (4 wavefronts x 32), 64 keys
//    per step, K codes and V^T double-buffered in LDS.  S = K Q^T per wavefront
//    with v_mfma_i32_32x32x32_i8 (lane l: query l % 32, keys 8 (r / 4) +
//    4 (l / 32) + r % 4 in register r); P V with v_mfma_f32_32x32x16_bf16, whose
//    contraction index is mapped to the keys so that each lane's own registers
//    8c .. 8c + 7 form its P operand: lane group g = l / 32 takes keys
//    16c + 4g + {0..3} and 16c + 8 + 4g + {0..3}, read from V^T as two 8-byte
//    runs.  exp2 with the log2(e) folded into the query scale; the softmax offset
//    is lazy (it moves only when a row maximum grows by more than 2^8).
#include <math.h>

#include <atomic>

#include "sdnq_internal.hpp"

namespace sdnq {
namespace {

constexpr int kMeanBlock = 64;       // tokens per block of the K-mean sum
constexpr int kBM = 128;             // query rows per workgroup
constexpr int kBN = 64;              // keys per step
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.0f;    // the softmax offset moves when the maximum grows past 2^8
constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;  // fl32(1/sqrt(128))

__device__ __forceinline__ float bf16_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// part[bh, blk, c] = sum_{j in block blk} k[bh, j, c] in token order (fp64)
__global__ __launch_bounds__(256) void attn_kmean_partial(const uint16_t *__restrict__ k, int64_t bh_count,
                                                          int64_t sk, int d, double *__restrict__ part) {
  const int64_t nblk = (sk + kMeanBlock - 1) / kMeanBlock;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= bh_count * nblk * d) return;
  const int c = (int)(idx % d);
  const int64_t blk = (idx / d) % nblk, bh = idx / (d * nblk);
  const int64_t j0 = blk * kMeanBlock, j1 = j0 + kMeanBlock < sk ? j0 + kMeanBlock : sk;
  const uint16_t *p = k + (bh * sk) * d + c;
  double s = 0.0;
#pragma unroll 16
  for (int64_t j = j0; j < j1; ++j) s += (double)bf16_f32(p[j * d]);
  part[idx] = s;
}

// mean[bh, c] = fl32((sum over blocks in order) / sk)
__global__ __launch_bounds__(256) void attn_kmean_finish(const double *__restrict__ part, int64_t bh_count,
                                                         int64_t sk, int d, float *__restrict__ mean) {
  const int64_t nblk = (sk + kMeanBlock - 1) / kMeanBlock;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= bh_count * d) return;
  const int c = (int)(idx % d);
  const int64_t bh = idx / d;
  double s = 0.0;
#pragma unroll 8
  for (int64_t b = 0; b < nblk; ++b) s += part[(bh * nblk + b) * d + c];
  mean[idx] = (float)(s / (double)sk);
}

template <int G>
__device__ __forceinline__ float norm_const() {
  if constexpr (G == 64) return 0.125f;
  else if constexpr (G == 128) return kInvSqrt128;
  else return 1.0f;
}

// Sixteen lanes per row of D values, four rows per wavefront; lane l of a row
// holds elements VPL*l .. VPL*l + VPL-1 (16 bytes of bf16 for D = 128).  Rows of
// x: [rows, D] with rows = bh * seq; offset [bh, D] (binary32) subtracted first
// when given.  Codes [rows, D], scales [rows].
template <int D, int G, bool OFFSET>
__global__ __launch_bounds__(256) void attn_prep_kernel(const uint16_t *__restrict__ x, int64_t rows, int64_t seq,
                                                        const float *__restrict__ offset, int8_t *__restrict__ codes,
                                                        float *__restrict__ scale) {
  constexpr int VPL = D / 16;
  const int l16 = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool ok = row < rows;  // lanes of a missing row still take part in the shuffles
  float v[VPL];
  if constexpr (VPL == 8) {
    const v4u raw = ok ? *reinterpret_cast<const v4u *>(x + row * D + 8 * l16) : v4u{0u, 0u, 0u, 0u};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      v[2 * w] = bf16_lo(raw[w]);
      v[2 * w + 1] = bf16_hi(raw[w]);
    }
  } else {
    const v2u raw = ok ? *reinterpret_cast<const v2u *>(x + row * D + 4 * l16) : v2u{0u, 0u};
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      v[2 * w] = bf16_lo(raw[w]);
      v[2 * w + 1] = bf16_hi(raw[w]);
    }
  }
  if constexpr (OFFSET) {
    if (ok) {
      const float *o = offset + (row / seq) * D + VPL * l16;
#pragma unroll
      for (int e = 0; e < VPL; e += 4) {
        const float4 f = *reinterpret_cast<const float4 *>(o + e);
        v[e] = v[e] - f.x;
        v[e + 1] = v[e + 1] - f.y;
        v[e + 2] = v[e + 2] - f.z;
        v[e + 3] = v[e + 3] - f.w;
      }
    }
  }
  if constexpr (G > 1) {
#pragma unroll
    for (int h = 1; h < G; h <<= 1) {
      if (h < VPL) {  // both elements of the pair in this lane
#pragma unroll
        for (int e = 0; e < VPL; ++e)
          if ((e & h) == 0) {
            const float a = v[e], b = v[e + h];
            v[e] = a + b;
            v[e + h] = a - b;
          }
      } else {
        const int hl = h / VPL;  // 1, 2, 4, 8: within the row's 16 lanes
#pragma unroll
        for (int e = 0; e < VPL; ++e) {
          const float p = __shfl_xor(v[e], hl);
          v[e] = (l16 & hl) ? p - v[e] : v[e] + p;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < VPL; ++e) v[e] = v[e] * norm_const<G>();
  }
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < VPL; ++e) a = fmaxf(a, fabsf(v[e]));
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  const float up = a < 0x1p-100f ? 0x1p100f : 1.0f;
  const float as = a * up;
  const float r = as > 0.0f ? 127.0f / as : 0.0f;
  if (!ok) return;
  if (l16 == 0) scale[row] = a / 127.0f;
  uint32_t packed[VPL / 4];
#pragma unroll
  for (int w = 0; w < VPL / 4; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float t = rintf((v[4 * w + e] * up) * r);
      t = fminf(fmaxf(t, -127.0f), 127.0f);
      word |= ((uint32_t)(int)t & 0xFFu) << (8 * e);
    }
    packed[w] = word;
  }
  if constexpr (VPL == 8)
    *reinterpret_cast<v2u *>(codes + row * D + 8 * l16) = v2u{packed[0], packed[1]};
  else
    *reinterpret_cast<uint32_t *>(codes + row * D + 4 * l16) = packed[0];
}

// vt[bh, c, p] = v[bh, key(p), c]: V^T with the keys of every 16-key group stored
// in the order 0-3, 8-11, 4-7, 12-15, so that the 8 keys one lane feeds to the
// P V product are 16 contiguous bytes.  64 x 64 tiles through LDS, grid
// (ceil(sk/64), D/64, bh); sk is a multiple of 16.
__device__ __forceinline__ int vt_key(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

__global__ __launch_bounds__(256) void attn_vt_kernel(const uint16_t *__restrict__ v, int64_t sk, int d,
                                                      uint16_t *__restrict__ vt) {
  __shared__ uint16_t tile[64][66];
  const int64_t bh = blockIdx.z;
  const int64_t j0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const uint16_t *src = v + bh * sk * d;
  uint16_t *dst = vt + bh * (int64_t)d * sk;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int jj = e / 64, cc = e % 64;
    tile[jj][cc] = j0 + jj < sk ? src[(j0 + jj) * d + c0 + cc] : (uint16_t)0;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int cc = e / 64, pp = e % 64;
    if (j0 + pp < sk) dst[(int64_t)(c0 + cc) * sk + j0 + pp] = tile[vt_key(pp)][cc];
  }
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

// Split tiles: partial state of each tile whose key tiles two workgroups share,
// and a ready flag per tile (zero before the launch).
struct AttnSplit {
  float *part_o;      // [tiles][4 wavefronts][D/32][64 lanes][16] fp32 (in register order)
  float *part_ml;     // [tiles][128 rows][2]: offset, row sum
  uint32_t *flags;    // [tiles]
  int64_t tiles;      // query tiles x heads x batch
  int64_t per;        // key tiles per workgroup
};
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
  //           16-key groups as attn_vt_kernel stores them): chunk c of row d at
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
  // kSegFull writes the output; kSegHead hands (o, offset, row sum) of a tile's
  // first key tiles to the workgroup that runs the rest (kSegTail), which merges
  // them and writes the output.
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
    const float qscale = row_ok ? qs[bh * sq + my_row] * scale_log2 : 0.0f;

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
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * qscale;
        // Lazy reference: the exponent's offset m_run moves only when the row's
        // maximum exceeds it by more than kLazyLog2, so p <= 2^kLazyLog2 and the
        // running output is rescaled rarely.  softmax is unchanged: numerator and
        // denominator share the offset.  The first half moves it (key 0 is valid
        // for every row, so it is finite from then on).
        const float m_new = mx > m_run + kLazyLog2 ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        const float neg_m = -m_new;
        float psum2[2] = {0.0f, 0.0f};
        v8bf pf[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[8 * c + e], qscale, neg_m));
            psum2[c] += p[e];
          }
          v4u packed;
#pragma unroll
          for (int w = 0; w < 4; ++w) packed[w] = pack_bf16x2(p[2 * w], p[2 * w + 1]);
          pf[c] = __builtin_bit_cast(v8bf, packed);
        }
        float psum = psum2[0] + psum2[1];
        psum += __shfl_xor(psum, 32);
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
      // The head's share of a tile (o, the offset and the row sum) goes through
      // agent-coherent (sc1) stores and loads: written through, read past any
      // cached copy.  No cache-wide write-back or invalidation is needed, which
      // would otherwise empty the XCD's L2 under every other workgroup.
      const int64_t tile = (int64_t)bh * nq + qt;
      const __amdgpu_buffer_rsrc_t rs_o = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(split.part_o + tile * (int64_t)kBM * D), 0, kBM * D * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t rs_ml = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(split.part_ml + tile * (int64_t)kBM * 2), 0, kBM * 2 * 4, 0x00020000);
      // o of (wave, dt): 64 lanes x 64 bytes, lane-contiguous; (m, l) of row 32 wave + lane % 32
      const unsigned o_off = (unsigned)((wave * DT * 64 + lane) * 64);
      const unsigned ml_off = (unsigned)((32 * wave + (lane & 31)) * 8);
      constexpr int kSc1 = 16;  // cache policy: agent-coherent
      if (mode == kSegHead) {
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
        if (tid == 0) __hip_atomic_store(split.flags + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
      // Tail: merge the head's share, both halves against the larger offset.  The
      // head ran first in its workgroup, which started no later than this one;
      // the wait is bounded (about a second) all the same, so no wavefront can
      // spin forever.
      if (tid == 0) {
        for (int spin = 0; spin < (1 << 24); ++spin) {
          if (__hip_atomic_load(split.flags + tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
          __builtin_amdgcn_s_sleep(2);
        }
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
        __builtin_amdgcn_sched_barrier(0);  // one tile of the head's output at a time: bounds registers
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
    // then has at most two owners: the first runs its head and hands it over,
    // the second runs the tail and finishes it.  Each workgroup runs its head
    // segment first, then whole tiles, then its tail segment, so a tail waits
    // only on a head that its owner ran first.
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
  L.flags = off; off += align256((size_t)split_tiles * 4);
  L.total = off;
  return L;
}

template <int D, int G>
hipError_t launch_prep(const uint16_t *x, int64_t rows, int64_t seq, const float *offset, int8_t *codes, float *scale,
                       hipStream_t s) {
  const unsigned blocks = (unsigned)((rows + 15) / 16);
  if (offset)
    hipLaunchKernelGGL((attn_prep_kernel<D, G, true>), dim3(blocks), dim3(256), 0, s, x, rows, seq, offset, codes,
                       scale);
  else
    hipLaunchKernelGGL((attn_prep_kernel<D, G, false>), dim3(blocks), dim3(256), 0, s, x, rows, seq, offset, codes,
                       scale);
  return hipGetLastError();
}

template <int D>
hipError_t prep_any(int block, const uint16_t *x, int64_t rows, int64_t seq, const float *offset, int8_t *codes,
                    float *scale, hipStream_t s) {
  switch (block) {
    case 1: return launch_prep<D, 1>(x, rows, seq, offset, codes, scale, s);
    case 64: return launch_prep<D, 64>(x, rows, seq, offset, codes, scale, s);
    case 128:
      if constexpr (D >= 128) return launch_prep<D, 128>(x, rows, seq, offset, codes, scale, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

// Resident split-tile workgroups per CU (all of them must be resident at once:
// a tail waits for a head that another workgroup runs).
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
  hipError_t e;
  if (smooth_k) {
    const int64_t nblk = (sk + kMeanBlock - 1) / kMeanBlock;
    const int64_t np = bhk * nblk * D, nm = bhk * D;
    hipLaunchKernelGGL(attn_kmean_partial, dim3((unsigned)((np + 255) / 256)), dim3(256), 0, s, k, bhk, sk, D, kpart);
    hipLaunchKernelGGL(attn_kmean_finish, dim3((unsigned)((nm + 255) / 256)), dim3(256), 0, s, kpart, bhk, sk, D,
                       kmean);
  }
  if ((e = prep_any<D>(block, q, bsz * hq * sq, sq, nullptr, qc, qs, s)) != hipSuccess) return e;
  if ((e = prep_any<D>(block, k, bhk * sk, sk, smooth_k ? kmean : nullptr, kc, ks, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(attn_vt_kernel, dim3((unsigned)((sk + 63) / 64), D / 64, (unsigned)bhk), dim3(256), 0, s, v, sk,
                     D, vt);
  const int64_t nq = (sq + kBM - 1) / kBM;
  const int64_t tiles = nq * bsz * hq;
  const float sl = scale * kLog2e;
  if (causal) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, true, false>), dim3((unsigned)tiles), dim3(256), 0, s, qc, qs, kc, ks, vt,
                       (int)hq, (int)hkv, sq, sk, sl, out, AttnSplit{});
    return hipGetLastError();
  }
  // Non-causal: when the tiles overfill the resident workgroups by a little, a
  // last round runs almost empty for nearly a full workgroup's time; split tiles
  // spread the key tiles evenly over exactly the resident workgroups instead.
  // Splitting costs about 7 % per tile (segment starts, the head's hand-over),
  // so it is used only while the leftover is at most a sixth of a round (flux.1,
  // 864 tiles on 768 workgroups: 357 -> 329 us; 1008 tiles would lose 3 %).
  const int64_t nkt = (sk + kBN - 1) / kBN;
  const int64_t slots = (int64_t)device_cu_count() * split_blocks_per_cu<D>();
  const int64_t leftover = tiles % slots;
  if (tiles > slots && leftover != 0 && 6 * leftover <= slots && tiles <= kMaxSplitTiles && nkt >= 8) {
    AttnSplit sp{};
    sp.part_o = reinterpret_cast<float *>(base + L.part_o);
    sp.part_ml = reinterpret_cast<float *>(base + L.part_ml);
    sp.flags = reinterpret_cast<uint32_t *>(base + L.flags);
    sp.tiles = tiles;
    sp.per = (tiles * nkt + slots - 1) / slots;  // >= nkt since tiles > slots
    if ((e = launch_fill_zero_u16(reinterpret_cast<uint16_t *>(sp.flags), 2 * tiles, s)) != hipSuccess) return e;
    hipLaunchKernelGGL((attn_fwd_kernel<D, false, true>), dim3((unsigned)slots), dim3(256), 0, s, qc, qs, kc, ks, vt,
                       (int)hq, (int)hkv, sq, sk, sl, out, sp);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((attn_fwd_kernel<D, false, false>), dim3((unsigned)tiles), dim3(256), 0, s, qc, qs, kc, ks, vt,
                     (int)hq, (int)hkv, sq, sk, sl, out, AttnSplit{});
  return hipGetLastError();
}

}  // namespace

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
