// Internal declarations shared by the HIP translation units of libsdnq_hip.
// Kernels are written for gfx950 (CDNA4): 64-lane wavefronts, MFMA, 160 KB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sdnq_hip.h"

namespace sdnq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// bf16 bits -> fp32 (exact): the bf16 pattern is the high half of the fp32 one.
__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even: one v_cvt_pk_bf16_f32 for the pair.
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){lo, hi}, v2bf));
}

// ------------------------------------------------------------------ launches --
// Each returns hipSuccess or the launch error; arguments are validated by the caller.

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cu_count();

// G1: rotate (block g) + per-row absmax int8 quantization of a bf16 [rows, cols] matrix.
hipError_t launch_rotate_quantize(const uint16_t *x, int64_t rows, int64_t cols, int g,
                                  const float *col_scale, int8_t *q, float *scale,
                                  hipStream_t stream);
// The same with the FP8 (E4M3) quantizer: s = a / 448, codes e4m3(clamp(y * r, +-448)).
hipError_t launch_rotate_quantize_fp8(const uint16_t *x, int64_t rows, int64_t cols, int g,
                                      const float *col_scale, uint8_t *q, float *scale, hipStream_t stream);

// G2 epilogue selector.
enum class Epilogue { kInt32, kForward, kBackward };

struct GemmArgs {
  const int8_t *a;        // [m, k]  column operand (tokens)
  const int8_t *b;        // [n, k]  row operand (weight rows, or transposed weight)
  int64_t m, n, k;
  // kInt32
  int32_t *c_i32;         // [m, n]
  // kForward / kBackward
  const float *row_scale; // [m]  token scale
  const float *col_scale; // [n]  weight row scale (forward only, else nullptr)
  const uint16_t *lora_t; // [m, rank] bf16 left factor (nullable)
  const uint16_t *lora_r; // [n, rank] bf16 right factor, one row per output column (nullable);
                          // the LoRA scale is already folded into one of the two factors
  int rank;
  int g;                  // backward: inverse rotation block along n (1, 64, 128, 256)
  uint16_t *out_bf16;     // [m, n]
  bool fp8;               // a and b hold E4M3 codes (fp32 accumulators); the kInt32 epilogue
                          // then stores the accumulators' bits
};

hipError_t launch_gemm_i8(Epilogue epi, const GemmArgs &args, hipStream_t stream);
// The int8 forward GEMM (no LoRA) with parts of its k loop removed, to measure
// its rate ceiling: mode 0 none (the product kernel), 1 the global loads after
// the first two k-tiles, 2 also the LDS fragment reads, 3 as 2 on operands made
// of loop indices.
hipError_t launch_gemm_i8_ceiling(const GemmArgs &args, int mode, hipStream_t stream);

// int8 [rows, cols] -> [cols, rows]
hipError_t launch_transpose_i8(const int8_t *in, int64_t rows, int64_t cols, int8_t *out,
                               hipStream_t stream);
// 16-bit [rows, cols] -> [cols, rows]
hipError_t launch_transpose_u16(const uint16_t *in, int64_t rows, int64_t cols, uint16_t *out,
                                hipStream_t stream);
// two such transposes in one launch (in1 == nullptr: only the first); sides multiples of 8
hipError_t launch_transpose_u16_pair(const uint16_t *in0, int64_t rows0, int64_t cols0, uint16_t *out0,
                                     const uint16_t *in1, int64_t rows1, int64_t cols1, uint16_t *out1,
                                     hipStream_t stream);
// bf16 [rows, cols] -> bf16(scale * in)^T [cols, rows]
hipError_t launch_transpose_scale_bf16(const uint16_t *in, int64_t rows, int64_t cols, float scale,
                                       uint16_t *out, hipStream_t stream);

// out[0 .. count) = 0 (16-bit elements)
hipError_t launch_fill_zero_u16(uint16_t *out, int64_t count, hipStream_t stream);

// out [out_rows, out_cols] = in [in_rows, in_cols] where both are defined, else 0
// (16-bit elements): zero-pads a LoRA factor to a rank multiple of 16, or crops a result.
hipError_t launch_copy2d_u16(const uint16_t *in, int64_t in_rows, int64_t in_cols, uint16_t *out, int64_t out_rows,
                             int64_t out_cols, hipStream_t stream);

// out[m, r] = bf16(scale * sum_c x[m, c] * rmat[r, c]); x [m, cols], rmat [rank, cols] bf16,
// rank a multiple of 16 (any number of 128-row slices).
hipError_t launch_lora_down(const uint16_t *x, int64_t m, int64_t cols, const uint16_t *rmat,
                            int rank, float scale, uint16_t *out, hipStream_t stream);
// Two such projections sharing m and rank in one launch (x1 == nullptr: only the first).
hipError_t launch_lora_down2(const uint16_t *x0, int64_t cols0, const uint16_t *rmat0, float scale0, uint16_t *out0,
                             const uint16_t *x1, int64_t cols1, const uint16_t *rmat1, float scale1, uint16_t *out1,
                             int64_t m, int rank, hipStream_t stream);

// Token reduction: part[s, a, b] = sum over the tokens of split s of p[t, a] * q[t, b]
// (p [m, pa] the wide operand, q [m, qb] the narrow one, qb a multiple of 16; bf16), then
// out[a, b] (or out[b, a] when transposed) = bf16(scale * sum_s part[s, a, b]).
// The tokens are cut into `splits` (1..16) equal runs; lora_grad_splits picks it
// from the token count and the launch's workgroups per split (lora_grad_tiles of
// the two jobs' widths pa0, pa1 and qb), and the partials hold that many slices.
int64_t lora_grad_tiles(int64_t pa0, int64_t pa1, int64_t qb);
int lora_grad_splits(int64_t m, int64_t tiles);
hipError_t launch_lora_grad(const uint16_t *p, int64_t pa, const uint16_t *q, int64_t qb, int64_t m,
                            float scale, bool transposed, float *partials, uint16_t *out, int splits,
                            hipStream_t stream);
// Two such reductions sharing m and qb in one launch each for the partials and
// the sums (p1 == nullptr: only the first); each job has its own partials.
hipError_t launch_lora_grad2(const uint16_t *p0, int64_t pa0, const uint16_t *q0, float scale0, bool transposed0,
                             float *partials0, uint16_t *out0, const uint16_t *p1, int64_t pa1, const uint16_t *q1,
                             float scale1, bool transposed1, float *partials1, uint16_t *out1, int64_t qb, int64_t m,
                             int splits, hipStream_t stream);

// Rotate (block g along the tokens) + per-feature int8 quantization of two
// operands sharing the token count m, each x [m, f] bf16 read as it is: q [f, m]
// (the codes of x^T) and scale [f].  colmax [f0 + f1] is scratch, zero on entry.
// m is a multiple of 16 and of g, f0 and f1 of 16 (f1 may be 0).
hipError_t launch_colq_pair(const uint16_t *x0, int64_t f0, int8_t *q0, float *s0, const uint16_t *x1, int64_t f1,
                            int8_t *q1, float *s1, int64_t m, int g, uint32_t *colmax, hipStream_t stream);

// Low-rank (SVD) split of w [n, k] with rank in {16, 32, 64}, then rotate + int8
// quantization of the binary32 residual.  The workspace holds the residual [n, k]
// (binary32) at offset 0 and the orthonormal basis Q [n, rank] (fp64) at
// svd_workspace_q_offset() when the call returns.
size_t svd_workspace_bytes(int64_t n, int64_t k, int rank);
size_t svd_workspace_q_offset(int64_t n, int64_t k, int rank);
hipError_t launch_svd_quantize_weight(const uint16_t *w, int64_t n, int64_t k, int g, int rank, int steps,
                                      const float *omega, int8_t *qw, float *w_scale, uint16_t *svd_a,
                                      uint16_t *svd_b, void *workspace, hipStream_t stream);

// Int8 Q K^T attention (q [B, Hq, Sq, D], k, v [B, Hkv, Sk, D] bf16, D in {64, 128},
// Sk % 16 == 0).  The workspace holds, in order, q codes [B, Hq, Sq, D], q scales,
// k codes [B, Hkv, Sk, D], k scales, the K mean [B, Hkv, D] and the hand-over
// status word (uint32) at the six offsets attention_workspace_offsets() returns,
// then scratch.
size_t attention_workspace_bytes(int64_t bsz, int64_t hq, int64_t hkv, int64_t sq, int64_t sk, int64_t d);
void attention_workspace_offsets(int64_t bsz, int64_t hq, int64_t hkv, int64_t sq, int64_t sk, int64_t d,
                                 size_t *offsets);
hipError_t launch_attention_int8(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t bsz, int64_t hq,
                                 int64_t hkv, int64_t sq, int64_t sk, int64_t d, bool causal, float scale,
                                 bool smooth_k, int g, uint16_t *out, void *workspace, hipStream_t stream);

}  // namespace sdnq
