/*
 * sdnq_hip.h -- C ABI of the Hadamard-rotated INT8 quantized linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is the SDNQ Hadamard path used by ConvRot:
 *  - "ConvRot / Hadamard SDNQ" (SimpleTuner docs), "What The Options Do": the
 *    weight is rotated block-wise along in-features with block size
 *    hadamard_group_size (256 for ConvRot, smaller blocks for the QuaRot-style
 *    path) and quantized to int8 with static full-row scales (group_size -1);
 *    the int8 quantized matmul stays active; "PEFT Behavior": LoRA adapters stay
 *    trainable in bf16 on the frozen int8 base.
 *  - "SDNQ: SD.Next Quantization Engine", feature list: Hadamard rotation on the
 *    quantized weights and on the quantized matmul, INT8 quantized matmul;
 *    SDNQConfig example: dequantize_fp32 keeps scales and dequantization in FP32;
 *    quantized-training example: the quantized matmul runs in the backward pass.
 *  - HSWQ README, "Rigorous grid / pack simulation": ConvRot INT8 is "Hadamard
 *    rotate, then channelwise absmax" on a symmetric INT8 grid.
 *
 * Definitions used throughout (the pages give the method in words only; these
 * are the readings this library implements):
 *  - H_g: the g x g Sylvester Hadamard matrix in natural order; the rotation of a
 *    row multiplies each contiguous block of g values by H_g and by fl32(1/sqrt(g)),
 *    evaluated as an in-place fp32 butterfly with stages h = 1, 2, ..., g/2, each
 *    pair (i, i+h) becoming (a+b, a-b).  g = 1 means no rotation.
 *  - row quantization: a = max |y| over the whole row, scale s = fl32(a/127),
 *    r = fl32(127/a) (0 if a == 0), code = round-half-even(fl32(y*r)) clamped to
 *    [-127, 127].  A row with a < 2^-100 is first multiplied by 2^100 (exact), so
 *    that r stays finite; s is always fl32(a/127) of the row as given.
 *
 * Conventions for every entry point:
 *  - All tensors are row-major and contiguous.  bf16 tensors are passed as
 *    uint16_t bit patterns.  Every pointer is a DEVICE pointer.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on `stream` and returns; it never allocates, frees or
 *    synchronizes and keeps no state between calls, so calls on different
 *    streams with disjoint buffers may run concurrently.
 *  - The caller owns every buffer, including the workspace.
 *  - Argument checks run before anything is enqueued: a call that returns an
 *    error has written nothing.  Errors raised by a kernel that already started
 *    (a memory fault on a bad pointer) surface at the caller's next
 *    synchronization, as with any HIP kernel.
 *  - Shape limits: m >= 0; n, k >= 1; every feature dimension (k, n) of the
 *    linear layer must be a multiple of 16 and at most 133136, so that
 *    127*127*K stays below 2^31 (exact int32 accumulators); k % g == 0.  Rows
 *    of up to 65536 values are rotated and quantized with the whole row on
 *    chip; longer rows in equal segments of whole blocks, in two passes (the
 *    row's absmax first, then the codes).  The weight gradient, the low-rank
 *    split and the attention keep their own limits (below).
 *  - m == 0 is an empty batch: pointers to buffers with m rows may be NULL, nothing
 *    is read, and the only work enqueued is zeroing grad_a / grad_b when the
 *    backward pass requests them (empty sums).
 *  - Alignment: every pointer must be 16-byte aligned.
 *  - LoRA rank: any rank in [1, 256] with both factors given; rank is ignored
 *    when both factors are NULL (no adapter).  Ranks that are not a multiple of
 *    16 run on zero-padded copies of the factors in the workspace (the padding
 *    adds exact zeros to every sum).
 *  - Non-finite inputs (NaN, Inf) give unspecified outputs; they are not checked.
 */
#ifndef SDNQ_HIP_H
#define SDNQ_HIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SDNQ_OK = 0,
    SDNQ_ERR_INVALID_ARG = 1,  /* null required pointer, negative or zero size, misaligned pointer */
    SDNQ_ERR_UNSUPPORTED = 2,  /* g not in {1,64,128,256}, k % g != 0, a feature dimension not a
                                  multiple of 16 or above its limit, LoRA rank outside [1, 256] */
    SDNQ_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than sdnq_workspace_bytes() */
    SDNQ_ERR_LAUNCH = 4        /* a kernel launch was rejected by the HIP runtime */
} sdnq_status_t;

/* Offline weight preparation: rotate each row of w[n,k] (bf16) along k with block
 * g, then quantize each row with its own absmax scale.
 *   out: qw[n,k] int8 codes, w_scale[n] fp32 (the full-row static scale). */
sdnq_status_t sdnq_rotate_quantize_weight(const uint16_t *w, int64_t n, int64_t k, int32_t g,
                                          int8_t *qw, float *w_scale, void *stream);

/* Run-time activation quantization: for each token (row) of x[m,k] (bf16),
 * optionally multiply column j by col_scale[j] (fp32, nullable; used by the
 * backward pass to fold the weight row scales into dY, with g = 1), rotate with
 * block g, then quantize the row with its own absmax scale (per-token).
 *   out: qx[m,k] int8, x_scale[m] fp32. */
sdnq_status_t sdnq_rotate_quantize_act(const uint16_t *x, int64_t m, int64_t k, int32_t g,
                                       const float *col_scale, int8_t *qx, float *x_scale,
                                       void *stream);

/* Forward of the quantized linear layer:
 *   y[m,n] = bf16( fp32(rotq(x) . qw^T) * x_scale[m] * w_scale[n]
 *                  + lora_scale * ((x lora_a) lora_b)[m,n] )
 * x[m,k] bf16; qw[n,k] int8 and w_scale[n] fp32 from sdnq_rotate_quantize_weight
 * with the same g; lora_a[k,rank] and lora_b[rank,n] bf16 (both NULL and rank 0
 * for no adapter; the adapter sees the unrotated x); y[m,n] bf16.
 * The int8 x codes and the int32 accumulators never leave the GPU's workspace and
 * registers; the LoRA factor lora_scale * (x lora_a) is rounded to bf16 in the workspace.
 * workspace: at least sdnq_workspace_bytes(m, n, k, rank, 0) bytes. */
sdnq_status_t sdnq_qlinear_forward(const uint16_t *x, int64_t m, int64_t k,
                                   const int8_t *qw, const float *w_scale, int64_t n, int32_t g,
                                   const uint16_t *lora_a, const uint16_t *lora_b, int32_t rank,
                                   float lora_scale, uint16_t *y,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Forward from activations that are already rotated and quantized (qx, x_scale
 * from sdnq_rotate_quantize_act with the weight's g): the int8 GEMM with its fused
 * dequantization epilogue.  t[m,rank] (bf16, = x lora_a) and lora_b[rank,n] are
 * nullable; when given, t . bf16(lora_scale * lora_b) is added (exactly
 * lora_scale * (t lora_b) when lora_scale is a power of two).
 * workspace: at least sdnq_workspace_bytes(m, n, k, rank, 0) bytes. */
sdnq_status_t sdnq_qlinear_forward_quantized(const int8_t *qx, const float *x_scale, int64_t m,
                                             int64_t k, const int8_t *qw, const float *w_scale,
                                             int64_t n, const uint16_t *t, const uint16_t *lora_b,
                                             int32_t rank, float lora_scale, uint16_t *y,
                                             void *workspace, size_t workspace_bytes,
                                             void *stream);

/* Input gradient of the layer, through the same int8 weight (PEFT backward):
 *   dY'      = dy[m,n] * w_scale[n]            (column-wise fold of the row scales)
 *   q, s     = per-token int8 quantization of dY' (no rotation along n)
 *   dx[m,k]  = bf16( R_g( fp32(q . qw) * s[m] ) + lora_scale * (dy lora_b^T) lora_a^T )
 * where R_g is the normalized block rotation along k (symmetric and orthogonal,
 * hence its own inverse).  When grad_a / grad_b are non-NULL (LoRA present):
 *   grad_a[k,rank] = bf16( x^T (lora_scale * dy lora_b^T) )
 *   grad_b[rank,n] = bf16( lora_scale * (x lora_a)^T dy )
 * x[m,k] bf16 is read only for grad_a / grad_b.  The LoRA factors are rounded to
 * bf16 in the workspace.  workspace: at least sdnq_workspace_bytes(m, n, k, rank, 1). */
sdnq_status_t sdnq_qlinear_backward_input(const uint16_t *dy, int64_t m, int64_t n,
                                          const int8_t *qw, const float *w_scale, int64_t k,
                                          int32_t g, const uint16_t *x, const uint16_t *lora_a,
                                          const uint16_t *lora_b, int32_t rank, float lora_scale,
                                          uint16_t *dx, uint16_t *grad_a, uint16_t *grad_b,
                                          void *workspace, size_t workspace_bytes, void *stream);

/* Byte transpose of weight codes (int8 or E4M3): out[cols, rows] = in[rows, cols]^T,
 * rows and cols multiples of 16, at most 133136; in and out 16-byte aligned, not
 * overlapping.  The input gradient reads the codes across their rows; during
 * adapter training the quantized weight is frozen ("ConvRot / Hadamard SDNQ",
 * "PEFT Behavior": the adapter trains on top of the frozen quantized base), so
 * the transpose can be made once, next to sdnq_rotate_quantize_weight, and
 * passed to sdnq_qlinear_backward_input_wt. */
sdnq_status_t sdnq_transpose_codes(const uint8_t *in, int64_t rows, int64_t cols, uint8_t *out, void *stream);

/* sdnq_qlinear_backward_input with the weight codes given transposed: qw_t[k,n] =
 * qw^T (sdnq_transpose_codes(qw, n, k, qw_t)).  Same arguments otherwise, same
 * results bit for bit, same limits, errors and workspace size; the call skips
 * its per-call transpose of qw. */
sdnq_status_t sdnq_qlinear_backward_input_wt(const uint16_t *dy, int64_t m, int64_t n,
                                             const int8_t *qw_t, const float *w_scale, int64_t k,
                                             int32_t g, const uint16_t *x, const uint16_t *lora_a,
                                             const uint16_t *lora_b, int32_t rank, float lora_scale,
                                             uint16_t *dx, uint16_t *grad_a, uint16_t *grad_b,
                                             void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): sdnq_qlinear_forward
 * with the same arguments and results, minus the workspace, which comes from a
 * fixed SDNQ_NOALLOC_SCRATCH_BYTES device array that the library holds on each
 * device it runs on until the process ends.  Nothing is allocated or freed.
 * Returns SDNQ_ERR_WORKSPACE, before any launch, when the call would need more
 * than that (sdnq_workspace_bytes(m, n, k, rank, 0) > SDNQ_NOALLOC_SCRATCH_BYTES),
 * and SDNQ_ERR_LAUNCH if the array's device address cannot be obtained.  Every
 * call on a device shares that device's array: calls that overlap on one device
 * (concurrent streams, other host threads) race and must be serialized by the
 * caller; consecutive calls on one stream are safe. */
#define SDNQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
sdnq_status_t sdnq_qlinear_forward_noalloc(const uint16_t *x, int64_t m, int64_t k,
                                           const int8_t *qw, const float *w_scale, int64_t n, int32_t g,
                                           const uint16_t *lora_a, const uint16_t *lora_b, int32_t rank,
                                           float lora_scale, uint16_t *y, void *stream);

/* Workspace size in bytes for sdnq_qlinear_forward(_quantized) (is_backward = 0) or
 * sdnq_qlinear_backward_input (is_backward = 1) at these sizes; 0 on invalid sizes. */
size_t sdnq_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t rank, int32_t is_backward);

/* Static, NUL-terminated description of a status code. */
const char *sdnq_status_string(sdnq_status_t status);

/* Diagnostics: the int8 GEMM of the layer with an int32 store instead of the
 * dequantization epilogue (the accumulators the forward uses, exact).
 *   b_layout 0: a[m,k], b[n,k] -> c[m,n] = a . b^T   (forward orientation)
 *   b_layout 1: a[m,k], b[k,n] -> c[m,n] = a . b     (backward orientation; b is
 *               transposed through the workspace first)
 * workspace: b_layout 1 needs k*n bytes, b_layout 0 none (may be NULL). */
sdnq_status_t sdnq_gemm_i8_i32(const int8_t *a, const int8_t *b, int64_t m, int64_t n, int64_t k,
                               int32_t b_layout, int32_t *c, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Diagnostics: the rate ceiling of the forward GEMM kernel on the device it runs
 * on.  Launches the kernel sdnq_qlinear_forward_quantized launches for these
 * arguments without LoRA (same tiles, prologue and dequantization epilogue, same
 * argument checks), with parts of its k loop removed:
 *   mode 0: nothing removed; y is exactly sdnq_qlinear_forward_quantized's y;
 *   mode 1: no global loads after the first two k-tiles: every k-tile multiplies
 *           what those two left in LDS (y is meaningless);
 *   mode 2: also no LDS reads: every MFMA multiplies the fragments of the first
 *           k-step, held in registers (y is meaningless);
 *   mode 3: as mode 2, with fragments made of the loop indices instead of the
 *           codes (y is meaningless).
 * Mode 2 issues the same MFMA instructions on operand bytes of the real codes
 * with no data movement in the k loop: the kernel's rate on the device's clock
 * and power budget when nothing but the matrix cores work.  Mode 3 shows how much
 * of that power the operands' bit patterns draw.  SDNQ_ERR_INVALID_ARG for a mode
 * outside 0..3; the other errors as sdnq_qlinear_forward_quantized. */
sdnq_status_t sdnq_gemm_i8_ceiling(const int8_t *qx, const float *x_scale, int64_t m, int64_t k,
                                   const int8_t *qw, const float *w_scale, int64_t n, int32_t mode,
                                   uint16_t *y, void *stream);

/* Weight gradient through the quantized matmul (full fine-tuning: "SDNQ: SD.Next
 * Quantization Engine", the training example runs the quantized matmul in the
 * backward pass and the feature list includes full-parameter quantized training):
 *   dw[n,k] = bf16( fp32(q_dy . q_x^T) * s_dy[n] * s_x[k] )
 * where the contraction runs over the m tokens, so both operands are quantized
 * along the tokens: (q_dy, s_dy) = sdnq_rotate_quantize_act applied to the rows of
 * dy^T [n,m] and (q_x, s_x) to the rows of x^T [k,m], each rotated with block g
 * along the tokens (the rotation is orthogonal along the contracted axis, so it
 * cancels in the product) and quantized with one scale per feature.
 * dy[m,n], x[m,k] bf16 (the layer's output gradient and input); dw[n,k] bf16.
 * m is a contraction length here: a multiple of 16, at most 65536, m % g == 0;
 * m == 0 writes zeros.  workspace: sdnq_weight_grad_workspace_bytes(m, n, k). */
sdnq_status_t sdnq_qlinear_weight_grad(const uint16_t *dy, const uint16_t *x, int64_t m, int64_t n, int64_t k,
                                       int32_t g, uint16_t *dw, void *workspace, size_t workspace_bytes,
                                       void *stream);

/* Workspace size in bytes for sdnq_qlinear_weight_grad; 0 on invalid sizes. */
size_t sdnq_weight_grad_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* Byte offset in that workspace of: 0 q_dy [n,m] (int8), 1 s_dy [n] (fp32),
 * 2 q_x [k,m] (int8), 3 s_x [k] (fp32), which hold the quantized operands once the
 * call has completed; 0 on invalid arguments. */
size_t sdnq_weight_grad_workspace_offset(int64_t m, int64_t n, int64_t k, int32_t which);

/* ---------------------------------------------------------------- FP8 ------
 * The FP8 variant of the quantized matmul ("SDNQ: SD.Next Quantization Engine":
 * INT8 and FP8 quantized matmul; the SDNQConfig example's matmul dtype
 * float8_e4m3fn).  Same rotation and row absmax as the INT8 path, with
 *   s = fl32(a/448), r = fl32(448/a), code = E4M3(clamp(fl32(y*r), -448, 448)),
 * E4M3 being the OCP FP8 format (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, subnormals, largest finite 448), rounded to nearest, ties to even.  Codes
 * are passed as uint8_t bit patterns.  The GEMM accumulates the products of the
 * decoded codes in fp32 (MFMA order), so its results match the exact sum within
 * fp32 accumulation error rather than bit for bit.  Shapes, alignment, limits,
 * errors and workspace sizes are those of the INT8 entry points. */

/* Weight preparation: qw[n,k] E4M3 codes, w_scale[n] fp32. */
sdnq_status_t sdnq_rotate_quantize_weight_fp8(const uint16_t *w, int64_t n, int64_t k, int32_t g,
                                              uint8_t *qw, float *w_scale, void *stream);

/* Per-token activation quantization: qx[m,k] E4M3 codes, x_scale[m] fp32
 * (col_scale as for sdnq_rotate_quantize_act, nullable). */
sdnq_status_t sdnq_rotate_quantize_act_fp8(const uint16_t *x, int64_t m, int64_t k, int32_t g,
                                           const float *col_scale, uint8_t *qx, float *x_scale,
                                           void *stream);

/* Forward: y[m,n] = bf16( fp32(dec(rotq8(x)) . dec(qw)^T) * x_scale[m] * w_scale[n]
 *                         + lora_scale * ((x lora_a) lora_b)[m,n] ),
 * arguments as for sdnq_qlinear_forward with E4M3 weight codes.
 * workspace: at least sdnq_workspace_bytes(m, n, k, rank, 0) bytes. */
sdnq_status_t sdnq_qlinear_forward_fp8(const uint16_t *x, int64_t m, int64_t k,
                                       const uint8_t *qw, const float *w_scale, int64_t n, int32_t g,
                                       const uint16_t *lora_a, const uint16_t *lora_b, int32_t rank,
                                       float lora_scale, uint16_t *y,
                                       void *workspace, size_t workspace_bytes, void *stream);

/* Forward from E4M3 activations (qx, x_scale from sdnq_rotate_quantize_act_fp8 with
 * the weight's g), arguments as for sdnq_qlinear_forward_quantized. */
sdnq_status_t sdnq_qlinear_forward_fp8_quantized(const uint8_t *qx, const float *x_scale, int64_t m,
                                                 int64_t k, const uint8_t *qw, const float *w_scale,
                                                 int64_t n, const uint16_t *t, const uint16_t *lora_b,
                                                 int32_t rank, float lora_scale, uint16_t *y,
                                                 void *workspace, size_t workspace_bytes,
                                                 void *stream);

/* Input gradient through E4M3 weight codes (the SDNQ README's quantized training
 * runs the quantized matmul in the backward pass too):
 *   dY'      = dy[m,n] * w_scale[n]             (column-wise fold of the row scales)
 *   q, s     = per-token E4M3 quantization of dY' (no rotation along n)
 *   dx[m,k]  = bf16( R_g( fp32(dec(q) . dec(qw)) * s[m] ) + lora_scale * (dy lora_b^T) lora_a^T )
 * and grad_a / grad_b as for sdnq_qlinear_backward_input, whose arguments,
 * limits, errors and workspace size (sdnq_workspace_bytes(m, n, k, rank, 1))
 * this takes, with qw[n,k] the E4M3 codes of sdnq_rotate_quantize_weight_fp8. */
sdnq_status_t sdnq_qlinear_backward_input_fp8(const uint16_t *dy, int64_t m, int64_t n,
                                              const uint8_t *qw, const float *w_scale, int64_t k,
                                              int32_t g, const uint16_t *x, const uint16_t *lora_a,
                                              const uint16_t *lora_b, int32_t rank, float lora_scale,
                                              uint16_t *dx, uint16_t *grad_a, uint16_t *grad_b,
                                              void *workspace, size_t workspace_bytes, void *stream);

/* sdnq_qlinear_backward_input_fp8 with the E4M3 codes given transposed, qw_t[k,n]
 * (sdnq_transpose_codes), as sdnq_qlinear_backward_input_wt is to
 * sdnq_qlinear_backward_input. */
sdnq_status_t sdnq_qlinear_backward_input_fp8_wt(const uint16_t *dy, int64_t m, int64_t n,
                                                 const uint8_t *qw_t, const float *w_scale, int64_t k,
                                                 int32_t g, const uint16_t *x, const uint16_t *lora_a,
                                                 const uint16_t *lora_b, int32_t rank, float lora_scale,
                                                 uint16_t *dx, uint16_t *grad_a, uint16_t *grad_b,
                                                 void *workspace, size_t workspace_bytes, void *stream);

/* Diagnostics: the FP8 GEMM with an fp32 store instead of the epilogue:
 * c[m,n] = sum_k dec(a[m,k]) * dec(b[n,k]), fp32 accumulation. */
sdnq_status_t sdnq_gemm_fp8_f32(const uint8_t *a, const uint8_t *b, int64_t m, int64_t n, int64_t k,
                                float *c, void *stream);

/* ------------------------------------------------- low-rank (SVD) split ------
 * SVD quantization ("SDNQ: SD.Next Quantization Engine": SVD quantization next to
 * the Hadamard rotation; SDNQConfig use_svd, svd_rank = 32, svd_steps = 8; the
 * SD.Next dev-branch commit log: a seeded SVD truncation, so the quantized weight
 * is integer codes plus low-rank factors).  The pages give no algorithm; this is
 * the randomized range finder with subspace iteration:
 *   Q = orth(w omega); `steps` times: Z = orth(w^T Q), Q = orth(w Z);
 *   svd_a[k,rank] = bf16(w^T Q), svd_b[rank,n] = bf16(Q^T)   (round to nearest even)
 *   residual[n,k] = fl32(w - svd_b^T svd_a^T)   (fp64 sum of the rounded factors)
 *   qw[n,k], w_scale[n] = rotation (block g) + row quantization of the residual,
 *   with the binary32 steps of sdnq_rotate_quantize_weight.
 * orth() is an orthonormal basis of the same span (computed in fp64 by shifted
 * CholeskyQR; where w omega is rank-deficient, the extra columns are arbitrary
 * directions that add nothing to the projection Q Q^T w).
 * The layer then runs as sdnq_qlinear_forward(x, ..., qw, w_scale, n, g,
 * lora_a = svd_a, lora_b = svd_b, rank, lora_scale = 1, ...).
 * w[n,k] bf16; omega[k,rank] fp32, the random test matrix (N(0,1) entries; the
 * caller draws it, so the split is reproducible from its seed); rank in {16, 32,
 * 64} and at most min(n, k); 0 <= steps <= 64; n and k multiples of 16, at most
 * 65536; k % g == 0.  Offline weight preparation: it reads w about 2 (steps + 1)
 * times and runs small fp64 kernels in between.
 * workspace: sdnq_svd_workspace_bytes(n, k, rank) bytes, 16-byte aligned.  When
 * the call's work has completed, the workspace holds the binary32 residual [n,k]
 * at offset 0 and Q [n,rank] (fp64) at sdnq_svd_workspace_q_offset(n, k, rank). */
sdnq_status_t sdnq_svd_quantize_weight(const uint16_t *w, int64_t n, int64_t k, int32_t g, int32_t rank,
                                       int32_t steps, const float *omega, int8_t *qw, float *w_scale,
                                       uint16_t *svd_a, uint16_t *svd_b, void *workspace, size_t workspace_bytes,
                                       void *stream);

/* Workspace size in bytes for sdnq_svd_quantize_weight; 0 on invalid sizes. */
size_t sdnq_svd_workspace_bytes(int64_t n, int64_t k, int32_t rank);

/* Byte offset of Q [n,rank] (fp64) in that workspace; 0 on invalid sizes. */
size_t sdnq_svd_workspace_q_offset(int64_t n, int64_t k, int32_t rank);

/* ------------------------------------------------------ int8 attention ------
 * The quantized attention of "SDNQ: SD.Next Quantization Engine" (its
 * SDPA-replacement example: Q K^T as an int8 quantized matmul, P V unquantized,
 * smooth_k, use_hadamard with hadamard_group_size, quantize_fp32, and SDPA's
 * is_causal, scale and enable_gqa).  The pages name the options only; readings:
 *  - q[batch, heads_q, seq_q, head_dim], k and v[batch, heads_kv, seq_k, head_dim],
 *    out like q, all bf16; query head h reads key/value head h / (heads_q / heads_kv);
 *  - smooth_k != 0: K minus its mean over the key tokens per (batch, head,
 *    channel), K' = fl32(k - mean).  The mean is the exact mean of the bf16 keys
 *    rounded once to binary32 wherever a binary64 sum of the channel is exact
 *    (sum |k| < 2^53 times the finest last-place unit among its nonzero keys,
 *    which holds for any realistic activations): the sum is taken in binary64
 *    (64-token blocks, then the block sums), divided once in binary64 and
 *    rounded to binary32.  Outside that domain the binary64 sum's error bound
 *    applies;
 *  - hadamard_group g in {64, 128, 256}: Q and K' rows are rotated with block
 *    min(g, head_dim) (the butterfly and normalization above); g = 0 or 1: none;
 *  - Q and K' are quantized per token (one scale per row over head_dim) with the
 *    row quantization above;
 *  - scores = fp32(int32 q . k) * s_q * s_k * scale (scale > 0; the usual value is
 *    1/sqrt(head_dim)); is_causal != 0 masks keys j > i (top-left aligned);
 *  - softmax, then P V with P rounded to bf16 and fp32 accumulation; bf16 out.
 * head_dim in {64, 128}; seq_k a multiple of 16; seq_q, seq_k <= 2^20;
 * batch * heads_q and batch * heads_kv <= 65535; batch * heads * seq <= 2^31 for
 * q and for k; heads_q % heads_kv == 0.
 * workspace: sdnq_attention_workspace_bytes(...) bytes, 16-byte aligned.  When the
 * work has completed it holds the q codes [batch, heads_q, seq_q, head_dim] (int8),
 * q scales (fp32), k codes, k scales and the K mean [batch, heads_kv, head_dim]
 * (fp32) at sdnq_attention_workspace_offset(..., which = 0 .. 4), and at which = 5
 * a uint32 status word: 0, or nonzero if a query tile whose keys two workgroups
 * shared was finished without the other workgroup's share (its bounded wait ran
 * out; that wait is only ever on a workgroup already past its key loop, so a
 * nonzero word means the device stalled a running workgroup for about a second).
 * Non-causal calls whose query tiles overfill the resident workgroups by at most
 * a sixth of a round share tiles that way; the result does not depend on which
 * workgroups are resident together. */
sdnq_status_t sdnq_attention_int8(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t batch,
                                  int64_t heads_q, int64_t heads_kv, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                                  int32_t is_causal, float scale, int32_t smooth_k, int32_t hadamard_group,
                                  uint16_t *out, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace size in bytes for sdnq_attention_int8; 0 on invalid sizes. */
size_t sdnq_attention_workspace_bytes(int64_t batch, int64_t heads_q, int64_t heads_kv, int64_t seq_q,
                                      int64_t seq_k, int64_t head_dim);

/* Byte offset in that workspace of: 0 q codes, 1 q scales, 2 k codes, 3 k scales,
 * 4 K mean, 5 the status word; 0 on invalid arguments. */
size_t sdnq_attention_workspace_offset(int64_t batch, int64_t heads_q, int64_t heads_kv, int64_t seq_q,
                                       int64_t seq_k, int64_t head_dim, int32_t which);

/* Test hook for the status word above: the bound of the shared-tile wait, in polls
 * of about 64 clocks, for sdnq_attention_int8 calls enqueued after this one, in
 * this process, on every device.  The default is SDNQ_ATTENTION_HANDOVER_POLLS
 * (about a second); pass it to restore.  With 0 the wait gives up before its
 * first poll: every shared tile is finished with whatever its partner's share
 * holds by then and the status word is set, while every kernel still exits
 * normally.  Always SDNQ_OK. */
#define SDNQ_ATTENTION_HANDOVER_POLLS 16777216u
sdnq_status_t sdnq_attention_set_handover_polls(uint32_t polls);

#ifdef __cplusplus
}
#endif

#endif /* SDNQ_HIP_H */
