/*
 * CPU oracle for the Hadamard-rotated INT8 quantized linear layer
 * (the SDNQ Hadamard path that ConvRot uses).
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the
 * benchmark's CPU-baseline leg are the only users.  The GPU library never links,
 * loads or calls this file, and this file includes nothing from the GPU library.
 *
 * Plain, slow and written to be read against the sources:
 *  - "ConvRot / Hadamard SDNQ" (SimpleTuner docs), section "What The Options Do":
 *    the rotation is block-wise along in-features with block size
 *    hadamard_group_size (256 for ConvRot, smaller for the QuaRot-style path);
 *    sdnq_group_size -1 means one static scale per full weight row.
 *  - "SDNQ: SD.Next Quantization Engine", feature list and the SDNQConfig example:
 *    Hadamard rotation applies to quantized weights and to the quantized matmul;
 *    INT8 quantized matmul; group_size -1 is row-wise; dequantize_fp32 keeps
 *    the scales and the dequantization in FP32; the training example says the
 *    quantized matmul is used in the backward pass too.
 *  - HSWQ README (Hybrid-Sensitivity-Weighted-Quantization), "Rigorous grid /
 *    pack simulation": ConvRot INT8 is "Hadamard rotate, then channelwise
 *    absmax" on a symmetric INT8 grid.
 *  - "ConvRot / Hadamard SDNQ", "PEFT Behavior": the adapter stays in bf16 on top
 *    of the frozen int8 base.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - H_g is the Sylvester (natural order) Hadamard matrix, i.e. the output order
 *    of the in-place butterfly below; stages run h = 1, 2, 4, ..., g/2, each pair
 *    (i, i+h) becomes (a+b, a-b) in fp32, with no fused multiply-add.
 *  - normalization: every rotated value is multiplied by fl32(1/sqrt(g)).
 *  - absmax over the whole row; s = fl32(a/127); codes = clamp(rne(fl32(y*r)),
 *    -127, 127) with r = fl32(127/a) (0 when a == 0); rne = round half to even.
 *    For a < 2^-100, 127/a can overflow binary32, so such a row is scaled by
 *    2^100 (exactly) before r and the codes are formed.
 *  - activations: one scale per token (row of x) over all in-features.
 *  - backward: dY is multiplied column-wise by the weight row scales before its
 *    own per-token quantization (no rotation on that axis); the int32 product
 *    with the int8 weight is scaled by the dY token scale and rotated back with
 *    the same normalized block transform (it is symmetric and orthogonal).
 *  - the LoRA side path sees the unrotated x; A is [K,r], B is [r,N]; its terms are
 *    computed in fp64 from the bf16 values with no intermediate rounding.
 *
 * FP8 variant (the float8_e4m3fn quantized matmul that the SDNQ README lists next
 * to INT8): the same rotation and absmax, with s = fl32(a/448), r = fl32(448/a),
 * v = fl32(y*r) clamped to [-448, 448] and each v encoded in OCP FP8 E4M3
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
 * infinities, 0x7F/0xFF = NaN, largest finite 448) with round half to even; an
 * exact zero is stored as +0 (0x00), while nonzero values that round to zero
 * keep their sign.  The
 * product of two E4M3 values has at most 8 significant bits between 2^-18 and
 * 2^17.6, so the fp64 sum over K <= 65536 of them is exact.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fno-fast-math -fPIC -shared.
 * x86-64 floats use SSE: every float operation below is one IEEE binary32
 * operation rounded to nearest even.  OpenMP only splits independent rows or
 * output elements; it never changes an order of summation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_OVERFLOW 2

/* ---------------------------------------------------------------- bf16 -- */

/* bfloat16 bit pattern -> binary32: the bf16 bits are the high half. */
static float bf16_decode(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary64 -> bfloat16 (8 significant bits, exponent range of binary32),
 * round to nearest, ties to even, in a single rounding. */
static uint16_t bf16_encode_f64(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v))
        return 0x7FC0u;
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    int e;
    frexp(a, &e);              /* a = m * 2^e with m in [0.5, 1) */
    int ulp_exp = e - 8;       /* spacing of 8-significant-bit numbers near a */
    if (ulp_exp < -133)        /* bf16 subnormal spacing: 2^(-126-7) */
        ulp_exp = -133;
    double q = ldexp(a, -ulp_exp);          /* exact scaling by a power of two */
    double rq = nearbyint(q);               /* default mode: ties to even */
    double r = ldexp(rq, ulp_exp);
    if (r >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);  /* rounds past the largest finite value */
    float f = (float)r;                     /* exact: at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/* --------------------------------------------------- Walsh-Hadamard core -- */

static int is_pow2_upto256(int g)
{
    return g >= 1 && g <= 256 && (g & (g - 1)) == 0;
}

/* In-place unnormalized fast Walsh-Hadamard transform of one block of g floats:
 * u = H_g v with H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]].
 * Stages h = 1, 2, ..., g/2; each pair (i, i+h) with bit h of i clear becomes
 * (a + b, a - b), each one binary32 operation. */
static void fwht_block(float *v, int g)
{
    for (int h = 1; h < g; h <<= 1) {
        for (int i = 0; i < g; i++) {
            if ((i & h) == 0) {
                float a = v[i];
                float b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
}

/* c_g = fl32(1/sqrt(g)); 1 for g == 1 (no rotation). */
static float norm_const(int g)
{
    if (g == 1)
        return 1.0f;
    return (float)(1.0 / sqrt((double)g));
}

/* One row: decode bf16, optional column pre-scale, block rotation along the row,
 * normalization.  y receives the rotated binary32 values. */
static void rotate_row(const uint16_t *xr, int64_t cols, int g, const float *col_scale, float *y)
{
    for (int64_t i = 0; i < cols; i++) {
        y[i] = bf16_decode(xr[i]);
        if (col_scale)
            y[i] = y[i] * col_scale[i];
    }
    if (g > 1) {
        float c = norm_const(g);
        for (int64_t b = 0; b < cols; b += g)
            fwht_block(y + b, g);
        for (int64_t i = 0; i < cols; i++)
            y[i] = y[i] * c;
    }
}

/* Symmetric absmax quantization of one rotated row to int8 codes in [-127, 127].
 * A row whose absmax is below 2^-100 is first multiplied by 2^100 (exact for every
 * binary32 value), so that r = 127/a stays finite; s is always fl32(a/127) of the
 * row as given.  Rows at or above 2^-100 are used as they are (the factor is 1). */
static void quantize_row(const float *y, int64_t cols, int8_t *q, float *s)
{
    float a = 0.0f;
    for (int64_t i = 0; i < cols; i++)
        a = fmaxf(a, fabsf(y[i]));
    *s = a / 127.0f;
    float up = (a < 0x1p-100f) ? 0x1p100f : 1.0f;
    float as = a * up;
    float r = (as > 0.0f) ? 127.0f / as : 0.0f;
    for (int64_t i = 0; i < cols; i++) {
        float t = nearbyintf((y[i] * up) * r);
        if (t > 127.0f)
            t = 127.0f;
        if (t < -127.0f)
            t = -127.0f;
        q[i] = (int8_t)t;
    }
}

/* ---------------------------------------------------------- fp8 e4m3 -- */

/* Value of an E4M3 code: exponent field 0 holds subnormals m/8 * 2^-6, fields
 * 1..15 hold (1 + m/8) * 2^(e-7).  0x7F and 0xFF (NaN) are never produced here. */
static double e4m3_decode(uint8_t c)
{
    int e = (c >> 3) & 15, mant = c & 7;
    double v = e == 0 ? ldexp(mant / 8.0, -6) : ldexp(1.0 + mant / 8.0, e - 7);
    return (c & 0x80) ? -v : v;
}

/* E4M3 code of a finite binary32 v with |v| <= 448, rounded to nearest, ties to
 * even.  Scaling by a power of two is exact in double, so the only rounding is
 * the nearbyint of the mantissa (default rounding mode: half to even). */
static uint8_t e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a < 0x1p-6) {                      /* subnormal binade, steps of 2^-9 */
        double r = nearbyint(ldexp(a, 9)); /* 0 .. 8; 8 is the smallest normal 0x08 */
        return (uint8_t)(sign | (uint8_t)r);
    }
    int ex;
    frexp(a, &ex);                         /* a in [2^(ex-1), 2^ex) */
    int eu = ex - 1;                       /* unbiased exponent */
    double r = nearbyint(ldexp(a, 3 - eu)); /* 8 .. 16 mantissa units */
    if (r >= 16.0) {
        r = 8.0;
        eu += 1;
    }
    return (uint8_t)(sign | (uint8_t)((eu + 7) << 3) | (uint8_t)(r - 8.0));
}

/* The FP8 counterpart of quantize_row: s = fl32(a/448), codes e4m3(clamp(fl32(y*r))). */
static void quantize_row_fp8(const float *y, int64_t cols, uint8_t *q, float *s)
{
    float a = 0.0f;
    for (int64_t i = 0; i < cols; i++)
        a = fmaxf(a, fabsf(y[i]));
    *s = a / 448.0f;
    float up = (a < 0x1p-100f) ? 0x1p100f : 1.0f;
    float as = a * up;
    float r = (as > 0.0f) ? 448.0f / as : 0.0f;
    for (int64_t i = 0; i < cols; i++) {
        /* + 0.0f stores an exact zero as +0 (0x00): the sign of a zero that the
         * butterfly's cancellations produce depends on evaluation order, not on the
         * data.  Nonzero values that round to zero keep their sign. */
        float t = (y[i] * up) * r + 0.0f;
        if (t > 448.0f)
            t = 448.0f;
        if (t < -448.0f)
            t = -448.0f;
        q[i] = e4m3_encode(t);
    }
}

/* ----------------------------------------------------------- exports -- */

int oracle_num_threads(void)
{
    return omp_get_max_threads();
}

void oracle_set_num_threads(int n)
{
    if (n > 0)
        omp_set_num_threads(n);
}

/* Unnormalized butterfly on `nblocks` consecutive blocks of g floats, in place. */
int oracle_fwht_unnormalized(float *v, int64_t nblocks, int g)
{
    if (!v || nblocks < 0 || !is_pow2_upto256(g))
        return ORACLE_ERR_ARG;
    for (int64_t b = 0; b < nblocks; b++)
        fwht_block(v + b * g, g);
    return ORACLE_OK;
}

float oracle_norm_const(int g)
{
    return norm_const(g);
}

void oracle_bf16_from_f64(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = bf16_encode_f64(v[i]);
}

void oracle_f32_from_bf16(const uint16_t *h, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = bf16_decode(h[i]);
}

/* Rotation only (no quantization): y[rows, cols] binary32. */
int oracle_rotate(const uint16_t *x, int64_t rows, int64_t cols, int g, const float *col_scale, float *y)
{
    if (!x || !y || rows < 0 || cols < 0 || !is_pow2_upto256(g) || cols % g != 0)
        return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < rows; m++)
        rotate_row(x + m * cols, cols, g, col_scale, y + m * cols);
    return ORACLE_OK;
}

/* Rotate, then quantize each row: q[rows, cols] int8 and s[rows] binary32.
 * Weights (offline) and activations (per token) go through the same steps. */
int oracle_rotate_quantize(const uint16_t *x, int64_t rows, int64_t cols, int g,
                           const float *col_scale, int8_t *q, float *s)
{
    if (!x || !q || !s || rows < 0 || cols < 0 || !is_pow2_upto256(g) || cols % g != 0)
        return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel
    {
        float *y = (float *)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
        if (!y) {
#pragma omp atomic write
            err = ORACLE_ERR_ARG;
        } else {
#pragma omp for schedule(static)
            for (int64_t m = 0; m < rows; m++) {
                rotate_row(x + m * cols, cols, g, col_scale, y);
                quantize_row(y, cols, q + m * cols, s + m);
            }
            free(y);
        }
    }
    return err;
}

/* Rotate, then quantize rows given as binary32 values: the same steps as
 * oracle_rotate_quantize without the bf16 decode (and with no column scale).
 * The low-rank split forms its residual weight in binary32 and quantizes it
 * through this path. */
int oracle_rotate_quantize_f32(const float *x, int64_t rows, int64_t cols, int g, int8_t *q, float *s)
{
    if (!x || !q || !s || rows < 0 || cols < 0 || !is_pow2_upto256(g) || cols % g != 0)
        return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel
    {
        float *y = (float *)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
        if (!y) {
#pragma omp atomic write
            err = ORACLE_ERR_ARG;
        } else {
#pragma omp for schedule(static)
            for (int64_t m = 0; m < rows; m++) {
                for (int64_t i = 0; i < cols; i++)
                    y[i] = x[m * cols + i];
                if (g > 1) {
                    float c = norm_const(g);
                    for (int64_t b = 0; b < cols; b += g)
                        fwht_block(y + b, g);
                    for (int64_t i = 0; i < cols; i++)
                        y[i] = y[i] * c;
                }
                quantize_row(y, cols, q + m * cols, s + m);
            }
            free(y);
        }
    }
    return err;
}

/* Integer matmul with exact int64 accumulation, stored as int32.
 *   b_layout 0: a[m,k], b[n,k]  ->  c[i,j] = sum_t a[i,t] * b[j,t]
 *   b_layout 1: a[m,k], b[k,n]  ->  c[i,j] = sum_t a[i,t] * b[t,j]
 * Returns ORACLE_ERR_OVERFLOW if any sum leaves the int32 range. */
int oracle_gemm_i8(const int8_t *a, const int8_t *b, int64_t m, int64_t n, int64_t k,
                   int b_layout, int32_t *c)
{
    if (!a || !b || !c || m < 0 || n < 0 || k < 0 || (b_layout != 0 && b_layout != 1))
        return ORACLE_ERR_ARG;
    int overflow = 0;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; i++) {
        for (int64_t j = 0; j < n; j++) {
            int64_t acc = 0;
            for (int64_t t = 0; t < k; t++) {
                int64_t bv = b_layout == 0 ? b[j * k + t] : b[t * n + j];
                acc += (int64_t)a[i * k + t] * bv;
            }
            if (acc > INT32_MAX || acc < INT32_MIN) {
#pragma omp atomic write
                overflow = 1;
            }
            c[i * n + j] = (int32_t)acc;
        }
    }
    return overflow ? ORACLE_ERR_OVERFLOW : ORACLE_OK;
}

/* Forward of the quantized linear layer for the rows of x:
 *   q_x, s_x   = rotate + per-token quantize (x row, block g)
 *   acc[m,n]   = sum_k q_x[m,k] * qw[n,k]                (exact, int32 range checked)
 *   base[m,n]  = fl32(fl32(acc) * fl32(s_x[m] * s_w[n]))  (fp32 dequantization)
 *   lora[m,n]  = ((x A) B)[m,n] * lora_scale              (fp64, unrotated x)
 *   y[m,n]     = bf16_rne(base + lora)
 * lora_a / lora_b may be NULL (rank ignored).  Every *_out pointer may be NULL. */
int oracle_qlinear_forward(const uint16_t *x, int64_t m, int64_t k,
                           const int8_t *qw, const float *sw, int64_t n, int g,
                           const uint16_t *lora_a, const uint16_t *lora_b, int rank, double lora_scale,
                           uint16_t *y, int8_t *qx_out, float *sx_out, int32_t *acc_out, float *base_out)
{
    if (!x || !qw || !sw || !y || m < 0 || k <= 0 || n < 0 || !is_pow2_upto256(g) || k % g != 0)
        return ORACLE_ERR_ARG;
    int use_lora = lora_a && lora_b && rank > 0;
    int overflow = 0, alloc_fail = 0;
#pragma omp parallel
    {
        float *yr = (float *)malloc(sizeof(float) * (size_t)k);
        int8_t *qr = (int8_t *)malloc((size_t)k);
        double *t = (double *)malloc(sizeof(double) * (size_t)(rank > 0 ? rank : 1));
        if (!yr || !qr || !t) {
#pragma omp atomic write
            alloc_fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t i = 0; i < m; i++) {
                const uint16_t *xr = x + i * k;
                float sx;
                rotate_row(xr, k, g, NULL, yr);
                quantize_row(yr, k, qr, &sx);
                if (qx_out)
                    memcpy(qx_out + i * k, qr, (size_t)k);
                if (sx_out)
                    sx_out[i] = sx;
                if (use_lora) {
                    for (int j = 0; j < rank; j++)
                        t[j] = 0.0;
                    for (int64_t kk = 0; kk < k; kk++) {
                        double xv = (double)bf16_decode(xr[kk]);
                        for (int j = 0; j < rank; j++)
                            t[j] += xv * (double)bf16_decode(lora_a[kk * rank + j]);
                    }
                }
                for (int64_t j = 0; j < n; j++) {
                    const int8_t *wr = qw + j * k;
                    int64_t acc = 0;
                    for (int64_t kk = 0; kk < k; kk++)
                        acc += (int64_t)qr[kk] * (int64_t)wr[kk];
                    if (acc > INT32_MAX || acc < INT32_MIN) {
#pragma omp atomic write
                        overflow = 1;
                    }
                    float base = (float)(int32_t)acc * (sx * sw[j]);
                    if (acc_out)
                        acc_out[i * n + j] = (int32_t)acc;
                    if (base_out)
                        base_out[i * n + j] = base;
                    double out = (double)base;
                    if (use_lora) {
                        double l = 0.0;
                        for (int r = 0; r < rank; r++)
                            l += t[r] * (double)bf16_decode(lora_b[(int64_t)r * n + j]);
                        out += l * lora_scale;
                    }
                    y[i * n + j] = bf16_encode_f64(out);
                }
            }
        }
        free(yr);
        free(qr);
        free(t);
    }
    if (alloc_fail)
        return ORACLE_ERR_ARG;
    return overflow ? ORACLE_ERR_OVERFLOW : ORACLE_OK;
}

/* Gradient with respect to the layer input, through the same int8 weight:
 *   dY'[m,j]    = fl32(dY[m,j] * s_w[j])                     (fold the weight row scales)
 *   q_dy, s_dy  = per-token absmax quantization of dY' (no rotation: g = 1)
 *   acc[m,kk]   = sum_j q_dy[m,j] * qw[j,kk]                  (exact, int32 range checked)
 *   z[m,kk]     = fl32(fl32(acc) * s_dy[m])
 *   dxbase      = the forward's normalized block rotation applied to each row of z
 *   g_r         = dY B^T * lora_scale                         (fp64)
 *   dx          = bf16_rne(dxbase + g_r A^T)
 *   grad_a      = bf16_rne(x^T g_r)          [k, rank]
 *   grad_b      = bf16_rne((x A)^T dY * lora_scale)  [rank, n]
 * x is read only when grad_a or grad_b is requested.  dx may be NULL to compute the
 * LoRA gradients only.  Every *_out may be NULL. */
int oracle_qlinear_backward_input(const uint16_t *dy, int64_t m, int64_t n,
                                  const int8_t *qw, const float *sw, int64_t k, int g,
                                  const uint16_t *x, const uint16_t *lora_a, const uint16_t *lora_b,
                                  int rank, double lora_scale,
                                  uint16_t *dx, uint16_t *grad_a, uint16_t *grad_b,
                                  int8_t *qdy_out, float *sdy_out, int32_t *acc_out, float *dxbase_out)
{
    if (!dy || !qw || !sw || m < 0 || n <= 0 || k <= 0 || !is_pow2_upto256(g) || k % g != 0)
        return ORACLE_ERR_ARG;
    int use_lora = lora_a && lora_b && rank > 0;
    int want_grads = use_lora && (grad_a || grad_b);
    if (!dx && !want_grads)
        return ORACLE_ERR_ARG;
    if (want_grads && !x)
        return ORACLE_ERR_ARG;
    int overflow = 0, alloc_fail = 0;

    double *gr = NULL, *tx = NULL;
    if (use_lora) {
        gr = (double *)calloc((size_t)(m > 0 ? m : 1) * (size_t)rank, sizeof(double));
        if (!gr)
            return ORACLE_ERR_ARG;
        /* g_r[m, r] = sum_j dY[m, j] * B[r, j] * lora_scale */
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < m; i++) {
            for (int r = 0; r < rank; r++) {
                double acc = 0.0;
                for (int64_t j = 0; j < n; j++)
                    acc += (double)bf16_decode(dy[i * n + j]) * (double)bf16_decode(lora_b[(int64_t)r * n + j]);
                gr[i * rank + r] = acc * lora_scale;
            }
        }
    }

#pragma omp parallel if (dx)
    if (dx) {
        float *yr = (float *)malloc(sizeof(float) * (size_t)n);
        int8_t *qr = (int8_t *)malloc((size_t)n);
        float *z = (float *)malloc(sizeof(float) * (size_t)k);
        int64_t *acc = (int64_t *)malloc(sizeof(int64_t) * (size_t)k);
        if (!yr || !qr || !z || !acc) {
#pragma omp atomic write
            alloc_fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t i = 0; i < m; i++) {
                float sdy;
                rotate_row(dy + i * n, n, 1, sw, yr);
                quantize_row(yr, n, qr, &sdy);
                if (qdy_out)
                    memcpy(qdy_out + i * n, qr, (size_t)n);
                if (sdy_out)
                    sdy_out[i] = sdy;
                for (int64_t kk = 0; kk < k; kk++)
                    acc[kk] = 0;
                for (int64_t j = 0; j < n; j++) {
                    int64_t qv = qr[j];
                    const int8_t *wr = qw + j * k;
                    for (int64_t kk = 0; kk < k; kk++)
                        acc[kk] += qv * (int64_t)wr[kk];
                }
                for (int64_t kk = 0; kk < k; kk++) {
                    if (acc[kk] > INT32_MAX || acc[kk] < INT32_MIN) {
#pragma omp atomic write
                        overflow = 1;
                    }
                    if (acc_out)
                        acc_out[i * k + kk] = (int32_t)acc[kk];
                    z[kk] = (float)(int32_t)acc[kk] * sdy;
                }
                if (g > 1) {
                    float c = norm_const(g);
                    for (int64_t b = 0; b < k; b += g)
                        fwht_block(z + b, g);
                    for (int64_t kk = 0; kk < k; kk++)
                        z[kk] = z[kk] * c;
                }
                for (int64_t kk = 0; kk < k; kk++) {
                    if (dxbase_out)
                        dxbase_out[i * k + kk] = z[kk];
                    double out = (double)z[kk];
                    if (use_lora) {
                        double l = 0.0;
                        for (int r = 0; r < rank; r++)
                            l += gr[i * rank + r] * (double)bf16_decode(lora_a[kk * rank + r]);
                        out += l;
                    }
                    dx[i * k + kk] = bf16_encode_f64(out);
                }
            }
        }
        free(yr);
        free(qr);
        free(z);
        free(acc);
    }

    if (want_grads && !alloc_fail) {
        if (grad_a) {
            /* grad_a[kk, r] = sum_i x[i, kk] * g_r[i, r], summed over ascending i */
#pragma omp parallel
            {
                int nt = omp_get_num_threads(), id = omp_get_thread_num();
                int64_t k_lo = k * id / nt, k_hi = k * (id + 1) / nt;
                double *acc = (double *)calloc((size_t)((k_hi - k_lo) * rank + 1), sizeof(double));
                if (!acc) {
#pragma omp atomic write
                    alloc_fail = 1;
                } else {
                    for (int64_t i = 0; i < m; i++)
                        for (int64_t kk = k_lo; kk < k_hi; kk++) {
                            double xv = (double)bf16_decode(x[i * k + kk]);
                            for (int r = 0; r < rank; r++)
                                acc[(kk - k_lo) * rank + r] += xv * gr[i * rank + r];
                        }
                    for (int64_t kk = k_lo; kk < k_hi; kk++)
                        for (int r = 0; r < rank; r++)
                            grad_a[kk * rank + r] = bf16_encode_f64(acc[(kk - k_lo) * rank + r]);
                    free(acc);
                }
            }
        }
        if (grad_b) {
            tx = (double *)calloc((size_t)(m > 0 ? m : 1) * (size_t)rank, sizeof(double));
            if (!tx) {
                alloc_fail = 1;
            } else {
                /* t[i, r] = sum_kk x[i, kk] * A[kk, r] */
#pragma omp parallel for schedule(static)
                for (int64_t i = 0; i < m; i++) {
                    for (int64_t kk = 0; kk < k; kk++) {
                        double xv = (double)bf16_decode(x[i * k + kk]);
                        for (int r = 0; r < rank; r++)
                            tx[i * rank + r] += xv * (double)bf16_decode(lora_a[kk * rank + r]);
                    }
                }
                /* grad_b[r, j] = lora_scale * sum_i t[i, r] * dY[i, j], summed over ascending i */
#pragma omp parallel
                {
                    int nt = omp_get_num_threads(), id = omp_get_thread_num();
                    int64_t j_lo = n * id / nt, j_hi = n * (id + 1) / nt;
                    double *acc = (double *)calloc((size_t)((j_hi - j_lo) * rank + 1), sizeof(double));
                    if (!acc) {
#pragma omp atomic write
                        alloc_fail = 1;
                    } else {
                        for (int64_t i = 0; i < m; i++)
                            for (int r = 0; r < rank; r++) {
                                double tv = tx[i * rank + r];
                                for (int64_t j = j_lo; j < j_hi; j++)
                                    acc[(int64_t)r * (j_hi - j_lo) + (j - j_lo)] += tv * (double)bf16_decode(dy[i * n + j]);
                            }
                        for (int r = 0; r < rank; r++)
                            for (int64_t j = j_lo; j < j_hi; j++)
                                grad_b[(int64_t)r * n + j] =
                                    bf16_encode_f64(acc[(int64_t)r * (j_hi - j_lo) + (j - j_lo)] * lora_scale);
                        free(acc);
                    }
                }
            }
        }
    }
    free(gr);
    free(tx);
    if (alloc_fail)
        return ORACLE_ERR_ARG;
    return overflow ? ORACLE_ERR_OVERFLOW : ORACLE_OK;
}

/* ------------------------------------------------------- fp8 exports -- */

void oracle_e4m3_encode(const float *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = e4m3_encode(v[i]);
}

void oracle_e4m3_decode(const uint8_t *c, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = e4m3_decode(c[i]);
}

/* Rotate, then quantize each row to E4M3 codes: q[rows, cols] and s[rows]. */
int oracle_rotate_quantize_fp8(const uint16_t *x, int64_t rows, int64_t cols, int g,
                               const float *col_scale, uint8_t *q, float *s)
{
    if (!x || !q || !s || rows < 0 || cols < 0 || !is_pow2_upto256(g) || cols % g != 0)
        return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel
    {
        float *y = (float *)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
        if (!y) {
#pragma omp atomic write
            err = ORACLE_ERR_ARG;
        } else {
#pragma omp for schedule(static)
            for (int64_t m = 0; m < rows; m++) {
                rotate_row(x + m * cols, cols, g, col_scale, y);
                quantize_row_fp8(y, cols, q + m * cols, s + m);
            }
            free(y);
        }
    }
    return err;
}

/* E4M3 matmul, exact: c[i,j] = sum_t dec(a[i,t]) * dec(b[j,t]) in fp64 (a[m,k], b[n,k]). */
int oracle_gemm_fp8(const uint8_t *a, const uint8_t *b, int64_t m, int64_t n, int64_t k, double *c)
{
    if (!a || !b || !c || m < 0 || n < 0 || k < 0 || k > 65536)
        return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; i++)
        for (int64_t j = 0; j < n; j++) {
            double acc = 0.0;
            for (int64_t t = 0; t < k; t++)
                acc += e4m3_decode(a[i * k + t]) * e4m3_decode(b[j * k + t]);
            c[i * n + j] = acc;
        }
    return ORACLE_OK;
}

/* FP8 forward, the same steps as oracle_qlinear_forward with the E4M3 quantizer:
 *   q_x, s_x   = rotate + per-token E4M3 quantization (x row, block g)
 *   acc[m,n]   = sum_k dec(q_x[m,k]) * dec(qw[n,k])          (exact, fp64)
 *   base[m,n]  = fl32(fl32(acc) * fl32(s_x[m] * s_w[n]))
 *   y[m,n]     = bf16_rne(base + lora_scale * ((x A) B)[m,n])  (LoRA in fp64)
 * Every *_out pointer may be NULL. */
int oracle_qlinear_forward_fp8(const uint16_t *x, int64_t m, int64_t k,
                               const uint8_t *qw, const float *sw, int64_t n, int g,
                               const uint16_t *lora_a, const uint16_t *lora_b, int rank, double lora_scale,
                               uint16_t *y, uint8_t *qx_out, float *sx_out, double *acc_out, float *base_out)
{
    if (!x || !qw || !sw || !y || m < 0 || k <= 0 || k > 65536 || n < 0 || !is_pow2_upto256(g) || k % g != 0)
        return ORACLE_ERR_ARG;
    int use_lora = lora_a && lora_b && rank > 0;
    int alloc_fail = 0;
#pragma omp parallel
    {
        float *yr = (float *)malloc(sizeof(float) * (size_t)k);
        uint8_t *qr = (uint8_t *)malloc((size_t)k);
        double *dq = (double *)malloc(sizeof(double) * (size_t)k);
        double *t = (double *)malloc(sizeof(double) * (size_t)(rank > 0 ? rank : 1));
        if (!yr || !qr || !dq || !t) {
#pragma omp atomic write
            alloc_fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t i = 0; i < m; i++) {
                const uint16_t *xr = x + i * k;
                float sx;
                rotate_row(xr, k, g, NULL, yr);
                quantize_row_fp8(yr, k, qr, &sx);
                for (int64_t kk = 0; kk < k; kk++)
                    dq[kk] = e4m3_decode(qr[kk]);
                if (qx_out)
                    memcpy(qx_out + i * k, qr, (size_t)k);
                if (sx_out)
                    sx_out[i] = sx;
                if (use_lora) {
                    for (int j = 0; j < rank; j++)
                        t[j] = 0.0;
                    for (int64_t kk = 0; kk < k; kk++) {
                        double xv = (double)bf16_decode(xr[kk]);
                        for (int j = 0; j < rank; j++)
                            t[j] += xv * (double)bf16_decode(lora_a[kk * rank + j]);
                    }
                }
                for (int64_t j = 0; j < n; j++) {
                    const uint8_t *wr = qw + j * k;
                    double acc = 0.0;
                    for (int64_t kk = 0; kk < k; kk++)
                        acc += dq[kk] * e4m3_decode(wr[kk]);
                    float base = (float)acc * (sx * sw[j]);
                    if (acc_out)
                        acc_out[i * n + j] = acc;
                    if (base_out)
                        base_out[i * n + j] = base;
                    double out = (double)base;
                    if (use_lora) {
                        double l = 0.0;
                        for (int r = 0; r < rank; r++)
                            l += t[r] * (double)bf16_decode(lora_b[(int64_t)r * n + j]);
                        out += l * lora_scale;
                    }
                    y[i * n + j] = bf16_encode_f64(out);
                }
            }
        }
        free(yr);
        free(qr);
        free(dq);
        free(t);
    }
    return alloc_fail ? ORACLE_ERR_ARG : ORACLE_OK;
}

/* FP8 input gradient, the same steps as oracle_qlinear_backward_input with the
 * E4M3 quantizer (the SDNQ README's quantized training runs the quantized matmul
 * in the backward pass too, and lists float8_e4m3fn next to int8):
 *   dY'[m,n]    = fl32(dY * s_w[n])                      (column fold)
 *   q, s_dy     = per-token E4M3 quantization of dY' (no rotation along n)
 *   acc[m,k]    = sum_n dec(q[m,n]) * dec(qw[n,k])      (exact, fp64)
 *   z[m,k]      = fl32(fl32(acc) * s_dy[m])
 *   dxbase      = the block rotation of z along k, then * fl32(1/sqrt(g))
 *   dx[m,k]     = bf16_rne(dxbase + ((lora_scale * dY B^T) A^T)[m,k])  (LoRA in fp64)
 * The LoRA weight gradients do not involve the quantized weight; they are the
 * ones of oracle_qlinear_backward_input.  Every *_out pointer may be NULL. */
int oracle_qlinear_backward_input_fp8(const uint16_t *dy, int64_t m, int64_t n, const uint8_t *qw,
                                      const float *sw, int64_t k, int g, const uint16_t *lora_a,
                                      const uint16_t *lora_b, int rank, double lora_scale, uint16_t *dx,
                                      uint8_t *qdy_out, float *sdy_out, double *acc_out, float *dxbase_out)
{
    if (!dy || !qw || !sw || !dx || m < 0 || n <= 0 || n > 65536 || k <= 0 || !is_pow2_upto256(g) || k % g != 0)
        return ORACLE_ERR_ARG;
    int use_lora = lora_a && lora_b && rank > 0;
    int alloc_fail = 0;
#pragma omp parallel
    {
        float *yr = (float *)malloc(sizeof(float) * (size_t)n);
        uint8_t *qr = (uint8_t *)malloc((size_t)n);
        double *dq = (double *)malloc(sizeof(double) * (size_t)n);
        float *z = (float *)malloc(sizeof(float) * (size_t)k);
        double *acc = (double *)malloc(sizeof(double) * (size_t)k);
        double *gr = (double *)malloc(sizeof(double) * (size_t)(rank > 0 ? rank : 1));
        if (!yr || !qr || !dq || !z || !acc || !gr) {
#pragma omp atomic write
            alloc_fail = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t i = 0; i < m; i++) {
                float sdy;
                rotate_row(dy + i * n, n, 1, sw, yr);
                quantize_row_fp8(yr, n, qr, &sdy);
                if (qdy_out)
                    memcpy(qdy_out + i * n, qr, (size_t)n);
                if (sdy_out)
                    sdy_out[i] = sdy;
                for (int64_t j = 0; j < n; j++)
                    dq[j] = e4m3_decode(qr[j]);
                for (int64_t kk = 0; kk < k; kk++)
                    acc[kk] = 0.0;
                for (int64_t j = 0; j < n; j++) {
                    const uint8_t *wr = qw + j * k;
                    for (int64_t kk = 0; kk < k; kk++)
                        acc[kk] += dq[j] * e4m3_decode(wr[kk]);
                }
                for (int64_t kk = 0; kk < k; kk++) {
                    if (acc_out)
                        acc_out[i * k + kk] = acc[kk];
                    z[kk] = (float)acc[kk] * sdy;
                }
                if (g > 1) {
                    float c = norm_const(g);
                    for (int64_t b = 0; b < k; b += g)
                        fwht_block(z + b, g);
                    for (int64_t kk = 0; kk < k; kk++)
                        z[kk] = z[kk] * c;
                }
                if (use_lora) {
                    /* g_r[r] = lora_scale * sum_j dY[i, j] B[r, j] */
                    for (int r = 0; r < rank; r++) {
                        double s = 0.0;
                        for (int64_t j = 0; j < n; j++)
                            s += (double)bf16_decode(dy[i * n + j]) * (double)bf16_decode(lora_b[(int64_t)r * n + j]);
                        gr[r] = s * lora_scale;
                    }
                }
                for (int64_t kk = 0; kk < k; kk++) {
                    if (dxbase_out)
                        dxbase_out[i * k + kk] = z[kk];
                    double out = (double)z[kk];
                    if (use_lora) {
                        double l = 0.0;
                        for (int r = 0; r < rank; r++)
                            l += gr[r] * (double)bf16_decode(lora_a[kk * rank + r]);
                        out += l;
                    }
                    dx[i * k + kk] = bf16_encode_f64(out);
                }
            }
        }
        free(yr);
        free(qr);
        free(dq);
        free(z);
        free(acc);
        free(gr);
    }
    return alloc_fail ? ORACLE_ERR_ARG : ORACLE_OK;
}
