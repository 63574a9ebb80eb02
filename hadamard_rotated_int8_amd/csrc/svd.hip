// Low-rank (SVD) split of a weight before its rotation and int8 quantization.
//
// What it computes ("SDNQ: SD.Next Quantization Engine": SVD quantization next to
// the Hadamard rotation, SDNQConfig use_svd / svd_rank / svd_steps; the SD.Next
// dev-branch commit log: a seeded SVD truncation whose quantized weight
// dequantizes off the integer grid, i.e. integer codes plus low-rank factors).
// The pages print no algorithm; this library reads it as the randomized range
// finder with subspace iteration (Halko, Martinsson and Tropp 2011):
//   Q = orth(W omega)                  omega [k, r] Gaussian, drawn by the caller
//   svd_steps times: Z = orth(W^T Q); Q = orth(W Z)
//   svd_a = bf16(W^T Q) [k, r], svd_b = bf16(Q^T) [r, n]
//   R = fl32(W - svd_b^T svd_a^T)      binary32 residual against the rounded factors
//   (qw, w_scale) = rotate (block g) + row absmax int8 quantization of R
// so that x W^T ~ dequant(q(xH) q(RH)^T) + (x svd_a) svd_b, the forward's LoRA
// term with scale 1.
//
// Kernels (all offline weight preparation; W is read ~2 (steps + 1) times):
//  - thin products M [rows, cols] (bf16) x In [cols, r] (fp64) split along cols
//    into partial sums, then a fixed-order sum of the partials;
//  - orth(): shifted CholeskyQR, three passes (Fukaya, Kannan, Nakatsukasa,
//    Yamamoto and Yanagisawa 2020): G = Y^T Y + s I, G = R^T R, Y <- Y R^-1.  The
//    shift s = 2^-40 max diag(G) keeps the factorization defined when Y is
//    rank-deficient (an exactly low-rank W): the extra columns then become
//    arbitrary directions outside the range of W, which add nothing to the
//    projection Q Q^T W.  Only the span of Q matters: any orthonormal basis of it
//    gives the same low-rank part;
//  - the factors in bf16 (fp64 -> bf16 with one rounding, to nearest even);
//  - the binary32 residual, then its rotation + absmax and its codes in two passes
//    over R, with the same binary32 steps as the bf16 path: butterfly stages
//    h = 1 .. g/2 with (a+b, a-b), a multiply by fl32(1/sqrt(g)), s = fl32(a/127),
//    r = fl32(127/a) (rows with a < 2^-100 first scaled by 2^100),
//    code = round-half-even(fl32(y * r)) clamped to +-127.
#include <math.h>

#include "sdnq_internal.hpp"

namespace sdnq {
namespace {

constexpr int kTile = 64;        // rows and staged contraction values of a thin product; residual tile
constexpr int kGramRows = 64;    // rows per workgroup of a Gram partial
constexpr int kGramStage = 32;   // rows staged at a time
constexpr int kBlock = 256;      // values per workgroup in the residual rotation

constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;  // fl32(1/sqrt(128))

__device__ __forceinline__ float bf16_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp64 -> bf16 bits, round to nearest even with one rounding: binary32 rounded to
// odd (truncate, then set the last bit when inexact) keeps 16 bits more than bf16,
// so rounding it to nearest even gives the correctly rounded bf16 value.
__device__ __forceinline__ uint16_t bf16_from_f64(double v) {
  const float t = __double2float_rz(v);
  uint32_t b = __float_as_uint(t);
  if ((double)t != v) b |= 1u;
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// part[s, i, j] = sum over contraction indices c of split s of m[i, c] * in[c, j]
// (m [rows, cols] bf16, in [cols, R] fp64).  A workgroup covers kTile rows; thread
// t owns rows 4 (t / 16) + a (a < 4) and columns t % 16 + 16 v (v < R / 16).  The
// bf16 tile is staged with 16-byte loads (cols is a multiple of 16, so a group of
// 8 values is wholly inside or outside the chunk).
template <int R>
__global__ __launch_bounds__(256) void thin_partial_kernel(const uint16_t *__restrict__ m, int64_t rows,
                                                           int64_t cols, const double *__restrict__ in,
                                                           int64_t chunk, double *__restrict__ part) {
  constexpr int CV = R / 16;
  __shared__ double ms[kTile][kTile + 1];
  __shared__ double is[kTile][R];
  const int tid = threadIdx.x;
  const int rg = 4 * (tid >> 4), cg = tid & 15;
  const int64_t row0 = (int64_t)blockIdx.x * kTile;
  const int64_t c_begin = (int64_t)blockIdx.y * chunk;
  const int64_t c_end = c_begin + chunk < cols ? c_begin + chunk : cols;
  double acc[4][CV];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int v = 0; v < CV; ++v) acc[a][v] = 0.0;
  for (int64_t c0 = c_begin; c0 < c_end; c0 += kTile) {
    __syncthreads();
#pragma unroll
    for (int e = tid; e < kTile * kTile / 8; e += 256) {
      const int rr = e / (kTile / 8), cc = 8 * (e % (kTile / 8));
      const int64_t gr = row0 + rr, gc = c0 + cc;
      v4u raw = {0u, 0u, 0u, 0u};
      if (gr < rows && gc < c_end) raw = *reinterpret_cast<const v4u *>(m + gr * cols + gc);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        ms[rr][cc + 2 * w] = (double)bf16_lo(raw[w]);
        ms[rr][cc + 2 * w + 1] = (double)bf16_hi(raw[w]);
      }
    }
    for (int e = tid; e < kTile * R; e += 256) {
      const int cc = e / R, j = e % R;
      const int64_t gc = c0 + cc;
      is[cc][j] = gc < c_end ? in[gc * R + j] : 0.0;
    }
    __syncthreads();
#pragma unroll 2
    for (int kk = 0; kk < kTile; ++kk) {
      double mv[4], iv[CV];
#pragma unroll
      for (int a = 0; a < 4; ++a) mv[a] = ms[rg + a][kk];
#pragma unroll
      for (int v = 0; v < CV; ++v) iv[v] = is[kk][cg + 16 * v];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int v = 0; v < CV; ++v) acc[a][v] = fma(mv[a], iv[v], acc[a][v]);
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t gr = row0 + rg + a;
    if (gr >= rows) continue;
    double *dst = part + ((int64_t)blockIdx.y * rows + gr) * R;
#pragma unroll
    for (int v = 0; v < CV; ++v) dst[cg + 16 * v] = acc[a][v];
  }
}

// out[i] = sum_s part[s, i] in the order s = 0, 1, ...
__global__ __launch_bounds__(256) void sum_partials_kernel(const double *__restrict__ part, int splits,
                                                           int64_t count, double *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  double s = 0.0;
  for (int p = 0; p < splits; ++p) s += part[(int64_t)p * count + i];
  out[i] = s;
}

// gpart[b, a, c] = sum over rows i of block b of y[i, a] * y[i, c]
template <int R>
__global__ __launch_bounds__(256) void gram_partial_kernel(const double *__restrict__ y, int64_t rows,
                                                           double *__restrict__ gpart) {
  constexpr int OPT = R * R / 256;  // outputs per thread (R >= 16)
  __shared__ double ys[kGramStage][R];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kGramRows;
  double acc[OPT];
#pragma unroll
  for (int u = 0; u < OPT; ++u) acc[u] = 0.0;
  for (int s0 = 0; s0 < kGramRows; s0 += kGramStage) {
    __syncthreads();
    for (int e = tid; e < kGramStage * R; e += 256) {
      const int rr = e / R, j = e % R;
      const int64_t gr = r0 + s0 + rr;
      ys[rr][j] = gr < rows ? y[gr * R + j] : 0.0;
    }
    __syncthreads();
    for (int rr = 0; rr < kGramStage; ++rr) {
#pragma unroll
      for (int u = 0; u < OPT; ++u) {
        const int o = tid + 256 * u;
        acc[u] = fma(ys[rr][o / R], ys[rr][o % R], acc[u]);
      }
    }
  }
  double *dst = gpart + (int64_t)blockIdx.x * R * R;
#pragma unroll
  for (int u = 0; u < OPT; ++u) dst[tid + 256 * u] = acc[u];
}

// One workgroup: G = sum of the partial Grams + s I, its Cholesky factor G = U^T U
// (U upper triangular), and rinv = U^-1.  Both factorizations are right-looking:
// step j finishes row j (column j) and updates the trailing block in parallel, so
// each thread does O(1) dependent work per step.
template <int R>
__global__ __launch_bounds__(256) void chol_inverse_kernel(const double *__restrict__ gpart, int parts,
                                                           double *__restrict__ rinv) {
  __shared__ double a[R][R + 1];   // G, overwritten by the trailing updates; then U in its upper part
  __shared__ double x[R][R + 1];   // U^-1
  __shared__ double shift;
  const int tid = threadIdx.x;
  constexpr int PER = (R * R + 255) / 256;
  double sum[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) sum[u] = 0.0;
#pragma unroll 4
  for (int p = 0; p < parts; ++p) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 256 * u;
      if (e < R * R) sum[u] += gpart[(int64_t)p * R * R + e];
    }
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + 256 * u;
    if (e < R * R) {
      a[e / R][e % R] = sum[u];
      x[e / R][e % R] = (e / R == e % R) ? 1.0 : 0.0;
    }
  }
  __syncthreads();
  if (tid == 0) {
    double dmax = 0.0;
    for (int j = 0; j < R; ++j) dmax = fmax(dmax, a[j][j]);
    shift = fmax(0x1p-40 * dmax, 0x1p-900);
  }
  __syncthreads();
  if (tid < R) a[tid][tid] += shift;
  __syncthreads();
  // Cholesky: after step j, row j of a (from the diagonal on) is row j of U
  for (int j = 0; j < R; ++j) {
    const double d = a[j][j];
    const double ujj = sqrt(d > shift ? d : shift);
    __syncthreads();
    if (tid >= j && tid < R) a[j][tid] = (tid == j) ? ujj : a[j][tid] / ujj;
    __syncthreads();
    // trailing block, rows and columns > j: a[r][c] -= U[j][r] U[j][c]
    for (int e = tid; e < (R - j - 1) * (R - j - 1); e += 256) {
      const int r = j + 1 + e / (R - j - 1), c = j + 1 + e % (R - j - 1);
      a[r][c] -= a[j][r] * a[j][c];
    }
    __syncthreads();
  }
  // U^-1 by rows from the bottom: x[i] = (e_i - sum_{k > i} U[i][k] x[k]) / U[i][i];
  // step i scales row i, then removes it from the rows above
  for (int i = R - 1; i >= 0; --i) {
    if (tid < R) x[i][tid] = x[i][tid] / a[i][i];
    __syncthreads();
    for (int e = tid; e < i * R; e += 256) {
      const int r = e / R, c = e % R;
      x[r][c] -= a[r][i] * x[i][c];
    }
    __syncthreads();
  }
  for (int e = tid; e < R * R; e += 256) rinv[e] = x[e / R][e % R];
}

// q[i, c] = sum_{k <= c} y[i, k] * rinv[k, c]
template <int R>
__global__ __launch_bounds__(256) void apply_rinv_kernel(const double *__restrict__ y, int64_t rows,
                                                         const double *__restrict__ rinv, double *__restrict__ q) {
  __shared__ double ri[R][R];
  const int tid = threadIdx.x;
  for (int e = tid; e < R * R; e += 256) ri[e / R][e % R] = rinv[e];
  __syncthreads();
  const int64_t idx = (int64_t)blockIdx.x * 256 + tid;
  if (idx >= rows * R) return;
  const int64_t i = idx / R;
  const int c = (int)(idx % R);
  const double *yr = y + i * R;
  double s = 0.0;
  for (int k = 0; k <= c; ++k) s = fma(yr[k], ri[k][c], s);
  q[idx] = s;
}

__global__ __launch_bounds__(256) void f32_to_f64_kernel(const float *__restrict__ in, int64_t count,
                                                         double *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) out[i] = (double)in[i];
}

// svd_a[k, r] = bf16(a[k, r]); svd_b[c, i] = bf16(q[i, c])
__global__ __launch_bounds__(256) void factors_kernel(const double *__restrict__ a, int64_t k,
                                                      const double *__restrict__ q, int64_t n, int r,
                                                      uint16_t *__restrict__ svd_a, uint16_t *__restrict__ svd_b) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < k * r) svd_a[idx] = bf16_from_f64(a[idx]);
  if (idx < n * r) {
    const int64_t c = idx / n, i = idx % n;
    svd_b[idx] = bf16_from_f64(q[i * r + c]);
  }
}

// res[i, j] = fl32(w[i, j] - sum_c svd_b[c, i] * svd_a[j, c]), the sum in fp64.
// A workgroup covers 64 x 64 outputs, each thread 4 x 4.
template <int R>
__global__ __launch_bounds__(256) void residual_kernel(const uint16_t *__restrict__ w, int64_t n, int64_t k,
                                                       const uint16_t *__restrict__ svd_a,
                                                       const uint16_t *__restrict__ svd_b, float *__restrict__ res) {
  __shared__ double bs[R][kTile + 1];  // bs[c][ii] = svd_b[c, i0 + ii]
  __shared__ double as[kTile][R + 1];  // as[jj][c] = svd_a[j0 + jj, c]
  const int tid = threadIdx.x;
  const int64_t i0 = (int64_t)blockIdx.y * kTile, j0 = (int64_t)blockIdx.x * kTile;
  for (int e = tid; e < R * kTile; e += 256) {
    const int c = e / kTile, ii = e % kTile;
    bs[c][ii] = i0 + ii < n ? (double)bf16_f32(svd_b[(int64_t)c * n + i0 + ii]) : 0.0;
  }
  for (int e = tid; e < kTile * R; e += 256) {
    const int jj = e / R, c = e % R;
    as[jj][c] = j0 + jj < k ? (double)bf16_f32(svd_a[(j0 + jj) * R + c]) : 0.0;
  }
  __syncthreads();
  const int ti = 4 * (tid / 16), tj = 4 * (tid % 16);
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
#pragma unroll 2
  for (int c = 0; c < R; ++c) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = fma(bs[c][ti + a], as[tj + b][c], acc[a][b]);
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t i = i0 + ti + a;
    if (i >= n) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t j = j0 + tj + b;
      if (j < k) res[i * k + j] = (float)((double)bf16_f32(w[i * k + j]) - acc[a][b]);
    }
  }
}

template <int G>
__device__ __forceinline__ float norm_const() {
  if constexpr (G == 64) return 0.125f;
  else if constexpr (G == 128) return kInvSqrt128;
  else if constexpr (G == 256) return 0.0625f;
  else return 1.0f;
}

// Rotated value of element col0 + tid of row `row` of res (block g along the row):
// butterfly through LDS, one binary32 add or subtract per stage, then the
// normalization multiply.  Every thread of the workgroup reaches every barrier.
template <int G>
__device__ __forceinline__ float rotated_value(const float *__restrict__ res, int64_t k, int64_t row, int64_t col0,
                                               float (&buf)[kBlock], bool in_row) {
  const int tid = threadIdx.x;
  float v = in_row ? res[row * k + col0 + tid] : 0.0f;
  if constexpr (G > 1) {
#pragma unroll
    for (int h = 1; h < G; h <<= 1) {
      buf[tid] = v;
      __syncthreads();
      const float p = buf[tid ^ h];
      v = (tid & h) ? p - v : v + p;
      __syncthreads();
    }
    v = v * norm_const<G>();
  }
  return v;
}

// Pass 1: rowmax[row] = max |y| over the row (as binary32 bits: non-negative floats
// order like their bit patterns).
template <int G>
__global__ __launch_bounds__(kBlock) void residual_absmax_kernel(const float *__restrict__ res, int64_t n, int64_t k,
                                                                 uint32_t *__restrict__ rowmax) {
  __shared__ float buf[kBlock];
  __shared__ float wmax[kBlock / 64];
  const int64_t chunks = (k + kBlock - 1) / kBlock;
  const int64_t row = blockIdx.x / chunks, col0 = (blockIdx.x % chunks) * kBlock;
  const bool in_row = col0 + threadIdx.x < k;
  const float y = rotated_value<G>(res, k, row, col0, buf, in_row);
  float a = in_row ? fabsf(y) : 0.0f;
  for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = wmax[0];
    for (int i = 1; i < kBlock / 64; ++i) m = fmaxf(m, wmax[i]);
    atomicMax(rowmax + row, __float_as_uint(m));
  }
}

// Pass 2: codes and scales.
template <int G>
__global__ __launch_bounds__(kBlock) void residual_quantize_kernel(const float *__restrict__ res, int64_t n, int64_t k,
                                                                   const uint32_t *__restrict__ rowmax,
                                                                   int8_t *__restrict__ q, float *__restrict__ scale) {
  __shared__ float buf[kBlock];
  const int64_t chunks = (k + kBlock - 1) / kBlock;
  const int64_t row = blockIdx.x / chunks, col0 = (blockIdx.x % chunks) * kBlock;
  const bool in_row = col0 + threadIdx.x < k;
  const float y = rotated_value<G>(res, k, row, col0, buf, in_row);
  const float a = __uint_as_float(rowmax[row]);
  const float up = a < 0x1p-100f ? 0x1p100f : 1.0f;
  const float as = a * up;
  const float r = as > 0.0f ? 127.0f / as : 0.0f;
  if (col0 == 0 && threadIdx.x == 0) scale[row] = a / 127.0f;
  if (in_row) {
    float t = rintf((y * up) * r);
    t = fminf(fmaxf(t, -127.0f), 127.0f);
    q[row * k + col0 + threadIdx.x] = (int8_t)(int)t;
  }
}

struct SvdLayout {
  size_t res, q, wt, y, t, part, gpart, rinv, rowmax, total;
  int64_t part_max, gparts_max;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Split of the contraction of a thin product: about 1024 workgroups, chunks of a
// multiple of 64 values.
int64_t thin_chunk(int64_t rows, int64_t cols) {
  const int64_t tiles = (rows + kTile - 1) / kTile;
  int64_t chunk = (cols * tiles + 1023) / 1024;
  chunk = (chunk + kTile - 1) / kTile * kTile;
  return chunk < kTile ? kTile : chunk;
}

SvdLayout svd_layout(int64_t n, int64_t k, int r) {
  SvdLayout L{};
  const int64_t big = n > k ? n : k;
  const int64_t s1 = (k + thin_chunk(n, k) - 1) / thin_chunk(n, k);  // W Z: rows n, contraction k
  const int64_t s2 = (n + thin_chunk(k, n) - 1) / thin_chunk(k, n);  // W^T Q: rows k, contraction n
  L.part_max = (s1 * n > s2 * k ? s1 * n : s2 * k) * r;
  L.gparts_max = (big + kGramRows - 1) / kGramRows;
  size_t off = 0;
  L.res = off; off += align256((size_t)n * k * 4);
  L.q = off; off += align256((size_t)n * r * 8);
  L.wt = off; off += align256((size_t)n * k * 2);
  L.y = off; off += align256((size_t)big * r * 8);
  L.t = off; off += align256((size_t)big * r * 8);
  L.part = off; off += align256((size_t)L.part_max * 8);
  L.gpart = off; off += align256((size_t)L.gparts_max * r * r * 8);
  L.rinv = off; off += align256((size_t)r * r * 8);
  L.rowmax = off; off += align256((size_t)n * 4);
  L.total = off;
  return L;
}

template <int R>
hipError_t thin_product(const uint16_t *m, int64_t rows, int64_t cols, const double *in, double *part, double *out,
                        hipStream_t s) {
  const int64_t chunk = thin_chunk(rows, cols);
  const int64_t splits = (cols + chunk - 1) / chunk;
  hipLaunchKernelGGL(thin_partial_kernel<R>, dim3((unsigned)((rows + kTile - 1) / kTile), (unsigned)splits),
                     dim3(256), 0, s, m, rows, cols, in, chunk, part);
  const int64_t count = rows * R;
  hipLaunchKernelGGL(sum_partials_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, part,
                     (int)splits, count, out);
  return hipGetLastError();
}

// y [rows, R] -> q [rows, R] with orthonormal columns spanning the same space
// (three shifted CholeskyQR passes; y and q may not alias, y is overwritten).
template <int R>
hipError_t orth(double *y, int64_t rows, double *q, double *gpart, double *rinv, hipStream_t s) {
  const unsigned parts = (unsigned)((rows + kGramRows - 1) / kGramRows);
  const unsigned apply_blocks = (unsigned)((rows * R + 255) / 256);
  double *src = y, *dst = q;
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(gram_partial_kernel<R>, dim3(parts), dim3(256), 0, s, src, rows, gpart);
    hipLaunchKernelGGL(chol_inverse_kernel<R>, dim3(1), dim3(256), 0, s, gpart, (int)parts, rinv);
    hipLaunchKernelGGL(apply_rinv_kernel<R>, dim3(apply_blocks), dim3(256), 0, s, src, rows, rinv, dst);
    double *t = src; src = dst; dst = t;
  }
  // three passes: the result is in src, which is y after passes 1 and 3 swap back
  if (src != q)
    hipLaunchKernelGGL(sum_partials_kernel, dim3(apply_blocks), dim3(256), 0, s, src, 1, rows * R, q);
  return hipGetLastError();
}

template <int G>
hipError_t quantize_residual(const float *res, int64_t n, int64_t k, uint32_t *rowmax, int8_t *qw, float *scale,
                             hipStream_t s) {
  const int64_t blocks = n * ((k + kBlock - 1) / kBlock);
  hipLaunchKernelGGL(residual_absmax_kernel<G>, dim3((unsigned)blocks), dim3(kBlock), 0, s, res, n, k, rowmax);
  hipLaunchKernelGGL(residual_quantize_kernel<G>, dim3((unsigned)blocks), dim3(kBlock), 0, s, res, n, k, rowmax, qw,
                     scale);
  return hipGetLastError();
}

template <int R>
hipError_t svd_split(const uint16_t *w, int64_t n, int64_t k, int g, int steps, const float *omega, int8_t *qw,
                     float *w_scale, uint16_t *svd_a, uint16_t *svd_b, void *ws, hipStream_t s) {
  const SvdLayout L = svd_layout(n, k, R);
  char *base = static_cast<char *>(ws);
  float *res = reinterpret_cast<float *>(base + L.res);
  double *q = reinterpret_cast<double *>(base + L.q);
  uint16_t *wt = reinterpret_cast<uint16_t *>(base + L.wt);
  double *y = reinterpret_cast<double *>(base + L.y);
  double *t = reinterpret_cast<double *>(base + L.t);
  double *part = reinterpret_cast<double *>(base + L.part);
  double *gpart = reinterpret_cast<double *>(base + L.gpart);
  double *rinv = reinterpret_cast<double *>(base + L.rinv);
  uint32_t *rowmax = reinterpret_cast<uint32_t *>(base + L.rowmax);
  hipError_t e;
#define SDNQ_SVD_TRY(expr)            \
  if ((e = (expr)) != hipSuccess) return e
  SDNQ_SVD_TRY(launch_transpose_u16(w, n, k, wt, s));  // W^T [k, n]
  hipLaunchKernelGGL(f32_to_f64_kernel, dim3((unsigned)((k * R + 255) / 256)), dim3(256), 0, s, omega, k * R, t);
  SDNQ_SVD_TRY(thin_product<R>(w, n, k, t, part, y, s));  // W omega [n, R]
  SDNQ_SVD_TRY(orth<R>(y, n, q, gpart, rinv, s));
  for (int it = 0; it < steps; ++it) {
    SDNQ_SVD_TRY(thin_product<R>(wt, k, n, q, part, y, s));  // W^T Q [k, R]
    SDNQ_SVD_TRY(orth<R>(y, k, t, gpart, rinv, s));          // Z
    SDNQ_SVD_TRY(thin_product<R>(w, n, k, t, part, y, s));   // W Z [n, R]
    SDNQ_SVD_TRY(orth<R>(y, n, q, gpart, rinv, s));          // Q
  }
  SDNQ_SVD_TRY(thin_product<R>(wt, k, n, q, part, y, s));  // W^T Q [k, R]
  const int64_t fcount = (k > n ? k : n) * R;
  hipLaunchKernelGGL(factors_kernel, dim3((unsigned)((fcount + 255) / 256)), dim3(256), 0, s, y, k, q, n, R, svd_a,
                     svd_b);
  hipLaunchKernelGGL(residual_kernel<R>, dim3((unsigned)((k + kTile - 1) / kTile), (unsigned)((n + kTile - 1) / kTile)),
                     dim3(256), 0, s, w, n, k, svd_a, svd_b, res);
  SDNQ_SVD_TRY(launch_fill_zero_u16(reinterpret_cast<uint16_t *>(rowmax), 2 * n, s));
  switch (g) {
    case 1: return quantize_residual<1>(res, n, k, rowmax, qw, w_scale, s);
    case 64: return quantize_residual<64>(res, n, k, rowmax, qw, w_scale, s);
    case 128: return quantize_residual<128>(res, n, k, rowmax, qw, w_scale, s);
    case 256: return quantize_residual<256>(res, n, k, rowmax, qw, w_scale, s);
    default: return hipErrorInvalidValue;
  }
#undef SDNQ_SVD_TRY
}

}  // namespace

size_t svd_workspace_bytes(int64_t n, int64_t k, int rank) { return svd_layout(n, k, rank).total; }

size_t svd_workspace_q_offset(int64_t n, int64_t k, int rank) { return svd_layout(n, k, rank).q; }

hipError_t launch_svd_quantize_weight(const uint16_t *w, int64_t n, int64_t k, int g, int rank, int steps,
                                      const float *omega, int8_t *qw, float *w_scale, uint16_t *svd_a,
                                      uint16_t *svd_b, void *workspace, hipStream_t stream) {
  switch (rank) {
    case 16: return svd_split<16>(w, n, k, g, steps, omega, qw, w_scale, svd_a, svd_b, workspace, stream);
    case 32: return svd_split<32>(w, n, k, g, steps, omega, qw, w_scale, svd_a, svd_b, workspace, stream);
    case 64: return svd_split<64>(w, n, k, g, steps, omega, qw, w_scale, svd_a, svd_b, workspace, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdnq
