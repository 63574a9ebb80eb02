// G1: block Walsh-Hadamard rotation fused with per-row absmax int8 quantization.
//
// What it computes (one row of a bf16 [rows, cols] matrix at a time):
//   y = fl32(1/sqrt(g)) * H_g v on every contiguous block of g values of the row
//       ("ConvRot / Hadamard SDNQ", "What The Options Do": rotation block =
//       hadamard_group_size along in-features), with v = x (or x * col_scale);
//   a = max |y| over the whole row; s = fl32(a / 127); r = fl32(127 / a);
//   q = round_half_even(fl32(y * r)) in [-127, 127]  (a row with a < 2^-100 is
//       first scaled by 2^100, exactly, so that 127 / a stays finite)
//       (HSWQ README, "Rigorous grid / pack simulation": rotate, then absmax on
//       a symmetric INT8 grid).
// The butterfly runs the stages h = 1, 2, ..., g/2 in that order, every pair
// (i, i+h) becoming (a+b, a-b) in binary32, so the codes and scales are
// bit-identical to a scalar evaluation of the same steps.
//
// Layout.  A row is cut into superblocks of 256 values; a quad of 4 adjacent lanes
// owns one superblock.  Lane l4 of the quad holds the 64 values
//     e = 32*i + 8*l4 + j      (i = 0..7, j = 0..7)
// loaded as eight 16-byte loads (each quad reads 64 contiguous bytes per load).
// So value-index bits 0-2 (j) and 5-7 (i) live in registers and bits 3-4 in the
// lane-within-quad: stages h = 1, 2, 4, 32, 64, 128 are register butterflies and
// h = 8, 16 are quad_perm DPP exchanges.  Rows that would leave lanes idle this
// way (10240 values: 160 lanes in three wavefronts) use 8 lanes per superblock
// instead, 32 values each (e = 64*i + 8*l + j, i = 0..3): value bits 3-5 cross
// lanes 1, 2 and 8 apart (quad_perm and row_ror:8) and bits 6-7 stay in registers.  The whole row stays in registers until
// its absmax is known (one workgroup holds `rows_per_wg` complete rows at a
// time; a persistent grid walks over row groups, prefetching the next one).
//
// FP8 variant (the float8_e4m3fn quantized matmul listed next to INT8 in "SDNQ:
// SD.Next Quantization Engine"): s = fl32(a / 448), r = fl32(448 / a), and each
// fl32(y * r), clamped to +-448, is converted by v_cvt_pk_fp8_f32 (OCP E4M3,
// round half to even; it would give NaN from 464 up, which the clamp rules out);
// an exact zero is stored as +0, a nonzero value that rounds to zero keeps its sign.
//
// Cross-lane stages keep a per-lane sign: the upper lane of a pair computes
// fma(partner, -1, self) = self - partner = -(a - b), which rounds exactly like
// a - b up to the sign; the sign of every lane is (-1)^popcount(l4) after both
// stages and is folded into the normalization multiply.
#include <atomic>

#include "sdnq_internal.hpp"

namespace sdnq {
namespace {

constexpr int kMaxRowsPerWg = 32;
constexpr int kMaxThreads = 1024;
constexpr int64_t kMaxCols = 256 * (kMaxThreads / 4);  // values a workgroup can hold: 65536
// 1.5 * 2^23: adding it to |t| < 2^22 rounds t to an integer (ties to even) and
// leaves that integer, two's complement, in the low mantissa bits.
constexpr float kRoundMagic = 12582912.0f;

// fl32(1/sqrt(128)) = 2^-3.5 rounded to nearest binary32.
constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;
static_assert(__builtin_bit_cast(uint32_t, kInvSqrt128) == 0x3DB504F3u, "1/sqrt(128) constant");

template <int G>
__device__ __forceinline__ float norm_const() {
  if constexpr (G == 64) return 0.125f;
  else if constexpr (G == 128) return kInvSqrt128;
  else if constexpr (G == 256) return 0.0625f;
  else return 1.0f;
}

// Byte 0 of the magic-rounded value = the int8 code.
__device__ __forceinline__ uint32_t code_bits(float t) { return __float_as_uint(t + kRoundMagic); }

__device__ __forceinline__ uint32_t pack4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
  // v_perm_b32: selector byte values 0-3 pick the second operand's bytes, 4-7 the first's.
  uint32_t lo = __builtin_amdgcn_perm(c1, c0, 0x0c0c0400u);  // [c0.b0, c1.b0, 0, 0]
  uint32_t hi = __builtin_amdgcn_perm(c3, c2, 0x0c0c0400u);  // [c2.b0, c3.b0, 0, 0]
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);         // [lo.b0, lo.b1, hi.b0, hi.b1]
}

// One cross-lane butterfly stage on 8 registers: v = fma(v[partner lane], m, v)
// as a single v_fmac_f32 with a quad_perm DPP source.  The product by m = +-1 is
// exact and the fma rounds once, so each result equals fl(a + b) or -fl(a - b).
// The leading s_nop gives the two wait states a DPP read needs after a VALU write
// of its source; inside the block no instruction reads a register written by the
// two before it.
#define SDNQ_FMAC_DPP8(PERM)                                                                    \
  "s_nop 1\n\t"                                                                                \
  "v_fmac_f32_dpp %0, %0, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %1, %1, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %2, %2, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %3, %3, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %4, %4, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %5, %5, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %6, %6, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf\n\t"                \
  "v_fmac_f32_dpp %7, %7, %8 quad_perm:" PERM " row_mask:0xf bank_mask:0xf"

__device__ __forceinline__ void dpp_stage_xor1(float (&r)[8], float m) {
  asm volatile(SDNQ_FMAC_DPP8("[1,0,3,2]")
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7])
               : "v"(m));
}
__device__ __forceinline__ void dpp_stage_xor2(float (&r)[8], float m) {
  asm volatile(SDNQ_FMAC_DPP8("[2,3,0,1]")
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7])
               : "v"(m));
}
// Lane xor 8 (within each row of 16 lanes): the row rotation by 8.
#define SDNQ_FMAC_DPP8_ROR8                                                                     \
  "s_nop 1\n\t"                                                                                \
  "v_fmac_f32_dpp %0, %0, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"                         \
  "v_fmac_f32_dpp %1, %1, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"                         \
  "v_fmac_f32_dpp %2, %2, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"                         \
  "v_fmac_f32_dpp %3, %3, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"                         \
  "v_fmac_f32_dpp %4, %4, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"                         \
  "v_fmac_f32_dpp %5, %5, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"                         \
  "v_fmac_f32_dpp %6, %6, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"                         \
  "v_fmac_f32_dpp %7, %7, %8 row_ror:8 row_mask:0xf bank_mask:0xf"
__device__ __forceinline__ void dpp_stage_xor8(float (&r)[8], float m) {
  asm volatile(SDNQ_FMAC_DPP8_ROR8
               : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7])
               : "v"(m));
}

// Column scales up to this many columns are staged once per workgroup in LDS
// (dynamic shared memory), instead of re-read from L2 for every row.
constexpr int64_t kColScaleLds = 16384;

// Rows longer than one workgroup can hold (more than 65536 values) are cut into
// `chunks` equal segments of `cols` values (whole rotation blocks each) and run
// as the rows of a [rows * chunks, cols] view of the same memory, in phases:
//   phase 1: each segment's max |y| is merged into scale[row] (binary32 bits,
//            atomic max; scale zeroed first), nothing else is written;
//   phase 2: the codes, from the row's max read back from scale[row];
// then finish_scale_kernel turns the maxima into scales.  SEG = false is the
// whole-row path (chunks = 1, phase 0).
// WHOLE: cols is a multiple of 256, so all 8 loads and stores of every lane lie
// inside its row; they share one vector offset and add 64*i (32*i) bytes as the
// scalar offset, instead of holding 16 per-load offsets in VGPRs.
// NT: the codes are stored non-temporally (see kStreamCodesMax).
// LPS: lanes per 256-value superblock.  4: a quad of adjacent lanes, 64 values
// each (e = 32*i + 8*l + j, i < 8).  8: lanes 0-3 and 8-11 of a 16-lane row own
// one superblock and lanes 4-7 and 12-15 the next, 32 values each
// (e = 64*i + 8*l + j, i < 4, l = lane bits 0, 1 and 3), so that value bits 3-5
// cross lanes by xor 1, 2 (quad_perm) and 8 (row_ror:8); rows then take whole
// wavefronts where 4 lanes per superblock would leave some idle.
template <int G, bool COLSCALE, int MAXT, bool FP8, bool SEG = false, bool WHOLE = false, bool NT = false,
          int LPS = 4>
__global__ __launch_bounds__(MAXT) void rotq_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, const float *__restrict__ col_scale,
    int8_t *__restrict__ q, float *__restrict__ scale, int t_row, int rows_per_wg, int64_t groups, int chunks,
    int phase) {
  // Workgroup b handles row groups b, b + gridDim.x, ...: one each in the usual
  // launch of one workgroup per group, several in a persistent grid (column scales
  // staged in LDS), where it loads the next group's values while it transforms
  // the current one (a load past the last group reads nothing).  Row maxima go
  // through three rotating LDS slots: slot (it+1)%3 is cleared at the start of
  // iteration it, before that iteration's barrier, so one barrier per group
  // separates every clear from the atomics that follow it and from the reads
  // that precede it.
  __shared__ uint32_t row_max[3][kMaxRowsPerWg];

  const int tid = threadIdx.x;
  // one row per workgroup (the MLP widths) needs no division by t_row
  const int r_local = rows_per_wg == 1 ? 0 : tid / t_row;
  const int qt = tid - r_local * t_row;
  static_assert(LPS == 4 || LPS == 8, "4 or 8 lanes per superblock");
  constexpr int NI = 32 / LPS;   // 16-byte loads per lane and row group
  constexpr int SPAN = 8 * LPS;  // values between a lane's consecutive loads
  const int sb = LPS == 4 ? qt >> 2 : ((qt >> 4) << 1) | ((qt >> 2) & 1);  // superblock of this lane
  const int l4 = LPS == 4 ? qt & 3 : (qt & 3) | ((qt >> 1) & 4);          // lane within the superblock
  const int64_t base = sb * 256 + 8 * l4;
  if (tid < rows_per_wg) {
    row_max[0][tid] = 0u;
    row_max[1][tid] = 0u;
  }
  extern __shared__ __attribute__((aligned(16))) float cs_lds[];  // [cols] when staged
  const bool cs_staged = COLSCALE && !SEG && cols <= kColScaleLds;
  if (cs_staged) {
    for (int64_t c = 4 * tid; c < cols; c += 4 * blockDim.x)
      *reinterpret_cast<float4 *>(cs_lds + c) = *reinterpret_cast<const float4 *>(col_scale + c);
  }
  __syncthreads();

  // ---- load: NI x 16 bytes, e0(i) = sb*256 + SPAN*i + 8*l4.  Buffer loads over the
  // group's rows: lanes past the last row or column read zeros, without a branch.
  auto group_rows = [&](int64_t grp) -> int64_t {
    const int64_t first = grp * rows_per_wg;
    const int64_t left = rows - first;
    return grp < groups ? (left < rows_per_wg ? left : rows_per_wg) : 0;
  };
  auto load = [&](int64_t grp, v4u (&raw)[NI]) {
    const int64_t nrows = group_rows(grp);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(x + (grp < groups ? grp : 0) * rows_per_wg * cols), 0, (int)(nrows * cols * 2), 0x00020000);
    const unsigned off0 = (unsigned)((r_local * cols + base) * 2);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int64_t e0 = base + SPAN * i;
      const unsigned off = WHOLE ? off0 : (e0 < cols) ? (unsigned)((r_local * cols + e0) * 2) : 0x80000000u;
      raw[i] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, off, WHOLE ? 2 * SPAN * i : 0, 0));
    }
  };

  v4u raw[NI];
  int64_t grp = blockIdx.x;
  load(grp, raw);
  for (int it = 0; grp < groups; ++it, grp += gridDim.x) {
    const int64_t row = grp * rows_per_wg + r_local;
    const bool row_ok = row < rows;
    int64_t full_row = row, col_off = 0;  // row of the matrix, first column of this segment
    if constexpr (SEG) {
      full_row = row / chunks;
      col_off = (row - full_row * chunks) * cols;
    }
    if (tid < rows_per_wg) row_max[(it + 1) % 3][tid] = 0u;

    float v[NI][8];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v[i][2 * w] = bf16_lo(raw[i][w]);
        v[i][2 * w + 1] = bf16_hi(raw[i][w]);
      }
    }
    // The raw registers are free again: fetch the next group into them, so its
    // loads stay in flight through the whole transform of this group.
    __builtin_amdgcn_sched_barrier(0);
    load(grp + gridDim.x, raw);
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (COLSCALE) {
      // Two loops, one per memory: a pointer that could be either would make
      // these flat loads, which wait for every outstanding global access too
      // (the next group's prefetch and this workgroup's code stores).
      auto fold = [&](int i, const float4 c0, const float4 c1) {
        v[i][0] = v[i][0] * c0.x; v[i][1] = v[i][1] * c0.y;
        v[i][2] = v[i][2] * c0.z; v[i][3] = v[i][3] * c0.w;
        v[i][4] = v[i][4] * c1.x; v[i][5] = v[i][5] * c1.y;
        v[i][6] = v[i][6] * c1.z; v[i][7] = v[i][7] * c1.w;
      };
      if (cs_staged) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int64_t e0 = base + SPAN * i;
          if (e0 < cols)
            fold(i, *reinterpret_cast<const float4 *>(cs_lds + e0), *reinterpret_cast<const float4 *>(cs_lds + e0 + 4));
        }
      } else {
        const float *cg = col_scale + col_off;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int64_t e0 = base + SPAN * i;
          if (e0 < cols)
            fold(i, *reinterpret_cast<const float4 *>(cg + e0), *reinterpret_cast<const float4 *>(cg + e0 + 4));
        }
      }
    }

    float sign = 1.0f;  // per-lane sign of the stored values after the DPP stages
    if constexpr (G > 1) {
      // h = 1, 2, 4: value bits 0-2 (register index j)
#pragma unroll
      for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if ((j & h) == 0) {
              const float a = v[i][j], b = v[i][j + h];
              v[i][j] = a + b;
              v[i][j + h] = a - b;
            }
          }
        }
      }
      // h = 8: lane xor 1; h = 16: lane xor 2; with 8 lanes per superblock also
      // h = 32: lane xor 8
      {
        const float m1 = (l4 & 1) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < NI; ++i) dpp_stage_xor1(v[i], m1);
        const float m2 = (l4 & 2) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < NI; ++i) dpp_stage_xor2(v[i], m2);
        sign = m1 * m2;
        if constexpr (LPS == 8) {
          const float m3 = (l4 & 4) ? -1.0f : 1.0f;
#pragma unroll
          for (int i = 0; i < NI; ++i) dpp_stage_xor8(v[i], m3);
          sign = sign * m3;
        }
      }
      // h = SPAN, 2*SPAN, ...: the value bits of the register index i, up to g/2
#pragma unroll
      for (int hi = 1; hi < NI; hi <<= 1) {
        if (SPAN * hi < G) {
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            if ((i & hi) == 0) {
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const float a = v[i][j], b = v[i + hi][j];
                v[i][j] = a + b;
                v[i + hi][j] = a - b;
              }
            }
          }
        }
      }
    }

    // g = 128: the normalization constant is inexact, so apply it to every value now.
    if constexpr (G == 128) {
      const float sc = sign * norm_const<G>();
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[i][j] = v[i][j] * sc;
    }

    float loc = 0.0f;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) loc = fmaxf(loc, fabsf(v[i][j]));

    uint32_t *slot = row_max[it % 3];
    if (row_ok) atomicMax(&slot[r_local], __float_as_uint(loc));
    // LDS-only barrier: the prefetch of the next group stays in flight.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float a = __uint_as_float(slot[r_local]);
    if constexpr (SEG) {
      if (phase == 1) {  // segment maximum into the row's maximum
        if (row_ok && qt == 0) atomicMax(reinterpret_cast<unsigned *>(scale) + full_row, __float_as_uint(a));
        continue;
      }
      a = row_ok ? __uint_as_float(reinterpret_cast<const unsigned *>(scale)[full_row]) : 0.0f;
    }

    // g = 64, 256: norm_const is a power of two, so a = fl32(max|u| * c) = max|fl32(u * c)|.
    if constexpr (G == 64 || G == 256) a = a * norm_const<G>();
    constexpr float kQMax = FP8 ? 448.0f : 127.0f;
    const float s = a / kQMax;
    // Rows with a < 2^-100 are scaled by 2^100 (exact) before r = 127/a is formed,
    // which would otherwise overflow binary32.
    const bool tiny = a < 0x1p-100f;
    const float up = tiny ? 0x1p100f : 1.0f;
    const float as = a * up;
    const float r = (as > 0.0f) ? kQMax / as : 0.0f;
    if (!SEG && row_ok && qt == 0) scale[row] = s;

    // Multiplier turning the stored value into fl32(y * r).
    //  - g = 64/256, a >= 2^-100: y = u*c exactly for every value that can get a
    //    nonzero code, and (c * r) is exact, so fl32(u * (c*r)) = fl32(fl32(u*c) * r);
    //    values with u*c below the normal range give |y*r| < 2^-19 on both routes.
    //  - g = 1/128: the stored value already is y.
    //  - tiny rows: normalize exactly as written, scale by 2^100, then multiply by r.
    float mult = r;
    if (!tiny) {
      if constexpr (G == 64 || G == 256) mult = r * norm_const<G>() * sign;
    } else {
      float sc = 1.0f;
      if constexpr (G == 64 || G == 256) sc = sign * norm_const<G>();
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[i][j] = (v[i][j] * sc) * up;
    }

    {
      // Buffer stores over the group's rows: lanes past the last row or column
      // fall outside the buffer and are dropped.
      const int64_t nrows = group_rows(grp);
      const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(q + grp * rows_per_wg * cols), 0, (int)(nrows * cols), 0x00020000);
      const unsigned soff0 = (unsigned)(r_local * cols + base);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int64_t e0 = base + SPAN * i;
        const unsigned off = WHOLE ? soff0 : (e0 < cols) ? (unsigned)(r_local * cols + e0) : 0x80000000u;
        v2u packed;
        if constexpr (FP8) {
          float t[8];
#pragma unroll
          // + 0.0f stores an exact zero as +0: the per-lane sign trick can leave -0
          // where the butterfly cancels exactly
          for (int j = 0; j < 8; ++j) t[j] = fminf(fmaxf(v[i][j] * mult, -448.0f), 448.0f) + 0.0f;
          // bytes 0-1 then 2-3 of each dword, in value order
          packed[0] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
              t[2], t[3], __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false), true);
          packed[1] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
              t[6], t[7], __builtin_amdgcn_cvt_pk_fp8_f32(t[4], t[5], 0, false), true);
        } else {
          uint32_t c[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float t = v[i][j] * mult;
            c[j] = code_bits(t);
          }
          packed = (v2u){pack4(c[0], c[1], c[2], c[3]), pack4(c[4], c[5], c[6], c[7])};
        }
        // aux 2: the non-temporal bit of gfx950 buffer stores
        __builtin_amdgcn_raw_buffer_store_b64(packed, rq, off, WHOLE ? SPAN * i : 0, NT ? 2 : 0);
      }
    }
  }
}

// scale[row] = fl32(a / qmax) from the row maxima the segment phases left in
// scale (binary32 bits), with the same normalization step as the whole-row path.
template <int G, bool FP8>
__global__ void finish_scale_kernel(float *__restrict__ scale, int64_t rows) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows) return;
  float a = scale[i];
  if constexpr (G == 64 || G == 256) a = a * norm_const<G>();
  constexpr float kQMax = FP8 ? 448.0f : 127.0f;
  scale[i] = a / kQMax;
}

__global__ void zero_f32_kernel(float *__restrict__ out, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) out[i] = 0.0f;
}

// Rows per workgroup.  Smaller workgroups wait on fewer wavefronts at the per-group
// barrier, which measured faster even with some idle lanes: a [4096, 10240] matrix
// (160 lanes per row) took 24.7 us at one row per workgroup (three wavefronts, a
// sixth of the lanes idle) against 30.5 us at two rows (five full wavefronts).  So
// the fewest wavefronts that hold whole rows (as many as fit) with at most a fifth
// of the lanes idle; failing that, the count with the fewest idle lanes, then the
// one closest to 256 threads.
int pick_rows_per_wg(int t_row, int max_threads) {
  for (int waves = 1; 64 * waves <= max_threads; ++waves) {
    int r = 64 * waves / t_row;
    if (r > kMaxRowsPerWg) r = kMaxRowsPerWg;
    if (r < 1) continue;
    const int threads = r * t_row;
    if (5 * (64 * waves - threads) <= 64 * waves) return r;
  }
  int best_r = 1;
  double best_waste = 2.0;
  int best_dist = 1 << 30;
  for (int r = 1; r <= kMaxRowsPerWg && r * t_row <= max_threads; ++r) {
    const int threads = r * t_row;
    const int padded = (threads + 63) / 64 * 64;
    const double waste = double(padded - threads) / padded;
    const int dist = threads > 256 ? threads - 256 : 256 - threads;
    if (waste < best_waste - 1e-9 || (waste < best_waste + 1e-9 && dist < best_dist)) {
      best_r = r;
      best_waste = waste;
      best_dist = dist;
    }
  }
  return best_r;
}

// Resident workgroups per CU for a kernel at a block size, cached per block size
// (one atomic word holding both, so concurrent callers read a consistent pair).
// (One atomic word holds block size, dynamic LDS in 16-byte units and the count.)
template <int G, bool CS, int MAXT, bool FP8, bool SEG, bool WHOLE, bool NT, int LPS>
int blocks_per_cu(int threads, size_t smem) {
  static std::atomic<uint64_t> cache[kMaxThreads / 4 + 1];
  std::atomic<uint64_t> &slot = cache[threads / 4];
  const uint64_t key = ((uint64_t)(uint32_t)threads << 12) | (uint64_t)(smem / 16);
  const uint64_t c = slot.load(std::memory_order_relaxed);
  if ((c >> 32) == key) return (int)(c & 0xffffffffu);
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void *)rotq_kernel<G, CS, MAXT, FP8, SEG, WHOLE, NT, LPS>, threads, smem) !=
          hipSuccess ||
      n < 1)
    n = 1;
  slot.store((key << 32) | (uint32_t)n, std::memory_order_relaxed);
  return n;
}

// Codes written by plain stores stay dirty in the L2s (4 MB per XCD) when the
// whole output fits there, and the write-back at the kernel's end then runs after
// its last wave: x [4096, 3840] (15.7 MB of codes) took 10.5 us against 8.8 us
// with non-temporal stores.  Larger outputs are evicted while the kernel runs, as
// whole lines; non-temporal stores of them measured slower (h [4096, 10240], 42 MB:
// 23.8 against 27.6 us), so only outputs up to this size stream out.
constexpr int64_t kStreamCodesMax = 24ll << 20;

template <int G, bool CS, int MAXT, bool FP8, bool SEG, bool WHOLE, bool NT, int LPS>
hipError_t launch_grid(const uint16_t *x, int64_t rows, int64_t cols, const float *col_scale, int8_t *q,
                       float *scale, int t_row, int rpw, hipStream_t stream, int chunks, int phase) {
  const int threads = rpw * t_row;
  const int64_t groups = (rows + rpw - 1) / rpw;
  const size_t smem = (CS && !SEG && cols <= kColScaleLds) ? (size_t)cols * 4 : 0;
  // One workgroup per row group: the hardware starts each one as a slot frees,
  // which measured faster than a persistent grid walking the groups with its
  // prefetch (h [4096, 10240]: 23.2 against 24.9 us; x [8192, 3072] at g = 64:
  // 19.1 against 22.1 us).  With column scales staged in LDS every workgroup
  // first copies them (up to 64 KB), and the persistent grid, which copies them
  // once per workgroup, stays faster (dY [16384, 3072]: 26.9 against 28.6 us).
  // It takes as many workgroups as fit at once, evened out so that each walks the
  // same number of row groups (no last round that leaves most CUs idle).  So does
  // a group count beyond the grid's 2^31 - 1 workgroups.
  int64_t blocks = groups;
  if (smem > 0 || groups > 0x7fffffff) {
    blocks = (int64_t)device_cu_count() * blocks_per_cu<G, CS, MAXT, FP8, SEG, WHOLE, NT, LPS>(threads, smem);
    if (blocks > groups) blocks = groups;
    const int64_t rounds = (groups + blocks - 1) / blocks;
    blocks = (groups + rounds - 1) / rounds;
  }
  hipLaunchKernelGGL((rotq_kernel<G, CS, MAXT, FP8, SEG, WHOLE, NT, LPS>), dim3((unsigned)blocks), dim3(threads), smem,
                     stream, x, rows, cols, col_scale, q, scale, t_row, rpw, groups, chunks, phase);
  return hipGetLastError();
}

// LPS = 8 runs only on rows of an even number of whole superblocks (cols % 512 == 0),
// so that no lane of a row lies past its end.
template <int G, bool CS, int MAXT, bool FP8, bool SEG = false, int LPS = 4>
hipError_t launch_sized(const uint16_t *x, int64_t rows, int64_t cols, const float *col_scale, int8_t *q,
                        float *scale, int t_row, int rpw, hipStream_t stream, int chunks = 1, int phase = 0) {
  if constexpr (LPS == 4) {
    if (cols % 256 != 0)
      return launch_grid<G, CS, MAXT, FP8, SEG, false, false, 4>(x, rows, cols, col_scale, q, scale, t_row, rpw,
                                                                 stream, chunks, phase);
  } else if (cols % 512 != 0) {
    return hipErrorInvalidValue;
  }
  if (rows * cols <= kStreamCodesMax)
    return launch_grid<G, CS, MAXT, FP8, SEG, true, true, LPS>(x, rows, cols, col_scale, q, scale, t_row, rpw,
                                                               stream, chunks, phase);
  return launch_grid<G, CS, MAXT, FP8, SEG, true, false, LPS>(x, rows, cols, col_scale, q, scale, t_row, rpw,
                                                              stream, chunks, phase);
}

// Fraction of a workgroup's lanes that hold no values: rpw rows of t_row lanes,
// `used` of them holding values, rounded up to whole wavefronts.
double idle_lanes(int used, int t_row, int rpw) {
  const int padded = (rpw * t_row + 63) / 64 * 64;
  return double(padded - rpw * used) / padded;
}

// Segments per row for rows above 65536 values: the fewest equal segments of at
// most 65536 values that hold whole rotation blocks and keep 16-value alignment.
int64_t row_segments(int64_t cols, int g) {
  const int64_t unit = g > 16 ? g : 16;
  for (int64_t c = (cols + kMaxCols - 1) / kMaxCols; c <= cols / unit; ++c)
    if (cols % c == 0 && (cols / c) % unit == 0) return c;
  return 0;
}

template <int G, bool CS, bool FP8>
hipError_t launch_segmented(const uint16_t *x, int64_t rows, int64_t cols, const float *col_scale, int8_t *q,
                            float *scale, hipStream_t stream) {
  const int64_t chunks = row_segments(cols, G);
  if (chunks < 2) return hipErrorInvalidValue;
  const int64_t seg = cols / chunks, vrows = rows * chunks;
  const int t_row = 4 * (int)((seg + 255) / 256);
  const int rpw = pick_rows_per_wg(t_row, kMaxThreads);
  const unsigned fb = (unsigned)((rows + 255) / 256);
  hipLaunchKernelGGL(zero_f32_kernel, dim3(fb), dim3(256), 0, stream, scale, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int phase = 1; phase <= 2; ++phase) {
    e = launch_sized<G, CS, kMaxThreads, FP8, true>(x, vrows, seg, col_scale, q, scale, t_row, rpw, stream,
                                                    (int)chunks, phase);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((finish_scale_kernel<G, FP8>), dim3(fb), dim3(256), 0, stream, scale, rows);
  return hipGetLastError();
}

// Rows of up to 32768 values run in workgroups of at most 512 threads (up to 256
// VGPRs per lane, room for the prefetch buffer); longer rows need up to 1024.
template <int G, bool CS, bool FP8>
hipError_t launch_typed(const uint16_t *x, int64_t rows, int64_t cols, const float *col_scale,
                        int8_t *q, float *scale, hipStream_t stream) {
  if (cols > kMaxCols) return launch_segmented<G, CS, FP8>(x, rows, cols, col_scale, q, scale, stream);
  const int t_row = 4 * (int)((cols + 255) / 256);
  if (t_row <= 512) {
    const int rpw = pick_rows_per_wg(t_row, 512);
    // 8 lanes per superblock where that leaves fewer lanes idle: a 10240-wide row
    // fills five wavefronts (against three with a sixth of the lanes idle), 21.4
    // against 22.7 us for h [4096, 10240].  With column scales staged in LDS also
    // where both leave as many idle (dY [16384, 3072]: 25.9 against 26.9 us).
    if (cols % 512 == 0 && 2 * t_row <= 512) {
      const int rpw8 = pick_rows_per_wg(2 * t_row, 512);
      const double i8 = idle_lanes(2 * t_row, 2 * t_row, rpw8), i4 = idle_lanes(t_row, t_row, rpw);
      if (i8 < i4 || (CS && cols <= kColScaleLds && i8 <= i4))
        return launch_sized<G, CS, 512, FP8, false, 8>(x, rows, cols, col_scale, q, scale, 2 * t_row, rpw8, stream);
    }
    return launch_sized<G, CS, 512, FP8>(x, rows, cols, col_scale, q, scale, t_row, rpw, stream);
  }
  const int rpw = pick_rows_per_wg(t_row, kMaxThreads);
  return launch_sized<G, CS, kMaxThreads, FP8>(x, rows, cols, col_scale, q, scale, t_row, rpw, stream);
}

template <bool FP8>
hipError_t launch_any(const uint16_t *x, int64_t rows, int64_t cols, int g, const float *col_scale, int8_t *q,
                      float *scale, hipStream_t stream) {
  const bool cs = col_scale != nullptr;
  switch (g) {
    case 1: return cs ? launch_typed<1, true, FP8>(x, rows, cols, col_scale, q, scale, stream)
                      : launch_typed<1, false, FP8>(x, rows, cols, col_scale, q, scale, stream);
    case 64: return cs ? launch_typed<64, true, FP8>(x, rows, cols, col_scale, q, scale, stream)
                       : launch_typed<64, false, FP8>(x, rows, cols, col_scale, q, scale, stream);
    case 128: return cs ? launch_typed<128, true, FP8>(x, rows, cols, col_scale, q, scale, stream)
                        : launch_typed<128, false, FP8>(x, rows, cols, col_scale, q, scale, stream);
    case 256: return cs ? launch_typed<256, true, FP8>(x, rows, cols, col_scale, q, scale, stream)
                        : launch_typed<256, false, FP8>(x, rows, cols, col_scale, q, scale, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_rotate_quantize(const uint16_t *x, int64_t rows, int64_t cols, int g,
                                  const float *col_scale, int8_t *q, float *scale,
                                  hipStream_t stream) {
  return launch_any<false>(x, rows, cols, g, col_scale, q, scale, stream);
}

hipError_t launch_rotate_quantize_fp8(const uint16_t *x, int64_t rows, int64_t cols, int g,
                                      const float *col_scale, uint8_t *q, float *scale, hipStream_t stream) {
  return launch_any<true>(x, rows, cols, g, col_scale, reinterpret_cast<int8_t *>(q), scale, stream);
}

}  // namespace sdnq
