// C ABI of libsdnq_hip: argument validation, workspace carving and the launch
// sequence of each entry point.  Every check runs before the first launch, so a
// call that fails writes nothing.  See sdnq_hip.h for the contract.
#include <math.h>
#include <string.h>

#include <atomic>

#include "sdnq_internal.hpp"

using namespace sdnq;

namespace sdnq {
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
// bound of attn.hip's split-tile hand-over wait for later launches (0: give up
// at once)
void set_attention_handover_polls(uint32_t polls);
}  // namespace sdnq

namespace {

// Feature dimensions of the weight gradient, the low-rank split and their kernels.
constexpr int64_t kMaxFeature = 65536;
// Feature dimensions of the linear layer's forward and input gradient: 127 * 127 *
// K stays below 2^31 (exact int32 accumulators) up to K = 133144; the largest
// multiple of 16 below it.  Rows above 65536 values are quantized in segments.
constexpr int64_t kMaxLinearFeature = 133136;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_group(int32_t g) { return g == 1 || g == 64 || g == 128 || g == 256; }

constexpr int32_t kMaxSvdSteps = 64;

constexpr int32_t kMaxRank = 256;

bool valid_rank(int32_t rank) { return rank >= 1 && rank <= kMaxRank; }

// The kernels take LoRA ranks in multiples of 16 (one bf16 MFMA step); other ranks
// run zero-padded to the next multiple, which adds nothing to any product.
int32_t padded_rank(int32_t rank) { return (rank + 15) / 16 * 16; }

sdnq_status_t check_feature(int64_t d) {
  if (d <= 0) return SDNQ_ERR_INVALID_ARG;
  if (d % 16 != 0 || d > kMaxFeature) return SDNQ_ERR_UNSUPPORTED;
  return SDNQ_OK;
}

sdnq_status_t check_linear(int64_t d) {
  if (d <= 0) return SDNQ_ERR_INVALID_ARG;
  if (d % 16 != 0 || d > kMaxLinearFeature) return SDNQ_ERR_UNSUPPORTED;
  return SDNQ_OK;
}

// Workspace layouts (each region starts on a 256-byte boundary).
// With a rank that is not a multiple of 16, the regions marked "padded only" hold
// the zero-padded copies of the factors (and, in the forward with quantized
// activations, of the caller's t) and the padded LoRA gradients before cropping.
struct FwdLayout {
  size_t qx, sx, t, at, bt, bp, tp, total;
};
FwdLayout fwd_layout(int64_t m, int64_t n, int64_t k, int32_t rank) {
  FwdLayout L{};
  size_t off = 0;
  L.qx = off; off += align_up((size_t)m * (size_t)k);
  L.sx = off; off += align_up((size_t)m * 4);
  if (rank > 0) {
    const size_t rp = (size_t)padded_rank(rank);
    L.t = off; off += align_up((size_t)m * rp * 2);
    L.at = off; off += align_up(rp * (size_t)k * 2);
    L.bt = off; off += align_up((size_t)n * rp * 2);
    if (rp != (size_t)rank) {
      L.bp = off; off += align_up(rp * (size_t)n * 2);   // padded only: B [rp, n]
      L.tp = off; off += align_up((size_t)m * rp * 2);   // padded only: the caller's t [m, rp]
    }
  }
  L.total = off;
  return L;
}

struct BwdLayout {
  size_t qdy, sdy, wt, gr, tx, at, part, part2, bp, ap, gap, gbp, total;
  int splits;  // token splits of the LoRA gradient reduction
};
BwdLayout bwd_layout(int64_t m, int64_t n, int64_t k, int32_t rank) {
  BwdLayout L{};
  size_t off = 0;
  L.qdy = off; off += align_up((size_t)m * (size_t)n);
  L.sdy = off; off += align_up((size_t)m * 4);
  L.wt = off; off += align_up((size_t)k * (size_t)n);
  if (rank > 0) {
    const size_t rp = (size_t)padded_rank(rank);
    L.gr = off; off += align_up((size_t)m * rp * 2);
    L.tx = off; off += align_up((size_t)m * rp * 2);
    L.at = off; off += align_up(rp * (size_t)k * 2);
    L.splits = lora_grad_splits(m, lora_grad_tiles(k, n, (int64_t)rp));
    const size_t splits = (size_t)L.splits;
    L.part = off; off += align_up(splits * rp * (size_t)k * 4);   // dA partials
    L.part2 = off; off += align_up(splits * rp * (size_t)n * 4);  // dB partials
    if (rp != (size_t)rank) {
      L.bp = off; off += align_up(rp * (size_t)n * 2);    // padded only: B [rp, n]
      L.ap = off; off += align_up((size_t)k * rp * 2);    // padded only: A [k, rp]
      L.gap = off; off += align_up((size_t)k * rp * 2);   // padded only: dA [k, rp]
      L.gbp = off; off += align_up(rp * (size_t)n * 2);   // padded only: dB [rp, n]
    }
  }
  L.total = off;
  return L;
}

// Weight gradient: the per-feature absmax words of dy and x, then the two quantized
// transposed operands with their per-feature scales.
struct WgradLayout {
  size_t colmax, qdy, sdy, qx, sx, total;
};
WgradLayout wgrad_layout(int64_t m, int64_t n, int64_t k) {
  WgradLayout L{};
  size_t off = 0;
  L.colmax = off; off += align_up((size_t)(n + k) * 4);
  L.qdy = off; off += align_up((size_t)n * (size_t)m);
  L.sdy = off; off += align_up((size_t)n * 4);
  L.qx = off; off += align_up((size_t)k * (size_t)m);
  L.sx = off; off += align_up((size_t)k * 4);
  L.total = off;
  return L;
}

char *ws_at(void *ws, size_t off) { return static_cast<char *>(ws) + off; }

sdnq_status_t launched(hipError_t e) { return e == hipSuccess ? SDNQ_OK : SDNQ_ERR_LAUNCH; }

#define SDNQ_TRY(expr)                          \
  do {                                          \
    sdnq_status_t s_ = (expr);                  \
    if (s_ != SDNQ_OK) return s_;               \
  } while (0)

#define SDNQ_LAUNCH(expr)                       \
  do {                                          \
    hipError_t e_ = (expr);                     \
    if (e_ != hipSuccess) return SDNQ_ERR_LAUNCH; \
  } while (0)

// LoRA arguments: either no adapter (both factors NULL, any rank ignored) or both
// factors with a supported rank.
sdnq_status_t check_lora(const void *a, const void *b, int32_t rank, int32_t *eff_rank) {
  if (!a && !b) {
    *eff_rank = 0;
    return SDNQ_OK;
  }
  if (!a || !b) return SDNQ_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(b)) return SDNQ_ERR_INVALID_ARG;
  if (!valid_rank(rank)) return SDNQ_ERR_UNSUPPORTED;
  *eff_rank = rank;
  return SDNQ_OK;
}

sdnq_status_t check_rotq(const void *x, int64_t m, int64_t k, int32_t g, const void *col_scale, const void *q,
                         const void *s) {
  if (m < 0) return SDNQ_ERR_INVALID_ARG;
  if (m > 0 && (!x || !q || !s)) return SDNQ_ERR_INVALID_ARG;
  SDNQ_TRY(check_linear(k));
  if (!valid_group(g) || k % g != 0) return SDNQ_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return SDNQ_ERR_INVALID_ARG;
  if (col_scale && !aligned16(col_scale)) return SDNQ_ERR_INVALID_ARG;
  return SDNQ_OK;
}

}  // namespace

extern "C" {

const char *sdnq_status_string(sdnq_status_t status) {
  switch (status) {
    case SDNQ_OK: return "success";
    case SDNQ_ERR_INVALID_ARG: return "invalid argument (null pointer, non-positive size or misaligned pointer)";
    case SDNQ_ERR_UNSUPPORTED: return "unsupported configuration (block size, dimension multiple, size limit or rank)";
    case SDNQ_ERR_WORKSPACE: return "workspace missing or too small";
    case SDNQ_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

size_t sdnq_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t rank, int32_t is_backward) {
  if (m < 0 || check_linear(n) != SDNQ_OK || check_linear(k) != SDNQ_OK || rank < 0) return 0;
  if (rank > 0 && !valid_rank(rank)) return 0;
  return is_backward ? bwd_layout(m, n, k, rank).total : fwd_layout(m, n, k, rank).total;
}

sdnq_status_t sdnq_rotate_quantize_weight(const uint16_t *w, int64_t n, int64_t k, int32_t g, int8_t *qw,
                                          float *w_scale, void *stream) {
  SDNQ_TRY(check_rotq(w, n, k, g, nullptr, qw, w_scale));
  if (n == 0) return SDNQ_OK;
  (void)hipGetLastError();
  return launched(launch_rotate_quantize(w, n, k, g, nullptr, qw, w_scale, (hipStream_t)stream));
}

sdnq_status_t sdnq_rotate_quantize_act(const uint16_t *x, int64_t m, int64_t k, int32_t g, const float *col_scale,
                                       int8_t *qx, float *x_scale, void *stream) {
  SDNQ_TRY(check_rotq(x, m, k, g, col_scale, qx, x_scale));
  if (m == 0) return SDNQ_OK;
  (void)hipGetLastError();
  return launched(launch_rotate_quantize(x, m, k, g, col_scale, qx, x_scale, (hipStream_t)stream));
}

}  // extern "C"

namespace {

sdnq_status_t forward_quantized(bool fp8, const int8_t *qx, const float *x_scale, int64_t m, int64_t k,
                                const int8_t *qw, const float *w_scale, int64_t n, const uint16_t *t,
                                const uint16_t *lora_b, int32_t rank, float lora_scale, uint16_t *y,
                                void *workspace, size_t workspace_bytes, void *stream) {
  if (!qw || !w_scale || m < 0) return SDNQ_ERR_INVALID_ARG;
  if (m > 0 && (!qx || !x_scale || !y)) return SDNQ_ERR_INVALID_ARG;
  SDNQ_TRY(check_linear(k));
  SDNQ_TRY(check_linear(n));
  if (!aligned16(qx) || !aligned16(x_scale) || !aligned16(qw) || !aligned16(w_scale) || !aligned16(y))
    return SDNQ_ERR_INVALID_ARG;
  int32_t r = 0;
  SDNQ_TRY(check_lora(t, lora_b, rank, &r));
  const FwdLayout L = fwd_layout(m, n, k, r);
  if (r > 0 && (!workspace || workspace_bytes < L.total || !aligned16(workspace))) return SDNQ_ERR_WORKSPACE;
  if (m == 0) return SDNQ_OK;

  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  GemmArgs ga{};
  ga.a = qx; ga.b = qw; ga.m = m; ga.n = n; ga.k = k; ga.fp8 = fp8;
  ga.row_scale = x_scale; ga.col_scale = w_scale; ga.out_bf16 = y; ga.g = 1;
  if (r > 0) {
    const int32_t rp = padded_rank(r);
    const uint16_t *tsrc = t, *bsrc = lora_b;
    if (rp != r) {
      uint16_t *tp = reinterpret_cast<uint16_t *>(ws_at(workspace, L.tp));
      uint16_t *bp = reinterpret_cast<uint16_t *>(ws_at(workspace, L.bp));
      SDNQ_LAUNCH(launch_copy2d_u16(t, m, r, tp, m, rp, s));        // t [m, r] -> [m, rp]
      SDNQ_LAUNCH(launch_copy2d_u16(lora_b, r, n, bp, rp, n, s));   // B [r, n] -> [rp, n]
      tsrc = tp;
      bsrc = bp;
    }
    uint16_t *bt = reinterpret_cast<uint16_t *>(ws_at(workspace, L.bt));
    SDNQ_LAUNCH(launch_transpose_scale_bf16(bsrc, rp, n, lora_scale, bt, s));  // bf16(scale B)^T
    ga.lora_t = tsrc; ga.lora_r = bt; ga.rank = rp;
  }
  return launched(launch_gemm_i8(Epilogue::kForward, ga, s));
}

// Every check of the forward except the workspace's; *r is the effective rank.
sdnq_status_t check_forward(const uint16_t *x, int64_t m, int64_t k, const int8_t *qw, const float *w_scale,
                            int64_t n, int32_t g, const uint16_t *lora_a, const uint16_t *lora_b, int32_t rank,
                            const uint16_t *y, int32_t *r) {
  if (!qw || !w_scale || m < 0) return SDNQ_ERR_INVALID_ARG;
  if (m > 0 && (!x || !y)) return SDNQ_ERR_INVALID_ARG;
  SDNQ_TRY(check_linear(k));
  SDNQ_TRY(check_linear(n));
  if (!valid_group(g) || k % g != 0) return SDNQ_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(qw) || !aligned16(w_scale) || !aligned16(y)) return SDNQ_ERR_INVALID_ARG;
  return check_lora(lora_a, lora_b, rank, r);
}

sdnq_status_t forward(bool fp8, const uint16_t *x, int64_t m, int64_t k, const int8_t *qw, const float *w_scale,
                      int64_t n, int32_t g, const uint16_t *lora_a, const uint16_t *lora_b, int32_t rank,
                      float lora_scale, uint16_t *y, void *workspace, size_t workspace_bytes, void *stream) {
  int32_t r = 0;
  SDNQ_TRY(check_forward(x, m, k, qw, w_scale, n, g, lora_a, lora_b, rank, y, &r));
  const FwdLayout L = fwd_layout(m, n, k, r);
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return SDNQ_ERR_WORKSPACE;
  if (m == 0) return SDNQ_OK;

  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  int8_t *qx = reinterpret_cast<int8_t *>(ws_at(workspace, L.qx));
  float *sx = reinterpret_cast<float *>(ws_at(workspace, L.sx));
  if (fp8)
    SDNQ_LAUNCH(launch_rotate_quantize_fp8(x, m, k, g, nullptr, reinterpret_cast<uint8_t *>(qx), sx, s));
  else
    SDNQ_LAUNCH(launch_rotate_quantize(x, m, k, g, nullptr, qx, sx, s));

  GemmArgs ga{};
  ga.a = qx; ga.b = qw; ga.m = m; ga.n = n; ga.k = k; ga.fp8 = fp8;
  ga.row_scale = sx; ga.col_scale = w_scale; ga.out_bf16 = y; ga.g = 1;
  if (r > 0) {
    const int32_t rp = padded_rank(r);
    uint16_t *t = reinterpret_cast<uint16_t *>(ws_at(workspace, L.t));
    uint16_t *at = reinterpret_cast<uint16_t *>(ws_at(workspace, L.at));
    uint16_t *bt = reinterpret_cast<uint16_t *>(ws_at(workspace, L.bt));
    if (rp == r) {
      // A [k, r] -> A^T [r, k] and B [r, n] -> B^T [n, r] in one launch
      SDNQ_LAUNCH(launch_transpose_u16_pair(lora_a, k, r, at, lora_b, r, n, bt, s));
    } else {
      uint16_t *bp = reinterpret_cast<uint16_t *>(ws_at(workspace, L.bp));
      SDNQ_LAUNCH(launch_transpose_u16(lora_a, k, r, at, s));                           // A^T [r, k]
      SDNQ_LAUNCH(launch_fill_zero_u16(at + (int64_t)r * k, (int64_t)(rp - r) * k, s));  // A^T [rp, k]
      SDNQ_LAUNCH(launch_copy2d_u16(lora_b, r, n, bp, rp, n, s));                       // B [rp, n]
      SDNQ_LAUNCH(launch_transpose_u16(bp, rp, n, bt, s));                              // B^T [n, rp]
    }
    SDNQ_LAUNCH(launch_lora_down(x, m, k, at, rp, lora_scale, t, s));  // t = bf16(scale * x A)
    ga.lora_t = t; ga.lora_r = bt; ga.rank = rp;
  }
  return launched(launch_gemm_i8(Epilogue::kForward, ga, s));
}

}  // namespace

extern "C" {

sdnq_status_t sdnq_qlinear_forward_quantized(const int8_t *qx, const float *x_scale, int64_t m, int64_t k,
                                             const int8_t *qw, const float *w_scale, int64_t n, const uint16_t *t,
                                             const uint16_t *lora_b, int32_t rank, float lora_scale, uint16_t *y,
                                             void *workspace, size_t workspace_bytes, void *stream) {
  return forward_quantized(false, qx, x_scale, m, k, qw, w_scale, n, t, lora_b, rank, lora_scale, y, workspace,
                           workspace_bytes, stream);
}

sdnq_status_t sdnq_qlinear_forward(const uint16_t *x, int64_t m, int64_t k, const int8_t *qw, const float *w_scale,
                                   int64_t n, int32_t g, const uint16_t *lora_a, const uint16_t *lora_b,
                                   int32_t rank, float lora_scale, uint16_t *y, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  return forward(false, x, m, k, qw, w_scale, n, g, lora_a, lora_b, rank, lora_scale, y, workspace,
                 workspace_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------ forward without allocation --
// Callers that cannot allocate (code under HIP graph capture, tight serving
// loops) get the forward's workspace from this fixed device array instead.  The
// host-side name is only a stand-in: the device address is looked up once per
// device with hipGetSymbolAddress and that address is what the kernels get.
namespace {
constexpr size_t kScratchBytes = SDNQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_addr[kMaxDevices];

// The device address of `scratch` on the current device (nullptr on failure).
void *scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    scratch_addr[dev].store(p, std::memory_order_release);
  }
  return p;
}
}  // namespace

extern "C" {

sdnq_status_t sdnq_qlinear_forward_noalloc(const uint16_t *x, int64_t m, int64_t k, const int8_t *qw,
                                           const float *w_scale, int64_t n, int32_t g, const uint16_t *lora_a,
                                           const uint16_t *lora_b, int32_t rank, float lora_scale, uint16_t *y,
                                           void *stream) {
  int32_t r = 0;
  SDNQ_TRY(check_forward(x, m, k, qw, w_scale, n, g, lora_a, lora_b, rank, y, &r));
  if (fwd_layout(m, n, k, r).total > kScratchBytes) return SDNQ_ERR_WORKSPACE;
  void *ws = scratch_on_current_device();
  if (ws == nullptr) return SDNQ_ERR_LAUNCH;
  return forward(false, x, m, k, qw, w_scale, n, g, lora_a, lora_b, rank, lora_scale, y, ws, kScratchBytes, stream);
}

}  // extern "C"

namespace {

// The input gradient through the int8 (fp8 = false) or E4M3 (fp8 = true) weight codes.
// qw_transposed: qw holds the codes as [k, n] (made once by sdnq_transpose_codes)
// instead of [n, k], and the per-call transpose is skipped.
sdnq_status_t backward(bool fp8, bool qw_transposed, const uint16_t *dy, int64_t m, int64_t n, const int8_t *qw,
                       const float *w_scale,
                       int64_t k, int32_t g, const uint16_t *x, const uint16_t *lora_a, const uint16_t *lora_b,
                       int32_t rank, float lora_scale, uint16_t *dx, uint16_t *grad_a, uint16_t *grad_b,
                       void *workspace, size_t workspace_bytes, void *stream) {
  if (!qw || !w_scale || m < 0) return SDNQ_ERR_INVALID_ARG;
  if (m > 0 && (!dy || !dx)) return SDNQ_ERR_INVALID_ARG;
  SDNQ_TRY(check_linear(k));
  SDNQ_TRY(check_linear(n));
  if (!valid_group(g) || k % g != 0) return SDNQ_ERR_UNSUPPORTED;
  if (!aligned16(dy) || !aligned16(qw) || !aligned16(w_scale) || !aligned16(dx)) return SDNQ_ERR_INVALID_ARG;
  int32_t r = 0;
  SDNQ_TRY(check_lora(lora_a, lora_b, rank, &r));
  const bool want_ga = grad_a != nullptr, want_gb = grad_b != nullptr;
  if ((want_ga || want_gb) && (r == 0 || (m > 0 && !x))) return SDNQ_ERR_INVALID_ARG;
  if ((x && !aligned16(x)) || (grad_a && !aligned16(grad_a)) || (grad_b && !aligned16(grad_b)))
    return SDNQ_ERR_INVALID_ARG;
  const BwdLayout L = bwd_layout(m, n, k, r);
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return SDNQ_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  if (m == 0) {
    // Empty batch: the LoRA gradients are empty sums.
    (void)hipGetLastError();
    if (want_ga) SDNQ_LAUNCH(launch_fill_zero_u16(grad_a, k * r, s));
    if (want_gb) SDNQ_LAUNCH(launch_fill_zero_u16(grad_b, (int64_t)r * n, s));
    return SDNQ_OK;
  }
  (void)hipGetLastError();
  int8_t *qdy = reinterpret_cast<int8_t *>(ws_at(workspace, L.qdy));
  float *sdy = reinterpret_cast<float *>(ws_at(workspace, L.sdy));
  const int8_t *wt = qw_transposed ? qw : reinterpret_cast<int8_t *>(ws_at(workspace, L.wt));
  // dY' = dY * w_scale (column fold), per-token quantization, no rotation along n.
  if (fp8)
    SDNQ_LAUNCH(launch_rotate_quantize_fp8(dy, m, n, 1, w_scale, reinterpret_cast<uint8_t *>(qdy), sdy, s));
  else
    SDNQ_LAUNCH(launch_rotate_quantize(dy, m, n, 1, w_scale, qdy, sdy, s));
  if (!qw_transposed)  // qw [n, k] -> [k, n] (bytes, either code)
    SDNQ_LAUNCH(launch_transpose_i8(qw, n, k, const_cast<int8_t *>(wt), s));

  GemmArgs ga{};
  ga.a = qdy; ga.b = wt; ga.m = m; ga.n = k; ga.k = n; ga.fp8 = fp8;
  ga.row_scale = sdy; ga.out_bf16 = dx; ga.g = g;
  uint16_t *gr = nullptr, *tx = nullptr, *at = nullptr;
  const int32_t rp = r > 0 ? padded_rank(r) : 0;
  const bool padded = rp != r;
  const uint16_t *asrc = lora_a, *bsrc = lora_b;
  if (r > 0) {
    if (padded) {
      uint16_t *ap = reinterpret_cast<uint16_t *>(ws_at(workspace, L.ap));
      uint16_t *bp = reinterpret_cast<uint16_t *>(ws_at(workspace, L.bp));
      SDNQ_LAUNCH(launch_copy2d_u16(lora_a, k, r, ap, k, rp, s));   // A [k, r] -> [k, rp]
      SDNQ_LAUNCH(launch_copy2d_u16(lora_b, r, n, bp, rp, n, s));   // B [r, n] -> [rp, n]
      asrc = ap;
      bsrc = bp;
    }
    gr = reinterpret_cast<uint16_t *>(ws_at(workspace, L.gr));
    if (want_gb) {
      // g_r = scale * dY B^T and t = x A (for dB) in one launch
      tx = reinterpret_cast<uint16_t *>(ws_at(workspace, L.tx));
      at = reinterpret_cast<uint16_t *>(ws_at(workspace, L.at));
      SDNQ_LAUNCH(launch_transpose_u16(asrc, k, rp, at, s));
      SDNQ_LAUNCH(launch_lora_down2(dy, n, bsrc, lora_scale, gr, x, k, at, 1.0f, tx, m, rp, s));
    } else {
      SDNQ_LAUNCH(launch_lora_down(dy, m, n, bsrc, rp, lora_scale, gr, s));  // g_r = scale * dY B^T
    }
    ga.lora_t = gr; ga.lora_r = asrc; ga.rank = rp;  // + g_r A^T
  }
  SDNQ_LAUNCH(launch_gemm_i8(Epilogue::kBackward, ga, s));

  if (r > 0 && (want_ga || want_gb)) {
    // dA = x^T g_r and dB = scale * (dY^T t)^T, reduced over the tokens in one
    // launch (and their sums in another)
    float *part_a = reinterpret_cast<float *>(ws_at(workspace, L.part));
    float *part_b = reinterpret_cast<float *>(ws_at(workspace, L.part2));
    uint16_t *dst_a = padded ? reinterpret_cast<uint16_t *>(ws_at(workspace, L.gap)) : grad_a;
    uint16_t *dst_b = padded ? reinterpret_cast<uint16_t *>(ws_at(workspace, L.gbp)) : grad_b;
    if (want_ga && want_gb)
      SDNQ_LAUNCH(launch_lora_grad2(x, k, gr, 1.0f, false, part_a, dst_a, dy, n, tx, lora_scale, true, part_b, dst_b,
                                    rp, m, L.splits, s));
    else if (want_ga)
      SDNQ_LAUNCH(launch_lora_grad(x, k, gr, rp, m, 1.0f, false, part_a, dst_a, L.splits, s));
    else
      SDNQ_LAUNCH(launch_lora_grad(dy, n, tx, rp, m, lora_scale, true, part_b, dst_b, L.splits, s));
    if (padded && want_ga) SDNQ_LAUNCH(launch_copy2d_u16(dst_a, k, rp, grad_a, k, r, s));
    if (padded && want_gb) SDNQ_LAUNCH(launch_copy2d_u16(dst_b, rp, n, grad_b, r, n, s));
  }
  return SDNQ_OK;
}

}  // namespace

extern "C" {

sdnq_status_t sdnq_qlinear_backward_input(const uint16_t *dy, int64_t m, int64_t n, const int8_t *qw,
                                          const float *w_scale, int64_t k, int32_t g, const uint16_t *x,
                                          const uint16_t *lora_a, const uint16_t *lora_b, int32_t rank,
                                          float lora_scale, uint16_t *dx, uint16_t *grad_a, uint16_t *grad_b,
                                          void *workspace, size_t workspace_bytes, void *stream) {
  return backward(false, false, dy, m, n, qw, w_scale, k, g, x, lora_a, lora_b, rank, lora_scale, dx, grad_a,
                  grad_b, workspace, workspace_bytes, stream);
}

sdnq_status_t sdnq_qlinear_backward_input_wt(const uint16_t *dy, int64_t m, int64_t n, const int8_t *qw_t,
                                             const float *w_scale, int64_t k, int32_t g, const uint16_t *x,
                                             const uint16_t *lora_a, const uint16_t *lora_b, int32_t rank,
                                             float lora_scale, uint16_t *dx, uint16_t *grad_a, uint16_t *grad_b,
                                             void *workspace, size_t workspace_bytes, void *stream) {
  return backward(false, true, dy, m, n, qw_t, w_scale, k, g, x, lora_a, lora_b, rank, lora_scale, dx, grad_a,
                  grad_b, workspace, workspace_bytes, stream);
}

sdnq_status_t sdnq_qlinear_backward_input_fp8(const uint16_t *dy, int64_t m, int64_t n, const uint8_t *qw,
                                              const float *w_scale, int64_t k, int32_t g, const uint16_t *x,
                                              const uint16_t *lora_a, const uint16_t *lora_b, int32_t rank,
                                              float lora_scale, uint16_t *dx, uint16_t *grad_a, uint16_t *grad_b,
                                              void *workspace, size_t workspace_bytes, void *stream) {
  return backward(true, false, dy, m, n, reinterpret_cast<const int8_t *>(qw), w_scale, k, g, x, lora_a, lora_b,
                  rank, lora_scale, dx, grad_a, grad_b, workspace, workspace_bytes, stream);
}

sdnq_status_t sdnq_qlinear_backward_input_fp8_wt(const uint16_t *dy, int64_t m, int64_t n, const uint8_t *qw_t,
                                                 const float *w_scale, int64_t k, int32_t g, const uint16_t *x,
                                                 const uint16_t *lora_a, const uint16_t *lora_b, int32_t rank,
                                                 float lora_scale, uint16_t *dx, uint16_t *grad_a, uint16_t *grad_b,
                                                 void *workspace, size_t workspace_bytes, void *stream) {
  return backward(true, true, dy, m, n, reinterpret_cast<const int8_t *>(qw_t), w_scale, k, g, x, lora_a, lora_b,
                  rank, lora_scale, dx, grad_a, grad_b, workspace, workspace_bytes, stream);
}

sdnq_status_t sdnq_transpose_codes(const uint8_t *in, int64_t rows, int64_t cols, uint8_t *out, void *stream) {
  if (!in || !out || rows < 0 || cols < 0) return SDNQ_ERR_INVALID_ARG;
  SDNQ_TRY(check_linear(rows));
  SDNQ_TRY(check_linear(cols));
  if (!aligned16(in) || !aligned16(out)) return SDNQ_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return launched(launch_transpose_i8(reinterpret_cast<const int8_t *>(in), rows, cols,
                                      reinterpret_cast<int8_t *>(out), (hipStream_t)stream));
}

sdnq_status_t sdnq_gemm_i8_i32(const int8_t *a, const int8_t *b, int64_t m, int64_t n, int64_t k, int32_t b_layout,
                               int32_t *c, void *workspace, size_t workspace_bytes, void *stream) {
  if (!b || m < 0) return SDNQ_ERR_INVALID_ARG;
  if (m > 0 && (!a || !c)) return SDNQ_ERR_INVALID_ARG;
  SDNQ_TRY(check_linear(k));
  SDNQ_TRY(check_linear(n));
  if (b_layout != 0 && b_layout != 1) return SDNQ_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return SDNQ_ERR_INVALID_ARG;
  if (b_layout == 1 && (!workspace || workspace_bytes < (size_t)k * (size_t)n || !aligned16(workspace)))
    return SDNQ_ERR_WORKSPACE;
  if (m == 0) return SDNQ_OK;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  const int8_t *bb = b;
  if (b_layout == 1) {
    int8_t *bt = static_cast<int8_t *>(workspace);
    SDNQ_LAUNCH(launch_transpose_i8(b, k, n, bt, s));  // b [k, n] -> [n, k]
    bb = bt;
  }
  GemmArgs ga{};
  ga.a = a; ga.b = bb; ga.m = m; ga.n = n; ga.k = k; ga.c_i32 = c; ga.g = 1;
  return launched(launch_gemm_i8(Epilogue::kInt32, ga, s));
}

sdnq_status_t sdnq_gemm_i8_ceiling(const int8_t *qx, const float *x_scale, int64_t m, int64_t k, const int8_t *qw,
                                   const float *w_scale, int64_t n, int32_t mode, uint16_t *y, void *stream) {
  if (!qw || !w_scale || m < 0) return SDNQ_ERR_INVALID_ARG;
  if (m > 0 && (!qx || !x_scale || !y)) return SDNQ_ERR_INVALID_ARG;
  if (mode < 0 || mode > 3) return SDNQ_ERR_INVALID_ARG;
  SDNQ_TRY(check_linear(k));
  SDNQ_TRY(check_linear(n));
  if (!aligned16(qx) || !aligned16(x_scale) || !aligned16(qw) || !aligned16(w_scale) || !aligned16(y))
    return SDNQ_ERR_INVALID_ARG;
  if (m == 0) return SDNQ_OK;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  GemmArgs ga{};
  ga.a = qx; ga.b = qw; ga.m = m; ga.n = n; ga.k = k;
  ga.row_scale = x_scale; ga.col_scale = w_scale; ga.out_bf16 = y; ga.g = 1;
  return launched(launch_gemm_i8_ceiling(ga, mode, s));
}

// ----------------------------------------------------- weight gradient --
size_t sdnq_weight_grad_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || check_feature(n) != SDNQ_OK || check_feature(k) != SDNQ_OK) return 0;
  if (m > 0 && check_feature(m) != SDNQ_OK) return 0;
  return wgrad_layout(m, n, k).total;
}

size_t sdnq_weight_grad_workspace_offset(int64_t m, int64_t n, int64_t k, int32_t which) {
  if (which < 0 || which > 3 || sdnq_weight_grad_workspace_bytes(m, n, k) == 0) return 0;
  const WgradLayout L = wgrad_layout(m, n, k);
  const size_t off[4] = {L.qdy, L.sdy, L.qx, L.sx};
  return off[which];
}

sdnq_status_t sdnq_qlinear_weight_grad(const uint16_t *dy, const uint16_t *x, int64_t m, int64_t n, int64_t k,
                                       int32_t g, uint16_t *dw, void *workspace, size_t workspace_bytes,
                                       void *stream) {
  if (!dw || m < 0) return SDNQ_ERR_INVALID_ARG;
  if (m > 0 && (!dy || !x)) return SDNQ_ERR_INVALID_ARG;
  SDNQ_TRY(check_feature(n));
  SDNQ_TRY(check_feature(k));
  if (!valid_group(g)) return SDNQ_ERR_UNSUPPORTED;
  if (m > 0) {
    SDNQ_TRY(check_feature(m));  // the tokens are the contraction here
    if (m % g != 0) return SDNQ_ERR_UNSUPPORTED;
  }
  if (!aligned16(dy) || !aligned16(x) || !aligned16(dw)) return SDNQ_ERR_INVALID_ARG;
  const WgradLayout L = wgrad_layout(m, n, k);
  if (m > 0 && (!workspace || workspace_bytes < L.total || !aligned16(workspace))) return SDNQ_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (m == 0) return launched(launch_fill_zero_u16(dw, n * k, s));  // empty sum
  uint32_t *colmax = reinterpret_cast<uint32_t *>(ws_at(workspace, L.colmax));
  int8_t *qdy = reinterpret_cast<int8_t *>(ws_at(workspace, L.qdy));
  float *sdy = reinterpret_cast<float *>(ws_at(workspace, L.sdy));
  int8_t *qx = reinterpret_cast<int8_t *>(ws_at(workspace, L.qx));
  float *sx = reinterpret_cast<float *>(ws_at(workspace, L.sx));
  SDNQ_LAUNCH(launch_fill_zero_u16(reinterpret_cast<uint16_t *>(colmax), 2 * (n + k), s));
  // per feature, rotated along the tokens: the codes of dy^T [n, m] and x^T [k, m]
  SDNQ_LAUNCH(launch_colq_pair(dy, n, qdy, sdy, x, k, qx, sx, m, g, colmax, s));
  GemmArgs ga{};
  ga.a = qdy; ga.b = qx; ga.m = n; ga.n = k; ga.k = m;
  ga.row_scale = sdy; ga.col_scale = sx; ga.out_bf16 = dw; ga.g = 1;
  return launched(launch_gemm_i8(Epilogue::kForward, ga, s));
}

// ---------------------------------------------------------------- FP8 --
sdnq_status_t sdnq_rotate_quantize_weight_fp8(const uint16_t *w, int64_t n, int64_t k, int32_t g, uint8_t *qw,
                                              float *w_scale, void *stream) {
  SDNQ_TRY(check_rotq(w, n, k, g, nullptr, qw, w_scale));
  if (n == 0) return SDNQ_OK;
  (void)hipGetLastError();
  return launched(launch_rotate_quantize_fp8(w, n, k, g, nullptr, qw, w_scale, (hipStream_t)stream));
}

sdnq_status_t sdnq_rotate_quantize_act_fp8(const uint16_t *x, int64_t m, int64_t k, int32_t g,
                                           const float *col_scale, uint8_t *qx, float *x_scale, void *stream) {
  SDNQ_TRY(check_rotq(x, m, k, g, col_scale, qx, x_scale));
  if (m == 0) return SDNQ_OK;
  (void)hipGetLastError();
  return launched(launch_rotate_quantize_fp8(x, m, k, g, col_scale, qx, x_scale, (hipStream_t)stream));
}

sdnq_status_t sdnq_qlinear_forward_fp8(const uint16_t *x, int64_t m, int64_t k, const uint8_t *qw,
                                       const float *w_scale, int64_t n, int32_t g, const uint16_t *lora_a,
                                       const uint16_t *lora_b, int32_t rank, float lora_scale, uint16_t *y,
                                       void *workspace, size_t workspace_bytes, void *stream) {
  return forward(true, x, m, k, reinterpret_cast<const int8_t *>(qw), w_scale, n, g, lora_a, lora_b, rank,
                 lora_scale, y, workspace, workspace_bytes, stream);
}

sdnq_status_t sdnq_qlinear_forward_fp8_quantized(const uint8_t *qx, const float *x_scale, int64_t m, int64_t k,
                                                 const uint8_t *qw, const float *w_scale, int64_t n,
                                                 const uint16_t *t, const uint16_t *lora_b, int32_t rank,
                                                 float lora_scale, uint16_t *y, void *workspace,
                                                 size_t workspace_bytes, void *stream) {
  return forward_quantized(true, reinterpret_cast<const int8_t *>(qx), x_scale, m, k,
                           reinterpret_cast<const int8_t *>(qw), w_scale, n, t, lora_b, rank, lora_scale, y,
                           workspace, workspace_bytes, stream);
}

sdnq_status_t sdnq_gemm_fp8_f32(const uint8_t *a, const uint8_t *b, int64_t m, int64_t n, int64_t k, float *c,
                                void *stream) {
  if (!b || m < 0) return SDNQ_ERR_INVALID_ARG;
  if (m > 0 && (!a || !c)) return SDNQ_ERR_INVALID_ARG;
  SDNQ_TRY(check_linear(k));
  SDNQ_TRY(check_linear(n));
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return SDNQ_ERR_INVALID_ARG;
  if (m == 0) return SDNQ_OK;
  (void)hipGetLastError();
  GemmArgs ga{};
  ga.a = reinterpret_cast<const int8_t *>(a); ga.b = reinterpret_cast<const int8_t *>(b);
  ga.m = m; ga.n = n; ga.k = k; ga.c_i32 = reinterpret_cast<int32_t *>(c); ga.g = 1; ga.fp8 = true;
  return launched(launch_gemm_i8(Epilogue::kInt32, ga, (hipStream_t)stream));
}

// ------------------------------------------------------ low-rank (SVD) split --
size_t sdnq_svd_workspace_bytes(int64_t n, int64_t k, int32_t rank) {
  if (check_feature(n) != SDNQ_OK || check_feature(k) != SDNQ_OK) return 0;
  if (!(rank == 16 || rank == 32 || rank == 64) || rank > n || rank > k) return 0;
  return svd_workspace_bytes(n, k, rank);
}

size_t sdnq_svd_workspace_q_offset(int64_t n, int64_t k, int32_t rank) {
  if (sdnq_svd_workspace_bytes(n, k, rank) == 0) return 0;
  return svd_workspace_q_offset(n, k, rank);
}

sdnq_status_t sdnq_svd_quantize_weight(const uint16_t *w, int64_t n, int64_t k, int32_t g, int32_t rank,
                                       int32_t steps, const float *omega, int8_t *qw, float *w_scale,
                                       uint16_t *svd_a, uint16_t *svd_b, void *workspace, size_t workspace_bytes,
                                       void *stream) {
  if (!w || !omega || !qw || !w_scale || !svd_a || !svd_b) return SDNQ_ERR_INVALID_ARG;
  SDNQ_TRY(check_feature(n));
  SDNQ_TRY(check_feature(k));
  if (!valid_group(g) || k % g != 0) return SDNQ_ERR_UNSUPPORTED;
  if (!(rank == 16 || rank == 32 || rank == 64) || rank > n || rank > k) return SDNQ_ERR_UNSUPPORTED;
  if (steps < 0 || steps > kMaxSvdSteps) return SDNQ_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(omega) || !aligned16(qw) || !aligned16(w_scale) || !aligned16(svd_a) ||
      !aligned16(svd_b))
    return SDNQ_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace) || workspace_bytes < svd_workspace_bytes(n, k, rank))
    return SDNQ_ERR_WORKSPACE;
  (void)hipGetLastError();
  return launched(launch_svd_quantize_weight(w, n, k, g, rank, steps, omega, qw, w_scale, svd_a, svd_b, workspace,
                                             (hipStream_t)stream));
}

// ------------------------------------------------------- int8 attention --
static sdnq_status_t check_attention(const void *q, const void *k, const void *v, int64_t bsz, int64_t hq, int64_t hkv,
                                     int64_t sq, int64_t sk, int64_t d, float scale, int32_t g, const void *out) {
  if (!q || !k || !v || !out) return SDNQ_ERR_INVALID_ARG;
  if (bsz <= 0 || hq <= 0 || hkv <= 0 || sq <= 0 || sk <= 0) return SDNQ_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !(scale < INFINITY)) return SDNQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SDNQ_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SDNQ_ERR_UNSUPPORTED;
  if (hq % hkv != 0 || sk % 16 != 0 || sq > (1 << 20) || sk > (1 << 20)) return SDNQ_ERR_UNSUPPORTED;
  // grid limits: with at most 65535 heads and 2^20 tokens the forward's
  // one-dimensional grid of (head, 128-query tile) stays below 2^31 workgroups
  if (bsz * hq > 65535 || bsz * hkv > 65535) return SDNQ_ERR_UNSUPPORTED;
  if (bsz * hq * sq > (int64_t(1) << 31) || bsz * hkv * sk > (int64_t(1) << 31)) return SDNQ_ERR_UNSUPPORTED;
  if (!(g == 0 || g == 1 || g == 64 || g == 128 || g == 256)) return SDNQ_ERR_UNSUPPORTED;
  return SDNQ_OK;
}

size_t sdnq_attention_workspace_bytes(int64_t batch, int64_t heads_q, int64_t heads_kv, int64_t seq_q,
                                      int64_t seq_k, int64_t head_dim) {
  static const int probe[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
  if (check_attention(probe, probe, probe, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, 1.0f, 256, probe) !=
      SDNQ_OK)
    return 0;
  return attention_workspace_bytes(batch, heads_q, heads_kv, seq_q, seq_k, head_dim);
}

size_t sdnq_attention_workspace_offset(int64_t batch, int64_t heads_q, int64_t heads_kv, int64_t seq_q,
                                       int64_t seq_k, int64_t head_dim, int32_t which) {
  if (which < 0 || which > 5 || sdnq_attention_workspace_bytes(batch, heads_q, heads_kv, seq_q, seq_k, head_dim) == 0)
    return 0;
  size_t off[6];
  attention_workspace_offsets(batch, heads_q, heads_kv, seq_q, seq_k, head_dim, off);
  return off[which];
}

sdnq_status_t sdnq_attention_int8(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t batch,
                                  int64_t heads_q, int64_t heads_kv, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                                  int32_t is_causal, float scale, int32_t smooth_k, int32_t hadamard_group,
                                  uint16_t *out, void *workspace, size_t workspace_bytes, void *stream) {
  SDNQ_TRY(check_attention(q, k, v, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, scale, hadamard_group, out));
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < attention_workspace_bytes(batch, heads_q, heads_kv, seq_q, seq_k, head_dim))
    return SDNQ_ERR_WORKSPACE;
  (void)hipGetLastError();
  return launched(launch_attention_int8(q, k, v, batch, heads_q, heads_kv, seq_q, seq_k, head_dim, is_causal != 0,
                                        scale, smooth_k != 0, hadamard_group, out, workspace, (hipStream_t)stream));
}

sdnq_status_t sdnq_attention_set_handover_polls(uint32_t polls) {
  set_attention_handover_polls(polls);
  return SDNQ_OK;
}

}  // extern "C"
