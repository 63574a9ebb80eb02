"""ctypes binding of libsdnq_hip.so (the C ABI declared in include/sdnq_hip.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch tensors supply device memory and the current HIP stream; the
functions check dtype, device, shape and contiguity, allocate outputs (and the
workspace when none is given) with torch, and call the entry point of the same
name.  A missing or unloadable library raises at the first call; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsdnq_hip.so")

SDNQ_OK, SDNQ_ERR_INVALID_ARG, SDNQ_ERR_UNSUPPORTED, SDNQ_ERR_WORKSPACE, SDNQ_ERR_LAUNCH = range(5)

_lib = None


class SdnqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or python hadamard_rotated_int8_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    sigs = {
        "sdnq_rotate_quantize_weight": [p, i64, i64, i32, p, p, p],
        "sdnq_rotate_quantize_act": [p, i64, i64, i32, p, p, p, p],
        "sdnq_qlinear_forward": [p, i64, i64, p, p, i64, i32, p, p, i32, f32, p, p, sz, p],
        "sdnq_qlinear_forward_noalloc": [p, i64, i64, p, p, i64, i32, p, p, i32, f32, p, p],
        "sdnq_qlinear_forward_quantized": [p, p, i64, i64, p, p, i64, p, p, i32, f32, p, p, sz, p],
        "sdnq_qlinear_backward_input": [p, i64, i64, p, p, i64, i32, p, p, p, i32, f32, p, p, p, p, sz, p],
        "sdnq_qlinear_backward_input_fp8": [p, i64, i64, p, p, i64, i32, p, p, p, i32, f32, p, p, p, p, sz, p],
        "sdnq_qlinear_backward_input_wt": [p, i64, i64, p, p, i64, i32, p, p, p, i32, f32, p, p, p, p, sz, p],
        "sdnq_qlinear_backward_input_fp8_wt": [p, i64, i64, p, p, i64, i32, p, p, p, i32, f32, p, p, p, p, sz, p],
        "sdnq_transpose_codes": [p, i64, i64, p, p],
        "sdnq_gemm_i8_i32": [p, p, i64, i64, i64, i32, p, p, sz, p],
        "sdnq_gemm_i8_ceiling": [p, p, i64, i64, p, p, i64, i32, p, p],
        "sdnq_rotate_quantize_weight_fp8": [p, i64, i64, i32, p, p, p],
        "sdnq_rotate_quantize_act_fp8": [p, i64, i64, i32, p, p, p, p],
        "sdnq_qlinear_forward_fp8": [p, i64, i64, p, p, i64, i32, p, p, i32, f32, p, p, sz, p],
        "sdnq_qlinear_forward_fp8_quantized": [p, p, i64, i64, p, p, i64, p, p, i32, f32, p, p, sz, p],
        "sdnq_gemm_fp8_f32": [p, p, i64, i64, i64, p, p],
        "sdnq_qlinear_weight_grad": [p, p, i64, i64, i64, i32, p, p, sz, p],
        "sdnq_svd_quantize_weight": [p, i64, i64, i32, i32, i32, p, p, p, p, p, p, sz, p],
        "sdnq_attention_int8": [p, p, p, i64, i64, i64, i64, i64, i64, i32, ctypes.c_float, i32, i32, p, p, sz, p],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.sdnq_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    L.sdnq_workspace_bytes.restype = sz
    L.sdnq_weight_grad_workspace_bytes.argtypes = [i64, i64, i64]
    L.sdnq_weight_grad_workspace_bytes.restype = sz
    L.sdnq_weight_grad_workspace_offset.argtypes = [i64, i64, i64, i32]
    L.sdnq_weight_grad_workspace_offset.restype = sz
    L.sdnq_svd_workspace_bytes.argtypes = [i64, i64, i32]
    L.sdnq_svd_workspace_bytes.restype = sz
    L.sdnq_svd_workspace_q_offset.argtypes = [i64, i64, i32]
    L.sdnq_svd_workspace_q_offset.restype = sz
    L.sdnq_attention_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64]
    L.sdnq_attention_workspace_bytes.restype = sz
    L.sdnq_attention_workspace_offset.argtypes = [i64, i64, i64, i64, i64, i64, i32]
    L.sdnq_attention_workspace_offset.restype = sz
    L.sdnq_attention_set_handover_polls.argtypes = [ctypes.c_uint32]
    L.sdnq_attention_set_handover_polls.restype = ctypes.c_int
    L.sdnq_status_string.argtypes = [ctypes.c_int]
    L.sdnq_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().sdnq_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != SDNQ_OK:
        raise SdnqError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, dtype, ndim, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def _workspace(nbytes: int, dev, workspace):
    if workspace is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return workspace


def sdnq_workspace_bytes(m: int, n: int, k: int, rank: int = 0, is_backward: bool = False) -> int:
    return int(lib().sdnq_workspace_bytes(m, n, k, rank, int(bool(is_backward))))


def _rotate_quantize_weight(name, code_dtype, w, g):
    _need(w, torch.bfloat16, 2, "w")
    n, k = w.shape
    qw = torch.empty((n, k), dtype=code_dtype, device=w.device)
    sw = torch.empty((n,), dtype=torch.float32, device=w.device)
    _check(getattr(lib(), name)(_ptr(w), n, k, g, _ptr(qw), _ptr(sw), _stream(w.device)), name)
    return qw, sw


def _rotate_quantize_act(name, code_dtype, x, g, col_scale):
    _need(x, torch.bfloat16, 2, "x")
    if col_scale is not None:
        _need(col_scale, torch.float32, 1, "col_scale")
    m, k = x.shape
    qx = torch.empty((m, k), dtype=code_dtype, device=x.device)
    sx = torch.empty((m,), dtype=torch.float32, device=x.device)
    _check(getattr(lib(), name)(_ptr(x), m, k, g, _ptr(col_scale), _ptr(qx), _ptr(sx), _stream(x.device)), name)
    return qx, sx


def sdnq_rotate_quantize_weight(w: torch.Tensor, g: int):
    """W [n, k] bf16 -> (qw [n, k] int8, w_scale [n] fp32)."""
    return _rotate_quantize_weight("sdnq_rotate_quantize_weight", torch.int8, w, g)


def sdnq_rotate_quantize_act(x: torch.Tensor, g: int, col_scale: torch.Tensor | None = None):
    """x [m, k] bf16 -> (qx [m, k] int8, x_scale [m] fp32)."""
    return _rotate_quantize_act("sdnq_rotate_quantize_act", torch.int8, x, g, col_scale)


def sdnq_rotate_quantize_weight_fp8(w: torch.Tensor, g: int):
    """W [n, k] bf16 -> (qw [n, k] E4M3 codes as uint8, w_scale [n] fp32)."""
    return _rotate_quantize_weight("sdnq_rotate_quantize_weight_fp8", torch.uint8, w, g)


def sdnq_rotate_quantize_act_fp8(x: torch.Tensor, g: int, col_scale: torch.Tensor | None = None):
    """x [m, k] bf16 -> (qx [m, k] E4M3 codes as uint8, x_scale [m] fp32)."""
    return _rotate_quantize_act("sdnq_rotate_quantize_act_fp8", torch.uint8, x, g, col_scale)


def sdnq_qlinear_forward(x, qw, w_scale, g, lora_a=None, lora_b=None, lora_scale=0.0, out=None,
                         workspace=None):
    """y [m, n] bf16 = dequant(rotq(x) . qw^T) + lora_scale * (x lora_a) lora_b."""
    return _forward("sdnq_qlinear_forward", torch.int8, x, qw, w_scale, g, lora_a, lora_b, lora_scale, out,
                    workspace)


SDNQ_NOALLOC_SCRATCH_BYTES = 64 << 20


def sdnq_qlinear_forward_noalloc(x, qw, w_scale, g, lora_a=None, lora_b=None, lora_scale=0.0, out=None):
    """sdnq_qlinear_forward with the library's fixed device scratch array as the
    workspace (no workspace argument; calls on one device must not overlap)."""
    _need(x, torch.bfloat16, 2, "x")
    _need(qw, torch.int8, 2, "qw")
    _need(w_scale, torch.float32, 1, "w_scale")
    m, k = x.shape
    n = qw.shape[0]
    rank = 0
    if lora_a is not None or lora_b is not None:
        _need(lora_a, torch.bfloat16, 2, "lora_a")
        _need(lora_b, torch.bfloat16, 2, "lora_b")
        rank = lora_a.shape[1]
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _check(lib().sdnq_qlinear_forward_noalloc(_ptr(x), m, k, _ptr(qw), _ptr(w_scale), n, g, _ptr(lora_a),
                                              _ptr(lora_b), rank, float(lora_scale), _ptr(y), _stream(x.device)),
           "sdnq_qlinear_forward_noalloc")
    return y


def sdnq_qlinear_forward_fp8(x, qw, w_scale, g, lora_a=None, lora_b=None, lora_scale=0.0, out=None,
                             workspace=None):
    """The FP8 forward: qw are E4M3 codes (uint8) from sdnq_rotate_quantize_weight_fp8."""
    return _forward("sdnq_qlinear_forward_fp8", torch.uint8, x, qw, w_scale, g, lora_a, lora_b, lora_scale, out,
                    workspace)


def _forward(name, code_dtype, x, qw, w_scale, g, lora_a, lora_b, lora_scale, out, workspace):
    _need(x, torch.bfloat16, 2, "x")
    _need(qw, code_dtype, 2, "qw")
    _need(w_scale, torch.float32, 1, "w_scale")
    m, k = x.shape
    n = qw.shape[0]
    rank = 0
    if lora_a is not None or lora_b is not None:
        _need(lora_a, torch.bfloat16, 2, "lora_a")
        _need(lora_b, torch.bfloat16, 2, "lora_b")
        rank = lora_a.shape[1]
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    nb = sdnq_workspace_bytes(m, n, k, rank, False)
    ws = _workspace(nb, x.device, workspace)
    _check(getattr(lib(), name)(_ptr(x), m, k, _ptr(qw), _ptr(w_scale), n, g, _ptr(lora_a), _ptr(lora_b),
                                rank, float(lora_scale), _ptr(y), _ptr(ws), ws.numel(), _stream(x.device)), name)
    return y


def sdnq_qlinear_forward_quantized(qx, x_scale, qw, w_scale, t=None, lora_b=None, lora_scale=0.0, out=None,
                                   workspace=None):
    """y [m, n] bf16 from pre-quantized activations (qx, x_scale)."""
    return _forward_quantized("sdnq_qlinear_forward_quantized", torch.int8, qx, x_scale, qw, w_scale, t, lora_b,
                              lora_scale, out, workspace)


def sdnq_qlinear_forward_fp8_quantized(qx, x_scale, qw, w_scale, t=None, lora_b=None, lora_scale=0.0, out=None,
                                       workspace=None):
    """The FP8 forward from E4M3 activations (qx, x_scale from sdnq_rotate_quantize_act_fp8)."""
    return _forward_quantized("sdnq_qlinear_forward_fp8_quantized", torch.uint8, qx, x_scale, qw, w_scale, t,
                              lora_b, lora_scale, out, workspace)


def _forward_quantized(name, code_dtype, qx, x_scale, qw, w_scale, t, lora_b, lora_scale, out, workspace):
    _need(qx, code_dtype, 2, "qx")
    _need(x_scale, torch.float32, 1, "x_scale")
    _need(qw, code_dtype, 2, "qw")
    _need(w_scale, torch.float32, 1, "w_scale")
    m, k = qx.shape
    n = qw.shape[0]
    rank = 0
    if t is not None or lora_b is not None:
        _need(t, torch.bfloat16, 2, "t")
        _need(lora_b, torch.bfloat16, 2, "lora_b")
        rank = t.shape[1]
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=qx.device)
    nb = sdnq_workspace_bytes(m, n, k, rank, False)
    ws = _workspace(nb, qx.device, workspace) if rank else workspace
    _check(getattr(lib(), name)(_ptr(qx), _ptr(x_scale), m, k, _ptr(qw), _ptr(w_scale), n, _ptr(t), _ptr(lora_b),
                                rank, float(lora_scale), _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(),
                                _stream(qx.device)), name)
    return y


def sdnq_qlinear_backward_input(dy, qw, w_scale, g, x=None, lora_a=None, lora_b=None, lora_scale=0.0,
                                want_lora_grads=True, workspace=None):
    """Returns (dx [m, k] bf16, grad_a [k, r] or None, grad_b [r, n] or None)."""
    return _backward("sdnq_qlinear_backward_input", torch.int8, dy, qw, w_scale, g, x, lora_a, lora_b, lora_scale,
                     want_lora_grads, workspace)


def sdnq_qlinear_backward_input_fp8(dy, qw, w_scale, g, x=None, lora_a=None, lora_b=None, lora_scale=0.0,
                                    want_lora_grads=True, workspace=None):
    """The FP8 input gradient: qw are E4M3 codes (uint8) from sdnq_rotate_quantize_weight_fp8."""
    return _backward("sdnq_qlinear_backward_input_fp8", torch.uint8, dy, qw, w_scale, g, x, lora_a, lora_b,
                     lora_scale, want_lora_grads, workspace)


def sdnq_transpose_codes(codes):
    """[rows, cols] int8 or uint8 codes -> [cols, rows] (the backward's qw_t)."""
    if not isinstance(codes, torch.Tensor) or codes.dtype not in (torch.int8, torch.uint8) or codes.dim() != 2:
        raise ValueError("codes: expected a 2-d int8 or uint8 tensor")
    if not codes.is_contiguous():
        raise ValueError("codes: must be contiguous")
    rows, cols = codes.shape
    out = torch.empty((cols, rows), dtype=codes.dtype, device=codes.device)
    _check(lib().sdnq_transpose_codes(_ptr(codes), rows, cols, _ptr(out), _stream(codes.device)),
           "sdnq_transpose_codes")
    return out


def sdnq_qlinear_backward_input_wt(dy, qw_t, w_scale, g, x=None, lora_a=None, lora_b=None, lora_scale=0.0,
                                   want_lora_grads=True, workspace=None):
    """sdnq_qlinear_backward_input with qw_t = qw^T [k, n] (sdnq_transpose_codes(qw))."""
    return _backward("sdnq_qlinear_backward_input_wt", torch.int8, dy, qw_t, w_scale, g, x, lora_a, lora_b,
                     lora_scale, want_lora_grads, workspace, transposed=True)


def sdnq_qlinear_backward_input_fp8_wt(dy, qw_t, w_scale, g, x=None, lora_a=None, lora_b=None, lora_scale=0.0,
                                       want_lora_grads=True, workspace=None):
    """The FP8 input gradient with the E4M3 codes given transposed, qw_t [k, n]."""
    return _backward("sdnq_qlinear_backward_input_fp8_wt", torch.uint8, dy, qw_t, w_scale, g, x, lora_a, lora_b,
                     lora_scale, want_lora_grads, workspace, transposed=True)


def _backward(name, code_dtype, dy, qw, w_scale, g, x, lora_a, lora_b, lora_scale, want_lora_grads, workspace,
              transposed=False):
    _need(dy, torch.bfloat16, 2, "dy")
    _need(qw, code_dtype, 2, "qw")
    _need(w_scale, torch.float32, 1, "w_scale")
    m, n = dy.shape
    k = qw.shape[0] if transposed else qw.shape[1]
    rank = 0
    ga = gb = None
    if lora_a is not None or lora_b is not None:
        _need(lora_a, torch.bfloat16, 2, "lora_a")
        _need(lora_b, torch.bfloat16, 2, "lora_b")
        rank = lora_a.shape[1]
        if want_lora_grads and x is not None:
            _need(x, torch.bfloat16, 2, "x")
            ga = torch.empty((k, rank), dtype=torch.bfloat16, device=dy.device)
            gb = torch.empty((rank, n), dtype=torch.bfloat16, device=dy.device)
    dx = torch.empty((m, k), dtype=torch.bfloat16, device=dy.device)
    nb = sdnq_workspace_bytes(m, n, k, rank, True)
    ws = _workspace(nb, dy.device, workspace)
    _check(getattr(lib(), name)(_ptr(dy), m, n, _ptr(qw), _ptr(w_scale), k, g, _ptr(x), _ptr(lora_a), _ptr(lora_b),
                                rank, float(lora_scale), _ptr(dx), _ptr(ga), _ptr(gb), _ptr(ws), ws.numel(),
                                _stream(dy.device)), name)
    return dx, ga, gb


def sdnq_gemm_i8_i32(a, b, b_layout: int = 0, workspace=None):
    """Exact int32 product: b_layout 0: a [m,k] . b[n,k]^T;  1: a [m,k] . b [k,n]."""
    _need(a, torch.int8, 2, "a")
    _need(b, torch.int8, 2, "b")
    m, k = a.shape
    n = b.shape[0] if b_layout == 0 else b.shape[1]
    c = torch.empty((m, n), dtype=torch.int32, device=a.device)
    ws = _workspace(k * n, a.device, workspace) if b_layout == 1 else workspace
    _check(lib().sdnq_gemm_i8_i32(_ptr(a), _ptr(b), m, n, k, b_layout, _ptr(c), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(a.device)), "sdnq_gemm_i8_i32")
    return c


def sdnq_gemm_i8_ceiling(qx, x_scale, qw, w_scale, mode: int, y=None):
    """The forward GEMM kernel with parts of its k loop removed (0: none, 1: global
    loads, 2: also LDS reads, 3: as 2 on loop-index operands); y [m,n] bf16 is
    the forward's only for mode 0."""
    _need(qx, torch.int8, 2, "qx")
    _need(qw, torch.int8, 2, "qw")
    m, k = qx.shape
    n = qw.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=qx.device)
    _check(lib().sdnq_gemm_i8_ceiling(_ptr(qx), _ptr(x_scale), m, k, _ptr(qw), _ptr(w_scale), n, mode, _ptr(y),
                                      _stream(qx.device)), "sdnq_gemm_i8_ceiling")
    return y


def sdnq_gemm_fp8_f32(a, b):
    """fp32-accumulated E4M3 product a [m,k] . b [n,k]^T (codes as uint8)."""
    _need(a, torch.uint8, 2, "a")
    _need(b, torch.uint8, 2, "b")
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k:
        raise ValueError("contraction lengths differ")
    c = torch.empty((m, n), dtype=torch.float32, device=a.device)
    _check(lib().sdnq_gemm_fp8_f32(_ptr(a), _ptr(b), m, n, k, _ptr(c), _stream(a.device)), "sdnq_gemm_fp8_f32")
    return c


def sdnq_weight_grad_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(lib().sdnq_weight_grad_workspace_bytes(m, n, k))


def sdnq_weight_grad_workspace_offset(m: int, n: int, k: int, which: int) -> int:
    return int(lib().sdnq_weight_grad_workspace_offset(m, n, k, which))


def sdnq_qlinear_weight_grad(dy, x, g, out=None, workspace=None):
    """dw [n, k] bf16 = dequant(Q_g(dy^T) . Q_g(x^T)^T): quantized along the tokens."""
    _need(dy, torch.bfloat16, 2, "dy")
    _need(x, torch.bfloat16, 2, "x")
    m, n = dy.shape
    if x.shape[0] != m:
        raise ValueError("dy and x must have the same number of tokens")
    k = x.shape[1]
    dw = out if out is not None else torch.empty((n, k), dtype=torch.bfloat16, device=dy.device)
    ws = _workspace(sdnq_weight_grad_workspace_bytes(m, n, k), dy.device, workspace)
    _check(lib().sdnq_qlinear_weight_grad(_ptr(dy), _ptr(x), m, n, k, g, _ptr(dw), _ptr(ws), ws.numel(),
                                          _stream(dy.device)), "sdnq_qlinear_weight_grad")
    return dw



def sdnq_svd_workspace_bytes(n: int, k: int, rank: int) -> int:
    return int(lib().sdnq_svd_workspace_bytes(n, k, rank))


def sdnq_svd_workspace_q_offset(n: int, k: int, rank: int) -> int:
    return int(lib().sdnq_svd_workspace_q_offset(n, k, rank))


def sdnq_svd_quantize_weight(w, g, omega, steps: int, workspace=None):
    """Low-rank split of w [n, k] (bf16) with the test matrix omega [k, rank] (fp32),
    then rotate + int8 quantization of the residual.  Returns (qw, w_scale, svd_a
    [k, rank] bf16, svd_b [rank, n] bf16); the layer runs as sdnq_qlinear_forward
    with lora_a=svd_a, lora_b=svd_b, lora_scale=1."""
    _need(w, torch.bfloat16, 2, "w")
    _need(omega, torch.float32, 2, "omega")
    n, k = w.shape
    if omega.shape[0] != k:
        raise ValueError("omega must be [k, rank]")
    rank = omega.shape[1]
    dev = w.device
    qw = torch.empty((n, k), dtype=torch.int8, device=dev)
    sw = torch.empty((n,), dtype=torch.float32, device=dev)
    svd_a = torch.empty((k, rank), dtype=torch.bfloat16, device=dev)
    svd_b = torch.empty((rank, n), dtype=torch.bfloat16, device=dev)
    ws = _workspace(sdnq_svd_workspace_bytes(n, k, rank), dev, workspace)
    _check(lib().sdnq_svd_quantize_weight(_ptr(w), n, k, g, rank, steps, _ptr(omega), _ptr(qw), _ptr(sw),
                                          _ptr(svd_a), _ptr(svd_b), _ptr(ws), ws.numel(), _stream(dev)),
           "sdnq_svd_quantize_weight")
    return qw, sw, svd_a, svd_b


def sdnq_attention_workspace_bytes(batch, heads_q, heads_kv, seq_q, seq_k, head_dim) -> int:
    return int(lib().sdnq_attention_workspace_bytes(batch, heads_q, heads_kv, seq_q, seq_k, head_dim))


def sdnq_attention_workspace_offset(batch, heads_q, heads_kv, seq_q, seq_k, head_dim, which: int) -> int:
    return int(lib().sdnq_attention_workspace_offset(batch, heads_q, heads_kv, seq_q, seq_k, head_dim, which))


def sdnq_attention_int8(q, k, v, is_causal: bool = False, scale: float | None = None, smooth_k: bool = True,
                        hadamard_group: int = 256, out=None, workspace=None):
    """Int8-QK^T attention of q [B, Hq, Sq, D], k, v [B, Hkv, Sk, D] (bf16, SDPA's layout)."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, 4, nm)
    bsz, hq, sq, d = q.shape
    hkv, sk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (bsz, hkv, sk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, Sk, D] matching q's batch and head_dim")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    o = out if out is not None else torch.empty_like(q)
    ws = _workspace(sdnq_attention_workspace_bytes(bsz, hq, hkv, sq, sk, d), q.device, workspace)
    _check(lib().sdnq_attention_int8(_ptr(q), _ptr(k), _ptr(v), bsz, hq, hkv, sq, sk, d, int(bool(is_causal)),
                                     float(scale), int(bool(smooth_k)), int(hadamard_group), _ptr(o), _ptr(ws),
                                     ws.numel(), _stream(q.device)), "sdnq_attention_int8")
    return o


# default bound of sdnq_attention_int8's shared-tile wait (the header's SDNQ_ATTENTION_HANDOVER_POLLS)
SDNQ_ATTENTION_HANDOVER_POLLS = 16777216


def sdnq_attention_set_handover_polls(polls: int) -> None:
    """Bound of sdnq_attention_int8's shared-tile wait for later calls, in polls
    (0: give up before the first poll; SDNQ_ATTENTION_HANDOVER_POLLS: the default)."""
    _check(lib().sdnq_attention_set_handover_polls(int(polls)), "sdnq_attention_set_handover_polls")
