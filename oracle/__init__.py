"""CPU oracle for the Hadamard-rotated INT8 quantized linear layer.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the GPU library and its
Python binding never do.  It shares no code with the GPU path.

The arithmetic lives in ``sdnq_oracle.c`` (plain C, one binary32 operation per
step, see the header there for the passages each step follows).  This module only
builds that file with gcc and marshals numpy arrays in and out of it.

Bit patterns: bf16 tensors travel as ``numpy.uint16`` arrays holding the raw
bfloat16 bits.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sdnq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsdnq_oracle.so")
# A different build of the oracle (used by the mutation test, which compiles
# deliberately broken copies and checks that the pins reject them).
_LIB_OVERRIDE = os.environ.get("SDNQ_ORACLE_LIB")

# gcc flags: no contraction into FMA, no fast-math, generic x86-64 code so the
# library also runs on a host with a different CPU model.
_CFLAGS = ["-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]

_lib = None

OK, ERR_ARG, ERR_OVERFLOW = 0, 1, 2


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle shared library (in place by default) and return its path."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", *_CFLAGS, src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int
    lib.oracle_num_threads.restype = i32
    lib.oracle_set_num_threads.argtypes = [i32]
    lib.oracle_fwht_unnormalized.argtypes = [p, i64, i32]
    lib.oracle_norm_const.argtypes = [i32]
    lib.oracle_norm_const.restype = ctypes.c_float
    lib.oracle_bf16_from_f64.argtypes = [p, i64, p]
    lib.oracle_f32_from_bf16.argtypes = [p, i64, p]
    lib.oracle_rotate.argtypes = [p, i64, i64, i32, p, p]
    lib.oracle_rotate_quantize.argtypes = [p, i64, i64, i32, p, p, p]
    lib.oracle_rotate_quantize_f32.argtypes = [p, i64, i64, i32, p, p]
    lib.oracle_gemm_i8.argtypes = [p, p, i64, i64, i64, i32, p]
    lib.oracle_qlinear_forward.argtypes = [p, i64, i64, p, p, i64, i32, p, p, i32, ctypes.c_double,
                                           p, p, p, p, p]
    lib.oracle_qlinear_backward_input.argtypes = [p, i64, i64, p, p, i64, i32, p, p, p, i32,
                                                  ctypes.c_double, p, p, p, p, p, p, p]
    lib.oracle_e4m3_encode.argtypes = [p, i64, p]
    lib.oracle_e4m3_decode.argtypes = [p, i64, p]
    lib.oracle_rotate_quantize_fp8.argtypes = [p, i64, i64, i32, p, p, p]
    lib.oracle_gemm_fp8.argtypes = [p, p, i64, i64, i64, p]
    lib.oracle_qlinear_forward_fp8.argtypes = [p, i64, i64, p, p, i64, i32, p, p, i32, ctypes.c_double,
                                               p, p, p, p, p]
    lib.oracle_qlinear_backward_input_fp8.argtypes = [p, i64, i64, p, p, i64, i32, p, p, i32, ctypes.c_double,
                                                      p, p, p, p, p]
    for name in ("oracle_fwht_unnormalized", "oracle_rotate", "oracle_rotate_quantize", "oracle_rotate_quantize_f32",
                 "oracle_gemm_i8", "oracle_qlinear_forward", "oracle_qlinear_backward_input",
                 "oracle_rotate_quantize_fp8", "oracle_gemm_fp8", "oracle_qlinear_forward_fp8",
                 "oracle_qlinear_backward_input_fp8"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str) -> None:
    if rc == ERR_OVERFLOW:
        raise OverflowError(f"{what}: an integer accumulator left the int32 range")
    if rc != OK:
        raise ValueError(f"{what}: invalid arguments (code {rc})")


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def fwht_unnormalized(v: np.ndarray, g: int) -> np.ndarray:
    """Unnormalized butterfly H_g applied to every consecutive block of g values
    along the last axis (binary32, in the oracle's fixed stage order)."""
    a = _c(v, np.float32).copy()
    if a.shape[-1] % g:
        raise ValueError("last axis must be a multiple of g")
    _check(_load().oracle_fwht_unnormalized(_ptr(a), a.size // g, g), "fwht")
    return a


def norm_const(g: int) -> np.float32:
    return np.float32(_load().oracle_norm_const(g))


def bf16_from_f64(v) -> np.ndarray:
    a = _c(v, np.float64)
    out = np.empty(a.shape, np.uint16)
    _load().oracle_bf16_from_f64(_ptr(a), a.size, _ptr(out))
    return out


def f32_from_bf16(h) -> np.ndarray:
    a = _c(h, np.uint16)
    out = np.empty(a.shape, np.float32)
    _load().oracle_f32_from_bf16(_ptr(a), a.size, _ptr(out))
    return out


def rotate(x_bf16: np.ndarray, g: int, col_scale: np.ndarray | None = None) -> np.ndarray:
    """Normalized block rotation of each row (binary32 result), no quantization."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    cs = None if col_scale is None else _c(col_scale, np.float32)
    y = np.empty((rows, cols), np.float32)
    _check(_load().oracle_rotate(_ptr(x), rows, cols, g, _ptr(cs), _ptr(y)), "rotate")
    return y


def rotate_quantize(x_bf16: np.ndarray, g: int, col_scale: np.ndarray | None = None):
    """Rotate then quantize each row: returns (codes int8 [rows, cols], scales f32 [rows])."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    cs = None if col_scale is None else _c(col_scale, np.float32)
    q = np.empty((rows, cols), np.int8)
    s = np.empty((rows,), np.float32)
    _check(_load().oracle_rotate_quantize(_ptr(x), rows, cols, g, _ptr(cs), _ptr(q), _ptr(s)),
           "rotate_quantize")
    return q, s


def rotate_quantize_f32(x_f32: np.ndarray, g: int):
    """Rotate then quantize rows given as binary32 values (no bf16 decode, no column
    scale): returns (codes int8 [rows, cols], scales f32 [rows])."""
    x = _c(x_f32, np.float32)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty((rows,), np.float32)
    _check(_load().oracle_rotate_quantize_f32(_ptr(x), rows, cols, g, _ptr(q), _ptr(s)), "rotate_quantize_f32")
    return q, s


def gemm_i8(a: np.ndarray, b: np.ndarray, b_layout: int = 0) -> np.ndarray:
    """Exact integer matmul.  b_layout 0: b is [n, k] (C = A B^T); 1: b is [k, n] (C = A B)."""
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    m, k = a.shape
    n = b.shape[0] if b_layout == 0 else b.shape[1]
    kb = b.shape[1] if b_layout == 0 else b.shape[0]
    if kb != k:
        raise ValueError("contraction lengths differ")
    c = np.empty((m, n), np.int32)
    _check(_load().oracle_gemm_i8(_ptr(a), _ptr(b), m, n, k, b_layout, _ptr(c)), "gemm_i8")
    return c


def qlinear_forward(x: np.ndarray, qw: np.ndarray, sw: np.ndarray, g: int,
                    lora_a: np.ndarray | None = None, lora_b: np.ndarray | None = None,
                    lora_scale: float = 0.0, intermediates: bool = True) -> dict:
    """Forward of the layer for every row of x.  Returns y (bf16 bits) and, with
    ``intermediates``, qx, sx, acc (int32) and base (fp32 dequantized product)."""
    x = _c(x, np.uint16)
    qw = _c(qw, np.int8)
    sw = _c(sw, np.float32)
    m, k = x.shape
    n = qw.shape[0]
    if qw.shape[1] != k or sw.shape != (n,):
        raise ValueError("shape mismatch")
    la = None if lora_a is None else _c(lora_a, np.uint16)
    lb = None if lora_b is None else _c(lora_b, np.uint16)
    rank = 0 if la is None else la.shape[1]
    out = {"y": np.empty((m, n), np.uint16)}
    if intermediates:
        out.update(qx=np.empty((m, k), np.int8), sx=np.empty((m,), np.float32),
                   acc=np.empty((m, n), np.int32), base=np.empty((m, n), np.float32))
    rc = _load().oracle_qlinear_forward(
        _ptr(x), m, k, _ptr(qw), _ptr(sw), n, g, _ptr(la), _ptr(lb), rank, float(lora_scale),
        _ptr(out["y"]), _ptr(out.get("qx")), _ptr(out.get("sx")), _ptr(out.get("acc")),
        _ptr(out.get("base")))
    _check(rc, "qlinear_forward")
    return out


def qlinear_backward_input(dy: np.ndarray, qw: np.ndarray, sw: np.ndarray, g: int,
                           x: np.ndarray | None = None, lora_a: np.ndarray | None = None,
                           lora_b: np.ndarray | None = None, lora_scale: float = 0.0,
                           want_grads: bool = True, intermediates: bool = True,
                           want_dx: bool = True) -> dict:
    """Input gradient through the int8 weight (+ LoRA input gradient and, when x is
    given and ``want_grads``, the LoRA weight gradients).  ``want_dx=False`` computes
    the LoRA weight gradients only."""
    dy = _c(dy, np.uint16)
    qw = _c(qw, np.int8)
    sw = _c(sw, np.float32)
    m, n = dy.shape
    k = qw.shape[1]
    if qw.shape[0] != n or sw.shape != (n,):
        raise ValueError("shape mismatch")
    la = None if lora_a is None else _c(lora_a, np.uint16)
    lb = None if lora_b is None else _c(lora_b, np.uint16)
    rank = 0 if la is None else la.shape[1]
    xx = None if x is None else _c(x, np.uint16)
    out = {"dx": np.empty((m, k), np.uint16) if want_dx else None}
    if not want_dx:
        intermediates = False
    if la is not None and want_grads and xx is not None:
        out["grad_a"] = np.empty((k, rank), np.uint16)
        out["grad_b"] = np.empty((rank, n), np.uint16)
    if intermediates:
        out.update(qdy=np.empty((m, n), np.int8), sdy=np.empty((m,), np.float32),
                   acc=np.empty((m, k), np.int32), dxbase=np.empty((m, k), np.float32))
    rc = _load().oracle_qlinear_backward_input(
        _ptr(dy), m, n, _ptr(qw), _ptr(sw), k, g, _ptr(xx), _ptr(la), _ptr(lb), rank,
        float(lora_scale), _ptr(out["dx"]), _ptr(out.get("grad_a")), _ptr(out.get("grad_b")),
        _ptr(out.get("qdy")), _ptr(out.get("sdy")), _ptr(out.get("acc")), _ptr(out.get("dxbase")))
    _check(rc, "qlinear_backward_input")
    return out


# ------------------------------------------------------------- FP8 (E4M3) --

def e4m3_encode(v) -> np.ndarray:
    """E4M3 codes (uint8) of binary32 values with |v| <= 448, round half to even."""
    a = _c(v, np.float32)
    out = np.empty(a.shape, np.uint8)
    _load().oracle_e4m3_encode(_ptr(a), a.size, _ptr(out))
    return out


def e4m3_decode(c) -> np.ndarray:
    """Values (fp64) of E4M3 codes (NaN codes excluded)."""
    a = _c(c, np.uint8)
    out = np.empty(a.shape, np.float64)
    _load().oracle_e4m3_decode(_ptr(a), a.size, _ptr(out))
    return out


def rotate_quantize_fp8(x_bf16: np.ndarray, g: int, col_scale: np.ndarray | None = None):
    """Rotate then quantize each row to E4M3: returns (codes uint8 [rows, cols], scales f32 [rows])."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    cs = None if col_scale is None else _c(col_scale, np.float32)
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows,), np.float32)
    _check(_load().oracle_rotate_quantize_fp8(_ptr(x), rows, cols, g, _ptr(cs), _ptr(q), _ptr(s)),
           "rotate_quantize_fp8")
    return q, s


def gemm_fp8(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Exact E4M3 matmul C = dec(A) dec(B)^T in fp64 (a [m, k], b [n, k] uint8 codes)."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k:
        raise ValueError("contraction lengths differ")
    c = np.empty((m, n), np.float64)
    _check(_load().oracle_gemm_fp8(_ptr(a), _ptr(b), m, n, k, _ptr(c)), "gemm_fp8")
    return c


def qlinear_forward_fp8(x: np.ndarray, qw: np.ndarray, sw: np.ndarray, g: int,
                        lora_a: np.ndarray | None = None, lora_b: np.ndarray | None = None,
                        lora_scale: float = 0.0, intermediates: bool = True) -> dict:
    """FP8 forward of the layer for every row of x.  Returns y (bf16 bits) and, with
    ``intermediates``, qx (E4M3 codes), sx, acc (exact fp64) and base (fp32)."""
    x = _c(x, np.uint16)
    qw = _c(qw, np.uint8)
    sw = _c(sw, np.float32)
    m, k = x.shape
    n = qw.shape[0]
    if qw.shape[1] != k or sw.shape != (n,):
        raise ValueError("shape mismatch")
    la = None if lora_a is None else _c(lora_a, np.uint16)
    lb = None if lora_b is None else _c(lora_b, np.uint16)
    rank = 0 if la is None else la.shape[1]
    out = {"y": np.empty((m, n), np.uint16)}
    if intermediates:
        out.update(qx=np.empty((m, k), np.uint8), sx=np.empty((m,), np.float32),
                   acc=np.empty((m, n), np.float64), base=np.empty((m, n), np.float32))
    rc = _load().oracle_qlinear_forward_fp8(
        _ptr(x), m, k, _ptr(qw), _ptr(sw), n, g, _ptr(la), _ptr(lb), rank, float(lora_scale),
        _ptr(out["y"]), _ptr(out.get("qx")), _ptr(out.get("sx")), _ptr(out.get("acc")),
        _ptr(out.get("base")))
    _check(rc, "qlinear_forward_fp8")
    return out


def qlinear_backward_input_fp8(dy: np.ndarray, qw: np.ndarray, sw: np.ndarray, g: int,
                               x: np.ndarray | None = None, lora_a: np.ndarray | None = None,
                               lora_b: np.ndarray | None = None, lora_scale: float = 0.0,
                               want_grads: bool = True, intermediates: bool = True) -> dict:
    """FP8 input gradient through the E4M3 weight codes qw [n, k] (+ the LoRA
    input-gradient term and, when x is given and ``want_grads``, the LoRA weight
    gradients, which do not involve the quantized weight).  With
    ``intermediates``: qdy (E4M3 codes), sdy, acc (exact fp64) and dxbase."""
    dy = _c(dy, np.uint16)
    qw = _c(qw, np.uint8)
    sw = _c(sw, np.float32)
    m, n = dy.shape
    k = qw.shape[1]
    if qw.shape[0] != n or sw.shape != (n,):
        raise ValueError("shape mismatch")
    la = None if lora_a is None else _c(lora_a, np.uint16)
    lb = None if lora_b is None else _c(lora_b, np.uint16)
    rank = 0 if la is None else la.shape[1]
    out = {"dx": np.empty((m, k), np.uint16)}
    if intermediates:
        out.update(qdy=np.empty((m, n), np.uint8), sdy=np.empty((m,), np.float32),
                   acc=np.empty((m, k), np.float64), dxbase=np.empty((m, k), np.float32))
    rc = _load().oracle_qlinear_backward_input_fp8(
        _ptr(dy), m, n, _ptr(qw), _ptr(sw), k, g, _ptr(la), _ptr(lb), rank, float(lora_scale),
        _ptr(out["dx"]), _ptr(out.get("qdy")), _ptr(out.get("sdy")), _ptr(out.get("acc")), _ptr(out.get("dxbase")))
    _check(rc, "qlinear_backward_input_fp8")
    if la is not None and want_grads and x is not None:
        grads = qlinear_backward_input(dy, np.zeros((n, k), np.int8), sw, g, x, la, lb, lora_scale, want_dx=False)
        out["grad_a"], out["grad_b"] = grads["grad_a"], grads["grad_b"]
    return out


# -------------------------------------------------------- weight gradient --

def qlinear_weight_grad(dy: np.ndarray, x: np.ndarray, g: int, intermediates: bool = False) -> dict:
    """Weight gradient through the quantized matmul, contracting over the tokens:
    q_dy, s_dy = rotate (block g along the tokens) + per-feature quantization of
    the rows of dy^T [n, m]; q_x, s_x likewise for x^T [k, m]; then
    dw[n, k] = bf16(fl32(fl32(sum_t q_dy q_x) * fl32(s_dy[n] * s_x[k]))), i.e. the
    forward's steps with dy^T as the activations and x^T as the weight."""
    dyt = np.ascontiguousarray(_c(dy, np.uint16).T)
    xt = np.ascontiguousarray(_c(x, np.uint16).T)
    qx, sx = rotate_quantize(xt, g)
    out = qlinear_forward(dyt, qx, sx, g, intermediates=intermediates)
    res = {"dw": out["y"]}
    if intermediates:
        res.update(q_dy=out["qx"], s_dy=out["sx"], q_x=qx, s_x=sx, acc=out["acc"])
    return res



# ------------------------------------------------------ low-rank (SVD) split --
#
# "SDNQ: SD.Next Quantization Engine" lists SVD quantization next to the Hadamard
# rotation for quantized weights and the quantized matmul, and its SDNQConfig
# example carries use_svd, svd_rank=32 and svd_steps=8.  The SD.Next dev commit
# log ("automatic/commits/branch/dev/cli") calls the factorization a seeded SVD
# truncation and notes that a weight quantized with it dequantizes off the plain
# integer grid: the stored weight is integer codes plus low-rank factors.  The
# pages do not print the algorithm; the reading taken here is the randomized
# range finder with subspace iteration (Halko, Martinsson and Tropp, 2011,
# algorithms 4.1 and 4.4):
#   Q = orth(W omega)                        omega [K, r] Gaussian, seeded, an input
#   repeat svd_steps times: Z = orth(W^T Q); Q = orth(W Z)
#   low-rank part L = Q (Q^T W);  factors svd_a = W^T Q [K, r], svd_b = Q^T [r, N]
#   both rounded to bf16; residual R = fl32(W - svd_b^T svd_a^T) with the rounded
#   factors (the quantizer sees exactly what the factors leave out)
#   the residual is rotated and quantized like any weight (rotate_quantize_f32)
#   at run time y = dequant(q(xH) q(RH)^T) + (x svd_a) svd_b: the LoRA side term
#   with scale 1 on the unrotated x.
# orth() is a reduced QR (numpy's Householder QR): only the span of Q matters,
# so any orthonormal basis of the same span gives the same L.

def _orth(y: np.ndarray) -> np.ndarray:
    q, _ = np.linalg.qr(y, mode="reduced")
    return q


def svd_lowrank_split(w_bf16: np.ndarray, omega: np.ndarray, steps: int) -> dict:
    """Low-rank split of a bf16 weight [N, K] with rank r = omega.shape[1] and
    `steps` subspace iterations, in fp64.  Returns q [N, r] (fp64, orthonormal),
    svd_a [K, r] and svd_b [r, N] (bf16 bits) and the residual [N, K] (binary32)."""
    w = f32_from_bf16(w_bf16).astype(np.float64)
    om = np.asarray(omega, np.float64)
    if om.ndim != 2 or om.shape[0] != w.shape[1] or not 1 <= om.shape[1] <= min(w.shape):
        raise ValueError("omega must be [K, r] with 1 <= r <= min(N, K)")
    if steps < 0:
        raise ValueError("steps must be >= 0")
    q = _orth(w @ om)
    for _ in range(steps):
        z = _orth(w.T @ q)
        q = _orth(w @ z)
    a_bits = bf16_from_f64(w.T @ q)
    b_bits = bf16_from_f64(np.ascontiguousarray(q.T))
    lr = f32_from_bf16(b_bits).astype(np.float64).T @ f32_from_bf16(a_bits).astype(np.float64).T
    return {"q": q, "svd_a": a_bits, "svd_b": b_bits, "residual": (w - lr).astype(np.float32)}


def svd_quantize_weight(w_bf16: np.ndarray, g: int, omega: np.ndarray, steps: int) -> dict:
    """Low-rank split, then rotate + row-wise int8 quantization of the residual.
    Returns the split's fields plus qw [N, K] int8 and sw [N] f32."""
    out = svd_lowrank_split(w_bf16, omega, steps)
    out["qw"], out["sw"] = rotate_quantize_f32(out["residual"], g)
    return out


# ---------------------------------------------------- int8 attention (QK^T) --
#
# "SDNQ: SD.Next Quantization Engine", the SDPA-replacement example: the
# attention takes query/key/value in SDPA's layout with is_causal, scale and
# enable_gqa, runs Q K^T as an int8 quantized matmul (matmul_dtype "int8"),
# keeps P V unquantized (pv_matmul_dtype "disabled"), smooths K (smooth_k), can
# rotate Q and K with a Hadamard block (use_hadamard, hadamard_group_size 256),
# and quantizes in fp32 (quantize_fp32).  Readings (the pages give the options,
# not the arithmetic):
#   * q [B, Hq, Sq, D], k and v [B, Hkv, Sk, D]; query head h reads key/value
#     head h // (Hq / Hkv) (grouped-query attention);
#   * smooth_k subtracts from K its mean over the key tokens, per batch, head and
#     channel (the softmax of each query row is unchanged by a shift common to
#     all keys); the mean is the exact rational mean of the bf16 keys rounded
#     once to binary32 (to nearest, ties to even), so it does not depend on any
#     summation order; K' = fl32(k - mean);
#   * the rotation block along the head dimension is min(g, D) (g <= 1: none),
#     with the butterfly, normalization and per-row int8 quantizer of the
#     linear layer, one scale per token of Q and of K;
#   * scores = fp64(int Q K^T) * s_q[i] * s_k[j] * scale, scale = 1/sqrt(D) by
#     default; is_causal masks keys j > i (top-left aligned, as SDPA);
#   * softmax and P V in fp64 on the bf16 values of v, one rounding to bf16.

def _f32_nearest(num: int, den: int) -> float:
    """The binary32 value nearest to the rational num / den (den > 0), ties to
    even, as a Python float (exact: at most 24 significant bits).  The value must
    lie within the binary32 range, which a mean of bf16 values always does."""
    if num == 0:
        return 0.0
    neg, num = num < 0, abs(num)
    # e = floor(log2(num / den)): start from the bit lengths, correct by one
    e = num.bit_length() - den.bit_length()
    if (num << max(0, -e)) < (den << max(0, e)):
        e -= 1
    # binary32 keeps 24 significant bits down to 2^-126, then a fixed quantum 2^-149
    qexp = max(e, -126) - 23
    n, d = (num, den << qexp) if qexp >= 0 else (num << -qexp, den)
    qi, r = divmod(n, d)
    if 2 * r > d or (2 * r == d and qi & 1):
        qi += 1
    v = math.ldexp(qi, qexp)
    return -v if neg else v


def attention_k_mean(k_bf16: np.ndarray) -> np.ndarray:
    """Per (batch, head, channel) mean of k [B, H, S, D] over the tokens as
    binary32 [B, H, D]: the exact rational mean, rounded once to nearest (ties to
    even).

    A bf16 value with exponent field E and mantissa field m is
    (-1)^sign * sig * 2^(max(E, 1) - 134), with sig = m for E = 0 (subnormal) and
    128 + m otherwise, so 2^133 times any key is an integer.  The integer sum is
    formed exactly: the signed sigs are totalled per exponent (at most 255 * S
    per bucket, exact in binary64 for S <= 2^20), then the buckets are shifted
    into place and added as Python integers."""
    kb = np.ascontiguousarray(k_bf16, np.uint16)
    b, hh, s, d = kb.shape
    e = ((kb >> 7) & 0xFF).astype(np.int64)
    if np.any(e == 0xFF):
        raise ValueError("keys must be finite")
    sig = (kb & 0x7F).astype(np.int64) + np.where(e > 0, 128, 0)
    sig = np.where(kb & 0x8000, -sig, sig)
    pos = np.maximum(e, 1) - 1                               # key = sig * 2^(pos - 133)
    chan = np.arange(b * hh * d).reshape(b, hh, 1, d)        # one bucket row per (batch, head, channel)
    idx = (np.broadcast_to(chan, kb.shape) * 254 + pos).ravel()
    buckets = np.bincount(idx, weights=sig.ravel().astype(np.float64), minlength=b * hh * d * 254)
    buckets = buckets.reshape(b * hh * d, 254).astype(np.int64)
    out = np.empty(b * hh * d, np.float32)
    den = s << 133
    for c in range(b * hh * d):
        nz = np.nonzero(buckets[c])[0]
        total = sum(int(buckets[c, p]) << int(p) for p in nz)
        out[c] = np.float32(_f32_nearest(total, den))
    return out.reshape(b, hh, d)


def attention_block(g: int, d: int) -> int:
    return 1 if g <= 1 else min(g, d)


def attention_prep(x_bf16: np.ndarray, g: int, offset: np.ndarray | None = None):
    """Codes int8 [B, H, S, D] and scales f32 [B, H, S] of each token row, rotated
    with block min(g, D); offset [B, H, D] (binary32) is subtracted first."""
    b, hh, s, d = x_bf16.shape
    blk = attention_block(g, d)
    if offset is None:
        q, sc = rotate_quantize(np.ascontiguousarray(x_bf16).reshape(-1, d), blk)
    else:
        xf = f32_from_bf16(x_bf16) - np.asarray(offset, np.float32)[:, :, None, :]
        q, sc = rotate_quantize_f32(xf.astype(np.float32).reshape(-1, d), blk)
    return q.reshape(b, hh, s, d), sc.reshape(b, hh, s)


def attention_int8(q: np.ndarray, k: np.ndarray, v: np.ndarray, is_causal: bool = False,
                   scale: float | None = None, smooth_k: bool = True, g: int = 256,
                   intermediates: bool = False, q_rows: np.ndarray | None = None) -> dict:
    """Int8-QK^T attention of bf16 q [B, Hq, Sq, D], k, v [B, Hkv, Sk, D]:
    returns out (bf16 bits [B, Hq, Sq, D]) and, with intermediates, the codes,
    scales, K mean and the fp64 output before rounding.  q_rows (query token
    indices) restricts the work and the outputs to those rows of every head."""
    bsz, hq, sq, d = q.shape
    hkv, sk = k.shape[1], k.shape[2]
    if k.shape != (bsz, hkv, sk, d) or v.shape != k.shape or hq % hkv != 0:
        raise ValueError("q [B, Hq, Sq, D], k and v [B, Hkv, Sk, D] with Hq % Hkv == 0")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(sq) if q_rows is None else np.asarray(q_rows, np.int64)
    q = np.ascontiguousarray(np.asarray(q)[:, :, rows, :])
    sq = len(rows)
    qc, qs = attention_prep(q, g)
    mean = attention_k_mean(k) if smooth_k else None
    kc, ks = attention_prep(k, g, mean)
    vf = f32_from_bf16(v).astype(np.float64)
    rep = hq // hkv
    o = np.empty((bsz, hq, sq, d), np.float64)
    mask = (np.arange(sk)[None, :] > rows[:, None]) if is_causal else None
    for b in range(bsz):
        for h in range(hq):
            hk = h // rep
            acc = qc[b, h].astype(np.int64) @ kc[b, hk].astype(np.int64).T
            s = acc.astype(np.float64) * (qs[b, h].astype(np.float64)[:, None] *
                                          ks[b, hk].astype(np.float64)[None, :]) * scale
            if mask is not None:
                s[mask] = -np.inf
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            o[b, h] = (p @ vf[b, hk]) / p.sum(axis=1, keepdims=True)
    res = {"out": bf16_from_f64(o)}
    if intermediates:
        res.update(q_codes=qc, q_scales=qs, k_codes=kc, k_scales=ks, k_mean=mean, o=o)
    return res
