"""Host-side tests of the C ABI (no GPU needed).

The library must load and export every function `include/sdnq_hip.h` declares,
and every argument check must return its status before anything is enqueued.
The error-path calls pass fake device addresses that are never dereferenced
when validation rejects the call; they are skipped when a GPU is present, where
the GPU test file repeats them with real buffers.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import hadamard_rotated_int8_amd as h

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdnq_hip.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, LAUNCH = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdnq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("sdnq_rotate_quantize_weight", "sdnq_rotate_quantize_act", "sdnq_qlinear_forward",
              "sdnq_qlinear_backward_input", "sdnq_qlinear_forward_quantized", "sdnq_workspace_bytes",
              "sdnq_status_string", "sdnq_gemm_i8_i32", "sdnq_rotate_quantize_weight_fp8",
              "sdnq_rotate_quantize_act_fp8", "sdnq_qlinear_forward_fp8", "sdnq_qlinear_forward_fp8_quantized",
              "sdnq_gemm_fp8_f32", "sdnq_qlinear_weight_grad", "sdnq_weight_grad_workspace_bytes",
              "sdnq_weight_grad_workspace_offset",
              "sdnq_svd_quantize_weight", "sdnq_svd_workspace_bytes", "sdnq_svd_workspace_q_offset",
              "sdnq_attention_int8", "sdnq_attention_workspace_bytes", "sdnq_attention_workspace_offset",
              "sdnq_qlinear_forward_noalloc", "sdnq_qlinear_backward_input_fp8", "sdnq_transpose_codes",
              "sdnq_qlinear_backward_input_wt", "sdnq_qlinear_backward_input_fp8_wt", "sdnq_gemm_i8_ceiling"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = h.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", h._binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (sdnq_\w+)", out))
    assert set(declared_functions()) <= exported


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings():
    for s in range(5):
        assert len(h.status_string(s)) > 5
    assert "unknown" in h.status_string(99)


def test_workspace_bytes():
    f = h.sdnq_workspace_bytes
    assert f(4096, 3072, 3072) >= 4096 * 3072 + 4096 * 4
    assert f(4096, 3072, 3072, 32) > f(4096, 3072, 3072, 0)
    assert f(16384, 3072, 3072, 64, True) >= 16384 * 3072 + 3072 * 3072
    assert f(0, 16, 16) == 0 or f(0, 16, 16) >= 0
    assert f(-1, 16, 16) == 0
    assert f(16, 0, 16) == 0
    assert f(16, 16, 16, 257) == 0  # rank above 256
    assert f(16, 16, 16, -1) == 0
    # ranks off the multiple of 16 add room for the zero-padded factors
    for bwd in (False, True):
        assert f(4096, 3072, 3072, 17, bwd) > f(4096, 3072, 3072, 32, bwd) > f(4096, 3072, 3072, 16, bwd)
        assert f(4096, 3072, 3072, 1, bwd) > 0 and f(4096, 3072, 3072, 256, bwd) > f(4096, 3072, 3072, 128, bwd)


no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer validation runs only without a GPU")

A = 0x10000   # fake 16-byte-aligned device addresses (never dereferenced on these paths)
B = 0x20000
C = 0x30000
D = 0x40000
W = 0x50000
WS = 1 << 40


def rqa(x=A, m=4, k=256, g=256, cs=None, q=B, s=C):
    return h.lib().sdnq_rotate_quantize_act(x, m, k, g, cs, q, s, None)


def fwd(x=A, m=4, k=256, qw=B, sw=C, n=256, g=256, la=None, lb=None, r=0, y=D, ws=W, wsb=WS):
    return h.lib().sdnq_qlinear_forward(x, m, k, qw, sw, n, g, la, lb, r, 1.0, y, ws, wsb, None)


def bwd(dy=A, m=4, n=256, qw=B, sw=C, k=256, g=256, x=None, la=None, lb=None, r=0, dx=D, ga=None, gb=None,
        ws=W, wsb=WS):
    return h.lib().sdnq_qlinear_backward_input(dy, m, n, qw, sw, k, g, x, la, lb, r, 1.0, dx, ga, gb, ws, wsb, None)


@no_gpu
@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), INVALID), (dict(q=None), INVALID), (dict(s=None), INVALID),
    (dict(m=-1), INVALID), (dict(k=0), INVALID), (dict(k=-16), INVALID),
    (dict(g=32), UNSUPPORTED), (dict(g=512), UNSUPPORTED), (dict(g=0), UNSUPPORTED),
    (dict(k=320, g=256), UNSUPPORTED), (dict(k=200, g=1), UNSUPPORTED),
    (dict(k=133120 + 256, g=256), UNSUPPORTED), (dict(k=133136 + 16, g=1), UNSUPPORTED),  # the int32 bound
    (dict(x=A + 8), INVALID), (dict(q=B + 4), INVALID), (dict(s=C + 2), INVALID),
    (dict(g=1, cs=D + 4), INVALID),
    (dict(m=0), OK),
    (dict(m=0, x=None, q=None, s=None), OK),   # an empty batch may pass NULL row buffers
    (dict(m=0, g=32), UNSUPPORTED),            # ... but is still validated
])
def test_rotate_quantize_act_validation(kw, expect):
    assert rqa(**kw) == expect


@no_gpu
def test_rotate_quantize_weight_validation():
    L = h.lib()
    assert L.sdnq_rotate_quantize_weight(None, 4, 256, 256, B, C, None) == INVALID
    assert L.sdnq_rotate_quantize_weight(A, 4, 256, 100, B, C, None) == UNSUPPORTED
    assert L.sdnq_rotate_quantize_weight(A, 0, 256, 256, B, C, None) == OK


@no_gpu
@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), INVALID), (dict(qw=None), INVALID), (dict(sw=None), INVALID), (dict(y=None), INVALID),
    (dict(m=-3), INVALID), (dict(n=0), INVALID), (dict(k=0), INVALID),
    (dict(n=200), UNSUPPORTED), (dict(k=300, g=1), UNSUPPORTED), (dict(g=7), UNSUPPORTED),
    (dict(k=192, g=128), UNSUPPORTED),
    (dict(la=0x60000, lb=None, r=32), INVALID), (dict(la=None, lb=0x60000, r=32), INVALID),
    (dict(la=0x60000, lb=0x70000, r=257), UNSUPPORTED), (dict(la=0x60000, lb=0x70000, r=0), UNSUPPORTED),
    (dict(la=0x60000, lb=0x70000, r=-5), UNSUPPORTED), (dict(la=0x60008, lb=0x70000, r=32), INVALID),
    (dict(m=0, la=0x60000, lb=0x70000, r=1), OK), (dict(m=0, la=0x60000, lb=0x70000, r=24), OK),
    (dict(m=0, la=0x60000, lb=0x70000, r=200), OK), (dict(m=0, la=0x60000, lb=0x70000, r=256), OK),
    (dict(ws=None), WORKSPACE), (dict(wsb=100), WORKSPACE), (dict(ws=W + 8), WORKSPACE),
    (dict(y=D + 2), INVALID),
    (dict(m=0), OK),
    (dict(m=0, x=None, y=None), OK),
    (dict(m=0, qw=None), INVALID),
])
def test_forward_validation(kw, expect):
    assert fwd(**kw) == expect


@no_gpu
def test_forward_workspace_limit_is_exact():
    need = h.sdnq_workspace_bytes(4, 256, 256, 0, False)
    assert fwd(m=4, wsb=need - 1) == WORKSPACE
    need = h.sdnq_workspace_bytes(4, 256, 256, 32, False)
    assert fwd(m=4, la=0x60000, lb=0x70000, r=32, wsb=need - 1) == WORKSPACE


@no_gpu
@pytest.mark.parametrize("kw,expect", [
    (dict(dy=None), INVALID), (dict(qw=None), INVALID), (dict(dx=None), INVALID),
    (dict(m=-1), INVALID), (dict(n=0), INVALID),
    (dict(g=100), UNSUPPORTED), (dict(n=100), UNSUPPORTED),
    (dict(ga=0x80000), INVALID),                                    # grads without an adapter
    (dict(la=0x60000, lb=0x70000, r=32, ga=0x80000), INVALID),      # grads without x
    (dict(la=0x60000, lb=0x70000, r=32, x=0x90000, gb=0x80004), INVALID),
    (dict(ws=None), WORKSPACE),
    (dict(m=0), OK),
])
def test_backward_validation(kw, expect):
    assert bwd(**kw) == expect


@no_gpu
def test_transposed_weight_entry_points_validate():
    L = h.lib()
    assert L.sdnq_transpose_codes(None, 32, 32, B, None) == INVALID
    assert L.sdnq_transpose_codes(A, 32, 32, None, None) == INVALID
    assert L.sdnq_transpose_codes(A, 0, 32, B, None) == INVALID
    assert L.sdnq_transpose_codes(A, 24, 32, B, None) == UNSUPPORTED
    assert L.sdnq_transpose_codes(A, 32, 133152, B, None) == UNSUPPORTED
    assert L.sdnq_transpose_codes(A + 8, 32, 32, B, None) == INVALID
    for fn in (L.sdnq_qlinear_backward_input_wt, L.sdnq_qlinear_backward_input_fp8_wt):
        # dy, m, n, qw_t, w_scale, k, g, x, lora_a, lora_b, rank, scale, dx, ga, gb, ws, wsb, stream
        assert fn(A, 4, 256, B, C, 256, 7, None, None, None, 0, 0.0, D, None, None, W, WS, None) == UNSUPPORTED
        assert fn(A, 4, 256, None, C, 256, 256, None, None, None, 0, 0.0, D, None, None, W, WS, None) == INVALID
        assert fn(A, 4, 256, B, C, 256, 256, None, None, None, 0, 0.0, D, None, None, None, 0, None) == WORKSPACE
        assert fn(A, 4, 256, B, C, 256, 256, None, A, B, 300, 0.5, D, None, None, W, WS, None) == UNSUPPORTED


@no_gpu
def test_gemm_validation():
    L = h.lib()
    assert L.sdnq_gemm_i8_i32(None, B, 4, 32, 32, 0, C, None, 0, None) == INVALID
    assert L.sdnq_gemm_i8_i32(A, B, 4, 32, 32, 2, C, None, 0, None) == INVALID
    assert L.sdnq_gemm_i8_i32(A, B, 4, 30, 32, 0, C, None, 0, None) == UNSUPPORTED
    assert L.sdnq_gemm_i8_i32(A, B, 4, 32, 32, 1, C, None, 0, None) == WORKSPACE
    assert L.sdnq_gemm_i8_i32(A, B, 0, 32, 32, 0, C, None, 0, None) == OK
    # qx, x_scale, m, k, qw, w_scale, n, mode, y, stream
    assert L.sdnq_gemm_i8_ceiling(A, C, 4, 32, B, C, 32, 4, D, None) == INVALID
    assert L.sdnq_gemm_i8_ceiling(A, C, 4, 32, B, C, 32, -1, D, None) == INVALID
    assert L.sdnq_gemm_i8_ceiling(A, C, 4, 32, None, C, 32, 0, D, None) == INVALID
    assert L.sdnq_gemm_i8_ceiling(A, C, 4, 30, B, C, 32, 0, D, None) == UNSUPPORTED
    assert L.sdnq_gemm_i8_ceiling(A + 8, C, 4, 32, B, C, 32, 0, D, None) == INVALID
    assert L.sdnq_gemm_i8_ceiling(A, C, 0, 32, B, C, 32, 2, D, None) == OK


def test_binding_rejects_wrong_types_before_calling():
    with pytest.raises((TypeError, ValueError)):
        h.sdnq_rotate_quantize_act(torch.zeros(4, 256, dtype=torch.float32), 256)
    with pytest.raises((TypeError, ValueError)):
        h.sdnq_rotate_quantize_act(torch.zeros(4, 256, dtype=torch.bfloat16), 256)  # CPU tensor


@no_gpu
def test_fp8_entry_points_validate_like_the_int8_ones():
    L = h.lib()
    assert L.sdnq_rotate_quantize_act_fp8(A, 4, 256, 32, None, B, C, None) == UNSUPPORTED
    assert L.sdnq_rotate_quantize_act_fp8(A + 8, 4, 256, 256, None, B, C, None) == INVALID
    assert L.sdnq_rotate_quantize_weight_fp8(A, 0, 256, 256, B, C, None) == OK
    assert L.sdnq_qlinear_forward_fp8(A, 4, 256, B, C, 256, 7, None, None, 0, 1.0, D, W, WS, None) == UNSUPPORTED
    assert L.sdnq_qlinear_forward_fp8(A, 4, 256, B, C, 256, 256, None, None, 0, 1.0, D, None, 0, None) == WORKSPACE
    assert L.sdnq_qlinear_forward_fp8_quantized(A, C, 4, 256, B, C, 200, None, None, 0, 1.0, D, None, 0,
                                                None) == UNSUPPORTED
    assert L.sdnq_gemm_fp8_f32(A, B, 4, 30, 32, C, None) == UNSUPPORTED
    assert L.sdnq_gemm_fp8_f32(None, B, 4, 32, 32, C, None) == INVALID
    assert L.sdnq_gemm_fp8_f32(A, B, 0, 32, 32, C, None) == OK


@no_gpu
def test_weight_grad_validation():
    L = h.lib()
    f = lambda m=64, n=256, k=256, g=64, dy=A, x=B, dw=D, ws=W, wsb=WS: L.sdnq_qlinear_weight_grad(
        dy, x, m, n, k, g, dw, ws, wsb, None)
    assert f(m=-1) == INVALID and f(dw=None) == INVALID and f(dy=None) == INVALID
    assert f(m=40) == UNSUPPORTED          # tokens are the contraction: a multiple of 16 ...
    assert f(m=96, g=64) == UNSUPPORTED    # ... and of g
    assert f(n=100) == UNSUPPORTED and f(g=3) == UNSUPPORTED
    assert f(ws=None) == WORKSPACE and f(wsb=100) == WORKSPACE
    assert f(m=64, g=64, wsb=h.sdnq_weight_grad_workspace_bytes(64, 256, 256) - 1) == WORKSPACE
    assert h.sdnq_weight_grad_workspace_bytes(16384, 3072, 3072) >= 16384 * 3072 * 2   # codes of dy^T and x^T
    for m, n, k in ((16384, 3072, 3072), (64, 256, 256), (2048, 2000, 3008)):
        total = h.sdnq_weight_grad_workspace_bytes(m, n, k)
        off = [h.sdnq_weight_grad_workspace_offset(m, n, k, i) for i in range(4)]
        ends = [off[0] + n * m, off[1] + 4 * n, off[2] + k * m, off[3] + 4 * k]
        assert all(o % 256 == 0 for o in off) and off[0] > 0
        assert all(ends[i] <= off[i + 1] for i in range(3)) and ends[3] <= total
    assert h.sdnq_weight_grad_workspace_offset(64, 256, 256, 4) == 0
    assert h.sdnq_weight_grad_workspace_offset(64, 100, 256, 0) == 0



@no_gpu
def test_svd_split_validation():
    L = h.lib()
    E = 0x60000

    def f(w=A, n=256, k=256, g=256, rank=32, steps=8, omega=B, qw=C, sw=D, a=E, b=W, ws=0x70000,
          wsb=None):
        if wsb is None:
            wsb = h.sdnq_svd_workspace_bytes(n, k, rank) or WS
        return L.sdnq_svd_quantize_weight(w, n, k, g, rank, steps, omega, qw, sw, a, b, ws, wsb, None)
    assert f(w=None) == INVALID and f(omega=None) == INVALID and f(b=None) == INVALID
    assert f(n=0) == INVALID and f(k=-16) == INVALID
    assert f(n=100) == UNSUPPORTED and f(g=32) == UNSUPPORTED and f(k=320, g=256) == UNSUPPORTED
    assert f(rank=48) == UNSUPPORTED and f(rank=128) == UNSUPPORTED    # ranks 16, 32, 64 only
    assert f(n=32, k=256, rank=64) == UNSUPPORTED                     # rank above min(n, k)
    assert f(steps=-1) == INVALID and f(steps=65) == INVALID
    assert f(omega=B + 4) == INVALID and f(a=E + 8) == INVALID
    assert f(ws=None) == WORKSPACE
    assert f(wsb=h.sdnq_svd_workspace_bytes(256, 256, 32) - 1) == WORKSPACE


def test_svd_workspace_bytes():
    f = h.sdnq_svd_workspace_bytes
    n, k, r = 3072, 3072, 32
    assert f(n, k, r) >= n * k * 4 + n * k * 2 + n * r * 8   # residual, W^T, Q
    assert h.sdnq_svd_workspace_q_offset(n, k, r) >= n * k * 4
    assert f(n, k, 48) == 0 and f(n, 100, r) == 0 and f(16, 256, 32) == 0


@no_gpu
def test_attention_validation():
    L = h.lib()

    def f(q=A, k=B, v=C, b=1, hq=4, hkv=2, sq=64, sk=64, d=128, causal=0, scale=0.1, smooth=1, g=256, out=D,
          ws=W, wsb=WS):
        return L.sdnq_attention_int8(q, k, v, b, hq, hkv, sq, sk, d, causal, scale, smooth, g, out, ws, wsb, None)
    assert f(q=None) == INVALID and f(out=None) == INVALID and f(b=0) == INVALID and f(sq=0) == INVALID
    assert f(scale=0.0) == INVALID and f(scale=-1.0) == INVALID and f(scale=float("nan")) == INVALID
    assert f(q=A + 8) == INVALID and f(out=D + 2) == INVALID
    assert f(d=96) == UNSUPPORTED and f(d=256) == UNSUPPORTED
    assert f(hkv=3) == UNSUPPORTED and f(sk=40) == UNSUPPORTED and f(g=32) == UNSUPPORTED
    assert f(b=65536, hq=1, hkv=1) == UNSUPPORTED                      # grid z of the V transpose
    assert f(b=4096, hq=16, hkv=16, sq=1 << 16, sk=1 << 16) == UNSUPPORTED  # 2^32 rows
    assert f(ws=None) == WORKSPACE
    assert f(wsb=h.sdnq_attention_workspace_bytes(1, 4, 2, 64, 64, 128) - 1) == WORKSPACE


def test_attention_workspace():
    f = h.sdnq_attention_workspace_bytes
    b, hq, hkv, s, d = 1, 24, 24, 4608, 128
    n = f(b, hq, hkv, s, s, d)
    assert n >= b * hq * s * d + b * hkv * s * d + b * hkv * s * d * 2   # q and k codes, V^T
    offs = [h.sdnq_attention_workspace_offset(b, hq, hkv, s, s, d, i) for i in range(6)]
    assert offs == sorted(offs) and offs[0] == 0 and offs[1] >= b * hq * s * d and all(o % 256 == 0 for o in offs)
    assert offs[5] + 4 <= n                                              # the status word
    assert f(1, 4, 3, 64, 64, 128) == 0 and f(1, 4, 2, 64, 40, 128) == 0 and f(1, 4, 2, 64, 64, 80) == 0
    assert h.sdnq_attention_workspace_offset(1, 4, 2, 64, 64, 128, 6) == 0


def test_product_path_fails_loudly_without_the_library():
    """With the HIP library absent the entry points raise; nothing falls back to
    a CPU computation (a fresh interpreter, so no library is loaded yet)."""
    code = (
        "import hadamard_rotated_int8_amd._binding as B\n"
        "B.LIB_PATH = '/nonexistent/libsdnq_hip.so'\n"
        "import hadamard_rotated_int8_amd as h, torch\n"
        "try:\n"
        "    h.sdnq_workspace_bytes(64, 512, 512)\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    print('no error')\n")
    out = subprocess.run(["python3", "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert "raised:" in out.stdout and "is missing" in out.stdout, out.stdout + out.stderr


def test_host_tensors_are_rejected():
    """Host (CPU) tensors are refused before any call: the library computes on the
    GPU only, and there is no host path to fall back to."""
    w = torch.zeros(512, 512, dtype=torch.bfloat16)
    with pytest.raises((ValueError, RuntimeError)):
        h.sdnq_rotate_quantize_weight(w, 256)


@no_gpu
def test_noalloc_forward_validation():
    """Checked before any HIP call: arguments forward() rejects, and a call larger
    than the fixed scratch array."""
    L = h.lib()

    def f(x=A, m=4, k=256, qw=B, sw=C, n=256, g=256, la=None, lb=None, r=0, y=D):
        return L.sdnq_qlinear_forward_noalloc(x, m, k, qw, sw, n, g, la, lb, r, 1.0, y, None)
    assert f(m=-1) == INVALID and f(x=None) == INVALID and f(k=0) == INVALID
    assert f(g=32) == UNSUPPORTED and f(n=200) == UNSUPPORTED
    assert f(la=0x60000, lb=0x70000, r=300) == UNSUPPORTED
    assert f(m=8192, k=8192 + 256) == WORKSPACE                       # more than 64 MiB of codes
    assert h.SDNQ_NOALLOC_SCRATCH_BYTES == 64 << 20
    assert f"((size_t)64 << 20)" in open(HEADER).read()


def test_handover_bound_constant_matches_the_header():
    text = open(os.path.join(ROOT, "include", "sdnq_hip.h")).read()
    m = re.search(r"#define SDNQ_ATTENTION_HANDOVER_POLLS (\d+)u", text)
    assert m and int(m.group(1)) == h.SDNQ_ATTENTION_HANDOVER_POLLS
