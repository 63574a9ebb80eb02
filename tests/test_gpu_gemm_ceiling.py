"""The GEMM ceiling diagnostic (sdnq_gemm_i8_ceiling) through the C ABI.

Mode 0 launches the forward's own kernel, so its output must equal
sdnq_qlinear_forward_quantized's bit for bit; modes 1 to 3 run the same kernel
with parts of the k loop removed and must complete with finite outputs (their
values are not a product).  Shapes: one tile, ragged tiles of every tile width,
and the MLP step's two GEMMs, which the benchmark times in every mode.
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_int8_amd as h

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def operands(m, n, k, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    qx = torch.randint(-127, 128, (m, k), dtype=torch.int8, generator=g).to(DEV)
    qw = torch.randint(-127, 128, (n, k), dtype=torch.int8, generator=g).to(DEV)
    sx = (torch.rand(m, generator=g) * 1e-3 + 1e-4).to(DEV)
    sw = (torch.rand(n, generator=g) * 1e-3 + 1e-4).to(DEV)
    return qx, sx, qw, sw


# (m, n, k): one row of 256 x 192 tiles; 256 x 192 tiles with ragged m and k;
# 256 x 320 tiles with ragged last row and column tiles; the MLP up projection
# (256 x 320 tiles) and down projection (256 x 256 tiles)
SHAPES = [(256, 256, 256), (600, 3072, 1040), (4000, 4992, 384), (4096, 10240, 3840), (4096, 3840, 10240)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_mode0_is_the_forward_kernel(m, n, k):
    say(f"ceiling mode 0 m={m} n={n} k={k}")
    qx, sx, qw, sw = operands(m, n, k, seed=m + n + k)
    ref = h.sdnq_qlinear_forward_quantized(qx, sx, qw, sw)
    got = h.sdnq_gemm_i8_ceiling(qx, sx, qw, sw, 0)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("mode", [1, 2, 3])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_reduced_modes_complete(m, n, k, mode):
    say(f"ceiling mode {mode} m={m} n={n} k={k}")
    qx, sx, qw, sw = operands(m, n, k, seed=m + n + k)
    y = h.sdnq_gemm_i8_ceiling(qx, sx, qw, sw, mode)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y.float()).all())


def test_zero_tokens_is_a_no_op():
    qx, sx, qw, sw = operands(256, 256, 256, seed=1)
    y = h.sdnq_gemm_i8_ceiling(qx[:0], sx[:0], qw, sw, 2)
    assert y.shape == (0, 256)
