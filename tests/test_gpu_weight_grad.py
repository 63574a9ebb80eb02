"""GPU parity of the weight gradient through the quantized matmul (full
fine-tuning), through the C ABI, against the CPU oracle: the per-feature
rotate+quantize along the tokens and the exact int32 GEMM with the fp32
dequantization are all deterministic, so dW is compared bit for bit."""
import numpy as np
import pytest
import torch

import hadamard_rotated_int8_amd as h
import oracle
from hadamard_rotated_int8_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def d_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def h_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    h.lib()
    yield
    torch.cuda.synchronize()


def inputs(m, n, k, seed):
    rng = np.random.default_rng(seed)
    dy = synth.to_bf16_bits((rng.standard_normal((m, n)) * 1e-3).astype(np.float32))
    x = synth.to_bf16_bits(synth.outlier_activations(rng, m, k))
    return dy, x


@pytest.mark.parametrize("m,n,k,g", [(m, n, k, g) for (m, n, k) in [(512, 256, 256), (768, 272, 400), (256, 16, 48),
                                                                    (1280, 640, 3072), (400, 80, 48), (320, 96, 144),
                                                                    (16, 32, 16)]
                                     for g in (1, 64, 128, 256) if m % g == 0])  # the tokens hold whole blocks
def test_weight_grad_bit_exact(m, n, k, g):
    dy, x = inputs(m, n, k, m + n + k + g)
    say(f"  weight_grad m={m} n={n} k={k} g={g}")
    dw = h.sdnq_qlinear_weight_grad(d_bf16(dy), d_bf16(x), g)
    torch.cuda.synchronize()
    ref = oracle.qlinear_weight_grad(dy, x, g)["dw"]
    got = h_bits(dw)
    assert np.array_equal(got, ref), f"{np.mean(got != ref):.4f} of the outputs differ"


def test_weight_grad_empty_batch_is_zero():
    dy = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    x = torch.zeros((0, 32), dtype=torch.bfloat16, device=DEV)
    dw = h.sdnq_qlinear_weight_grad(dy, x, 256, out=torch.full((64, 32), 7.0, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw).item() == 0


def test_weight_grad_peft_size_sampled_rows():
    """16384 tokens, 3072 x 3072: all of x's codes and scales, and sampled rows of dW."""
    c = synth.CONFIGS["peft"]
    inp = synth.make_config("peft")
    m, n, k = c.m, c.n, c.k
    say(f"  weight_grad m={m} n={n} k={k} g=256")
    ws = torch.empty(h.sdnq_weight_grad_workspace_bytes(m, n, k), dtype=torch.uint8, device=DEV)
    dw = h.sdnq_qlinear_weight_grad(d_bf16(inp["dy"]), d_bf16(inp["x"]), 256, workspace=ws)
    torch.cuda.synchronize()
    oracle.set_num_threads(16)
    xt = np.ascontiguousarray(inp["x"].T)
    qx, sx = oracle.rotate_quantize(xt, 256)
    off = [h.sdnq_weight_grad_workspace_offset(m, n, k, i) for i in range(4)]
    qdy, sdy = oracle.rotate_quantize(np.ascontiguousarray(inp["dy"].T), 256)
    assert np.array_equal(ws[off[0]: off[0] + n * m].view(n, m).cpu().numpy().view(np.int8), qdy)
    sdy_gpu = ws[off[1]: off[1] + 4 * n].cpu().numpy().view(np.float32)
    assert np.array_equal(sdy_gpu.view(np.uint32), sdy.view(np.uint32))
    assert np.array_equal(ws[off[2]: off[2] + k * m].view(k, m).cpu().numpy().view(np.int8), qx)
    sx_gpu = ws[off[3]: off[3] + 4 * k].cpu().numpy().view(np.float32)
    assert np.array_equal(sx_gpu.view(np.uint32), sx.view(np.uint32))
    rows = np.array([0, 1, 1000, 2047, 3071])
    dyt = np.ascontiguousarray(inp["dy"].T)[rows]
    ref = oracle.qlinear_forward(dyt, qx, sx, 256, intermediates=False)["y"]
    assert np.array_equal(h_bits(dw)[rows], ref)


@pytest.mark.parametrize("m,n,k", [(16384, 3072, 3072), (2048, 2000, 3008), (4096, 2896, 3008)])
def test_weight_grad_matches_forward_gemm_on_its_codes(m, n, k):
    """dW against sdnq_qlinear_forward_quantized on the codes the call left in its
    workspace (the same int32 GEMM and epilogue through the forward entry point),
    at sizes too large for the oracle's int64 matmul, with ragged tile edges along
    both output axes."""
    rng = np.random.default_rng(m + n + k)
    dy = synth.to_bf16_bits((rng.standard_normal((m, n)) * 1e-3).astype(np.float32))
    x = synth.to_bf16_bits(synth.outlier_activations(rng, m, k))
    say(f"  weight_grad m={m} n={n} k={k} g=256 against the forward GEMM")
    ws = torch.empty(h.sdnq_weight_grad_workspace_bytes(m, n, k), dtype=torch.uint8, device=DEV)
    dw = h.sdnq_qlinear_weight_grad(d_bf16(dy), d_bf16(x), 256, workspace=ws)
    off = [h.sdnq_weight_grad_workspace_offset(m, n, k, i) for i in range(4)]
    qdy = ws[off[0]: off[0] + n * m].view(torch.int8).view(n, m)
    sdy = ws[off[1]: off[1] + 4 * n].view(torch.float32)
    qx = ws[off[2]: off[2] + k * m].view(torch.int8).view(k, m)
    sx = ws[off[3]: off[3] + 4 * k].view(torch.float32)
    whole = h.sdnq_qlinear_forward_quantized(qdy, sdy, qx, sx)
    torch.cuda.synchronize()
    got, ref = h_bits(dw), h_bits(whole)
    assert np.array_equal(got, ref), f"{np.mean(got != ref):.6f} of the outputs differ"
    assert np.count_nonzero(ref) > 0.9 * ref.size


def stress_columns(m, n, seed):
    """[m, n]: feature columns (along the tokens) at the quantizer's edge cases,
    then normal columns."""
    rng = np.random.default_rng(seed)
    cols = [np.zeros(m, np.float32)]                                        # all-zero feature
    c = rng.standard_normal(m).astype(np.float32); c[17] = 1e15; cols.append(c)   # one large token
    c = rng.standard_normal(m).astype(np.float32); c[rng.permutation(m)[:5]] *= 1000; cols.append(c)
    cols.append((rng.standard_normal(m) * 1e-38).astype(np.float32))      # tiny (normal and subnormal)
    cols.append((rng.standard_normal(m) * 1e-36).astype(np.float32))
    c = np.zeros(m, np.float32); c[:4] = [1.0, 2.0 ** -24, -1.0, 2.0 ** -24]; cols.append(c)  # stage order
    c = (rng.integers(-254, 255, m) / 2.0).astype(np.float32); c[3] = 127.0; cols.append(c)  # ties
    c = np.zeros(m, np.float32); c[:2] = [1.125, 0.5625]; cols.append(c)  # reciprocal case
    cols.append(np.full(m, 3.0, np.float32))                               # constant
    c = np.zeros(m, np.float32); c[m // 2] = 1.0; cols.append(c)           # one-hot
    cols.append(-np.abs(rng.standard_normal(m)).astype(np.float32))
    while len(cols) < n:
        cols.append(rng.standard_normal(m).astype(np.float32))
    return np.stack(cols[:n], axis=1)


@pytest.mark.parametrize("g", [1, 64, 256])
def test_weight_grad_stress_columns(g):
    """dY and x with feature columns at the quantizer's edge cases: dW bit for bit."""
    m = 512
    dy = synth.to_bf16_bits(stress_columns(m, 48, 60))
    x = synth.to_bf16_bits(stress_columns(m, 32, 61))
    say(f"  weight_grad stress columns m={m} n=48 k=32 g={g}")
    dw = h.sdnq_qlinear_weight_grad(d_bf16(dy), d_bf16(x), g)
    torch.cuda.synchronize()
    ref = oracle.qlinear_weight_grad(dy, x, g)["dw"]
    got = h_bits(dw)
    assert np.array_equal(got, ref), f"{np.mean(got != ref):.4f} of the outputs differ"
