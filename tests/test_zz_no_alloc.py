"""The forward entry point that allocates nothing (its workspace is the library's
fixed device array), through the C ABI, against the workspace forward on the same
inputs: two calls in a row, the second with a smaller input, must give the same
bits as sdnq_qlinear_forward (the same kernels on the same data); a call that
would need more than the array holds is refused before any launch."""
import ctypes

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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    h.lib()
    yield
    torch.cuda.synchronize()


def d_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def h_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("rank", [0, 32])
def test_noalloc_forward_equals_workspace_forward(rank):
    for (m, k, n, g, seed) in [(4096, 3072, 3072, 128, 1), (300, 768, 640, 64, 2)]:  # second call smaller
        say(f"  noalloc forward m={m} k={k} n={n} g={g} rank={rank}")
        inp = synth.make_linear(m, k, n, seed=seed, lora_rank=rank)
        x = d_bf16(inp["x"])
        la = d_bf16(inp["lora_a"]) if rank else None
        lb = d_bf16(inp["lora_b"]) if rank else None
        qw, sw = h.sdnq_rotate_quantize_weight(d_bf16(inp["w"]), g)
        y_ws = h.sdnq_qlinear_forward(x, qw, sw, g, la, lb, 0.5)
        y = torch.full((m, n), 7.0, dtype=torch.bfloat16, device=DEV)
        L = h.lib()
        P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        rc = L.sdnq_qlinear_forward_noalloc(P(x), m, k, P(qw), P(sw), n, g, P(la), P(lb), rank, 0.5, P(y),
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert rc == h.SDNQ_OK, h.status_string(rc)
        assert torch.equal(y.view(torch.int16), y_ws.view(torch.int16))
        if m <= 512:  # and against the oracle on the small call
            qwo, swo = oracle.rotate_quantize(inp["w"], g)
            ref = oracle.qlinear_forward(inp["x"], qwo, swo, g, inp.get("lora_a"), inp.get("lora_b"), 0.5)
            if rank == 0:
                assert np.array_equal(h_bits(y), ref["y"])
            else:
                a = synth.bf16_bits_to_f32(h_bits(y)).astype(np.float64)
                b = synth.bf16_bits_to_f32(ref["y"]).astype(np.float64)
                assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-2


def test_noalloc_forward_refuses_a_call_larger_than_its_array():
    m, k, n = 8192, 8192 + 256, 256  # m * k codes alone exceed the array
    assert h.sdnq_workspace_bytes(m, n, k, 0, False) > h.SDNQ_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((m, k), dtype=torch.bfloat16, device=DEV)
    qw = torch.zeros((n, k), dtype=torch.int8, device=DEV)
    sw = torch.zeros((n,), dtype=torch.float32, device=DEV)
    y = torch.full((m, n), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(h.SdnqError) as e:
        h.sdnq_qlinear_forward_noalloc(x, qw, sw, 256, out=y)
    assert e.value.status == h.SDNQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 3.0).item()  # nothing was written
