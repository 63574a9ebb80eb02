"""GPU parity at the workloads' full sizes, through the entry points and launch
configuration the benchmark uses.

Integer stages are compared in full and bit-exactly: the weight codes and
scales, and the activation (or upstream-gradient) codes and scales that the
forward / backward entry points leave in their workspace.  Outputs are compared
on sampled token rows (the first, the last and a seeded random set), which the
oracle computes row by row; without LoRA they are bit-exact, with LoRA and for
the input gradient within 1e-2 relative L2.  The LoRA weight gradients are a
reduction over all tokens and are compared in full.
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_int8_amd as h
import oracle
from hadamard_rotated_int8_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL_L2 = 1e-2


def say(*a):
    print(*a, flush=True)


def d_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def h_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def rel_l2(got_bits, ref_bits):
    g = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    r = synth.bf16_bits_to_f32(ref_bits).astype(np.float64)
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))


def max_token_rel(got_bits, ref_bits):
    g = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    r = synth.bf16_bits_to_f32(ref_bits).astype(np.float64)
    return float((np.linalg.norm(g - r, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-30)).max())


def assert_tokens_close(got_bits, ref_bits, what):
    """Relative L2 over the sampled rows and for the worst sampled token row, both below 1e-2."""
    err, tok = rel_l2(got_bits, ref_bits), max_token_rel(got_bits, ref_bits)
    say(f"    {what} rel-L2 {err:.3e}  max-row {tok:.3e}")
    assert err < REL_L2 and tok < REL_L2, f"{what}: rel-L2 {err:.3e}, worst token {tok:.3e}"


def sample_rows(m, count=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(range(16)) | set(range(m - 16, m)) | set(rng.choice(m, count - 32, replace=False).tolist())
    return np.array(sorted(rows))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    h.lib()
    oracle.set_num_threads(16)
    yield
    torch.cuda.synchronize()


def prep_weight(w_bits, g):
    say(f"  weight {w_bits.shape} g={g}")
    qw, sw = h.sdnq_rotate_quantize_weight(d_bf16(w_bits), g)
    torch.cuda.synchronize()
    qwo, swo = oracle.rotate_quantize(w_bits, g)
    assert np.array_equal(qw.cpu().numpy(), qwo), "weight codes"
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), swo.view(np.uint32)), "weight scales"
    return qw, sw, qwo, swo


def run_forward(x_bits, w_bits, g, lora=None, scale=0.0):
    m, k = x_bits.shape
    n = w_bits.shape[0]
    qw, sw, qwo, swo = prep_weight(w_bits, g)
    return forward_prepared(x_bits, qw, sw, qwo, swo, g, lora, scale)


def zero_weight(n, k):
    """All-zero codes and scales: the forward's output is the LoRA term alone and
    the backward's folded dY is zero, so dX is its LoRA term alone."""
    qwo, swo = np.zeros((n, k), np.int8), np.zeros(n, np.float32)
    return torch.from_numpy(qwo).to(DEV), torch.from_numpy(swo).to(DEV), qwo, swo


def forward_prepared(x_bits, qw, sw, qwo, swo, g, lora=None, scale=0.0):
    m, k = x_bits.shape
    n = qwo.shape[0]
    rank = 0 if lora is None else lora[0].shape[1]
    ws = torch.empty(h.sdnq_workspace_bytes(m, n, k, rank, False), dtype=torch.uint8, device=DEV)
    say(f"  forward m={m} k={k} n={n} g={g} rank={rank}")
    la = None if lora is None else d_bf16(lora[0])
    lb = None if lora is None else d_bf16(lora[1])
    y = h.sdnq_qlinear_forward(d_bf16(x_bits), qw, sw, g, la, lb, scale, workspace=ws)
    torch.cuda.synchronize()
    # the forward's own activation codes and scales: first two regions of its workspace
    qx = ws[: m * k].view(m, k).cpu().numpy().view(np.int8)
    off = (m * k + 255) // 256 * 256
    sx = ws[off: off + 4 * m].cpu().numpy().view(np.float32)
    qxo, sxo = oracle.rotate_quantize(x_bits, g)
    bad = np.nonzero(np.any(qx != qxo, axis=1))[0]
    assert bad.size == 0, f"activation codes differ in rows {bad[:8]}"
    assert np.array_equal(sx.view(np.uint32), sxo.view(np.uint32)), "activation scales"
    rows = sample_rows(m)
    ref = oracle.qlinear_forward(x_bits[rows], qwo, swo, g, None if lora is None else lora[0],
                                 None if lora is None else lora[1], scale, intermediates=False)
    return h_bits(y)[rows], ref["y"]


@pytest.mark.parametrize("name", ["attn", "mlp_up", "mlp_down"])
def test_forward_full_size_bit_exact(name):
    inp = synth.make_config(name)
    y, ref = run_forward(inp["x"], inp["w"], 256)
    assert np.array_equal(y, ref), f"rel-L2 {rel_l2(y, ref):.3e}"


def test_mlp_pair_as_benchmarked():
    """The benchmark's step: rotate_quantize_act + forward_quantized for both layers."""
    inp = synth.make_config("mlp")
    for xk, wk in (("x", "w_up"), ("h", "w_down")):
        qw, sw, qwo, swo = prep_weight(inp[wk], 256)
        say(f"  bench path {xk}")
        qx, sx = h.sdnq_rotate_quantize_act(d_bf16(inp[xk]), 256)
        y = h.sdnq_qlinear_forward_quantized(qx, sx, qw, sw)
        torch.cuda.synchronize()
        rows = sample_rows(inp[xk].shape[0], seed=1)
        ref = oracle.qlinear_forward(inp[xk][rows], qwo, swo, 256, intermediates=False)
        assert np.array_equal(h_bits(y)[rows], ref["y"])


@pytest.mark.parametrize("g", [64, 128])
def test_quarot_lora_full_size(g):
    c = synth.CONFIGS["quarot"]
    inp = synth.make_config("quarot")
    y, ref = run_forward(inp["x"], inp["w"], g, (inp["lora_a"], inp["lora_b"]), c.lora_scale)
    assert_tokens_close(y, ref, "y")


@pytest.mark.parametrize("g", [64, 128])
def test_quarot_lora_term_full_size(g):
    """The LoRA term alone (zero weight), so that a wrong term cannot hide under
    the int8 product, which is about 35 times larger."""
    c = synth.CONFIGS["quarot"]
    inp = synth.make_config("quarot")
    qw, sw, qwo, swo = zero_weight(c.n, c.k)
    y, ref = forward_prepared(inp["x"], qw, sw, qwo, swo, g, (inp["lora_a"], inp["lora_b"]), c.lora_scale)
    assert_tokens_close(y, ref, "LoRA term")


def test_peft_forward_full_size():
    c = synth.CONFIGS["peft"]
    inp = synth.make_config("peft")
    y, ref = run_forward(inp["x"], inp["w"], 256, (inp["lora_a"], inp["lora_b"]), c.lora_scale)
    assert_tokens_close(y, ref, "y")


def test_peft_backward_full_size():
    c = synth.CONFIGS["peft"]
    inp = synth.make_config("peft")
    m, k, n = c.m, c.k, c.n
    qw, sw, qwo, swo = prep_weight(inp["w"], 256)
    ws = torch.empty(h.sdnq_workspace_bytes(m, n, k, c.lora_rank, True), dtype=torch.uint8, device=DEV)
    say(f"  backward m={m} n={n} k={k} rank={c.lora_rank}")
    dx, ga, gb = h.sdnq_qlinear_backward_input(d_bf16(inp["dy"]), qw, sw, 256, d_bf16(inp["x"]),
                                               d_bf16(inp["lora_a"]), d_bf16(inp["lora_b"]), c.lora_scale,
                                               workspace=ws)
    torch.cuda.synchronize()
    qdy = ws[: m * n].view(m, n).cpu().numpy().view(np.int8)
    off = (m * n + 255) // 256 * 256
    sdy = ws[off: off + 4 * m].cpu().numpy().view(np.float32)
    qo, so = oracle.rotate_quantize(inp["dy"], 1, swo)
    assert np.array_equal(qdy, qo), "dY codes"
    assert np.array_equal(sdy.view(np.uint32), so.view(np.uint32)), "dY scales"
    rows = sample_rows(m, seed=2)
    ref = oracle.qlinear_backward_input(inp["dy"][rows], qwo, swo, 256, None, inp["lora_a"], inp["lora_b"],
                                        c.lora_scale, want_grads=False, intermediates=False)
    assert_tokens_close(h_bits(dx)[rows], ref["dx"], "dx")
    say("  LoRA gradients (oracle over all tokens)")
    grads = oracle.qlinear_backward_input(inp["dy"], qwo, swo, 256, inp["x"], inp["lora_a"], inp["lora_b"],
                                          c.lora_scale, want_dx=False)
    e_a, e_b = rel_l2(h_bits(ga), grads["grad_a"]), rel_l2(h_bits(gb), grads["grad_b"])
    say(f"    grad_a {e_a:.3e}  grad_b {e_b:.3e}")
    assert e_a < REL_L2 and e_b < REL_L2


def test_peft_backward_full_size_without_lora_bit_exact():
    """Without LoRA the input gradient is bit-exact: one fp32 conversion of the int32
    accumulator times the dY scale, the inverse butterfly in the oracle's stage
    order, the 1/sqrt(g) factor and one rounding to bf16."""
    c = synth.CONFIGS["peft"]
    inp = synth.make_config("peft")
    qw, sw, qwo, swo = prep_weight(inp["w"], 256)
    say(f"  backward m={c.m} n={c.n} k={c.k} without LoRA")
    dx, _, _ = h.sdnq_qlinear_backward_input(d_bf16(inp["dy"]), qw, sw, 256)
    torch.cuda.synchronize()
    rows = sample_rows(c.m, seed=3)
    ref = oracle.qlinear_backward_input(inp["dy"][rows], qwo, swo, 256, want_grads=False, intermediates=False)
    got = h_bits(dx)[rows]
    assert np.array_equal(got, ref["dx"]), f"dx rel-L2 {rel_l2(got, ref['dx']):.3e}"


def test_peft_backward_lora_term_full_size():
    """dX's LoRA term g_r A^T alone (zero weight folds dY to zero), per token."""
    c = synth.CONFIGS["peft"]
    inp = synth.make_config("peft")
    qw, sw, qwo, swo = zero_weight(c.n, c.k)
    say(f"  backward m={c.m} LoRA term alone")
    dx, _, _ = h.sdnq_qlinear_backward_input(d_bf16(inp["dy"]), qw, sw, 256, None, d_bf16(inp["lora_a"]),
                                             d_bf16(inp["lora_b"]), c.lora_scale)
    torch.cuda.synchronize()
    rows = sample_rows(c.m, seed=4)
    ref = oracle.qlinear_backward_input(inp["dy"][rows], qwo, swo, 256, None, inp["lora_a"], inp["lora_b"],
                                        c.lora_scale, want_grads=False, intermediates=False)
    assert_tokens_close(h_bits(dx)[rows], ref["dx"], "LoRA term")
