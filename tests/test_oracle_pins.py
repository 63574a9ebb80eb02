"""Pins for the CPU oracle: each test checks the oracle against something other
than itself (closed forms, hand-derived fixtures, textbook/library routines,
brute force, exact rational arithmetic, error bounds, autograd), chosen so that
a plausible slip (a dropped term, a wrong sign or index, a transposed operand, a
different Hadamard ordering or rounding mode) fails at least one of them.

Sources of the definitions being pinned: "ConvRot / Hadamard SDNQ" (SimpleTuner
docs, "What The Options Do"), "SDNQ: SD.Next Quantization Engine" (feature list,
SDNQConfig example, quantized-training example) and the HSWQ README ("Rigorous
grid / pack simulation").
"""
import json
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from hadamard_rotated_int8_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def nearest_f32(fr: Fraction) -> np.float32:
    """Binary32 nearest to a rational (ties to even), by exact comparison."""
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]

    def key(c):
        return (abs(Fraction(float(c)) - fr), int(np.float32(c).view(np.uint32)) & 1)
    return min(cands, key=key)


def f32_bits(v) -> int:
    return int(np.float32(v).view(np.uint32))


def bf(a):
    return synth.to_bf16_bits(np.asarray(a, np.float32))


# ------------------------------------------------------------- P1 / P3 --

@pytest.mark.parametrize("g", [2, 4, 8, 16, 32, 64, 128, 256])
def test_butterfly_on_identity_is_sylvester_hadamard(g):
    """P1: the butterfly applied to the identity reproduces scipy's Sylvester
    Hadamard matrix exactly; it is symmetric and H H^T = g I (integer exact)."""
    h = oracle.fwht_unnormalized(np.eye(g, dtype=np.float32), g)
    ref = scipy.linalg.hadamard(g)
    # row i of the result is H e_i = column i of H
    assert np.array_equal(h.T, ref.astype(np.float32))
    assert np.array_equal(h, h.T)
    assert np.array_equal(h.astype(np.int64) @ h.astype(np.int64).T, g * np.eye(g, dtype=np.int64))


@pytest.mark.parametrize("g", [64, 128, 256])
def test_sylvester_entry_closed_form(g):
    """H[i, j] = (-1)^popcount(i & j) for the natural-order Sylvester matrix."""
    h = oracle.fwht_unnormalized(np.eye(g, dtype=np.float32), g)
    i, j = np.meshgrid(np.arange(g), np.arange(g), indexing="ij")
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    assert np.array_equal(h, np.where(pc % 2 == 0, 1.0, -1.0).astype(np.float32))


@pytest.mark.parametrize("g", [64, 128, 256])
def test_butterfly_involution_on_integers(g):
    """H (H v) = g v exactly for small integer v (every partial sum is exact)."""
    rng = np.random.default_rng(1)
    v = rng.integers(-100, 101, size=(5, g)).astype(np.float32)
    hv = oracle.fwht_unnormalized(oracle.fwht_unnormalized(v, g), g)
    assert np.array_equal(hv, g * v)


@pytest.mark.parametrize("g", [64, 128, 256])
def test_butterfly_matches_dense_fp64_within_rounding(g):
    """P3: on random binary32 input the butterfly agrees with the fp64 dense
    product within the log2(g)-level rounding bound."""
    rng = np.random.default_rng(2)
    v = rng.standard_normal((7, 4 * g)).astype(np.float32)
    u = oracle.fwht_unnormalized(v, g).astype(np.float64)
    hd = scipy.linalg.hadamard(g).astype(np.float64)
    ref = (v.astype(np.float64).reshape(7, 4, g) @ hd.T).reshape(7, 4 * g)
    bound = np.log2(g) * 2.0 ** -24 * 1.01 * (np.abs(v.astype(np.float64)).reshape(7, 4, g).sum(-1))
    err = np.abs(u - ref).reshape(7, 4, g).max(-1)
    assert np.all(err <= bound)


# ------------------------------------------------------------------ P2 --

@pytest.mark.parametrize("g", [2, 4, 8, 16, 32, 64, 128, 256])
def test_norm_const_is_nearest_binary32_to_inverse_sqrt(g):
    """c_g = fl32(1/sqrt(g)), checked with 60-digit decimal arithmetic."""
    getcontext().prec = 60
    exact = Decimal(1) / Decimal(g).sqrt()
    c = oracle.norm_const(g)
    lo = np.nextafter(c, np.float32(0))
    hi = np.nextafter(c, np.float32(1))
    d = abs(Decimal(float(c)) - exact)
    assert d <= abs(Decimal(float(lo)) - exact) and d <= abs(Decimal(float(hi)) - exact)


def test_norm_const_bit_patterns():
    assert f32_bits(oracle.norm_const(64)) == 0x3E000000
    assert f32_bits(oracle.norm_const(128)) == 0x3DB504F3
    assert f32_bits(oracle.norm_const(256)) == 0x3D800000
    assert oracle.norm_const(1) == 1.0


@pytest.mark.parametrize("g", [64, 128, 256])
def test_normalized_transform_is_orthonormal(g):
    """P2: (c H)(c H)^T = I to a few binary32 ulps (exact for g = 64, 256)."""
    h = oracle.fwht_unnormalized(np.eye(g, dtype=np.float32), g).astype(np.float64)
    c = float(oracle.norm_const(g))
    dev = np.abs((c * h) @ (c * h).T - np.eye(g)).max()
    if g in (64, 256):
        assert dev == 0.0
    else:
        assert dev < 4 * 2.0 ** -24


# ------------------------------------------------------------------ P4 --

@pytest.mark.parametrize("g", [64, 128, 256])
def test_rotation_invariance_of_the_product(g):
    """P4: x W^T = (x R)(W R)^T with R the normalized block rotation, on the
    oracle's unquantized binary32 rotation (within binary32 rounding)."""
    rng = np.random.default_rng(3)
    x = bf(rng.standard_normal((16, 512)))
    w = bf(rng.standard_normal((24, 512)) * 0.02)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    ref = xf @ wf.T
    rot = oracle.rotate(x, g).astype(np.float64) @ oracle.rotate(w, g).astype(np.float64).T
    assert np.linalg.norm(rot - ref) / np.linalg.norm(ref) < 2e-6


@pytest.mark.parametrize("g", [64, 128, 256])
def test_rotation_equals_block_diagonal_dense_product(g):
    """The rotation acts on contiguous g-blocks along the row, in block order."""
    rng = np.random.default_rng(4)
    x = bf(rng.standard_normal((5, 3 * g)))
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    r = np.kron(np.eye(3), scipy.linalg.hadamard(g) / np.sqrt(g))
    ref = xf @ r.T
    got = oracle.rotate(x, g).astype(np.float64)
    assert np.abs(got - ref).max() < 1e-5 * np.abs(xf).max() * np.sqrt(g)


def test_rotation_g1_is_identity_and_column_scale_multiplies():
    rng = np.random.default_rng(5)
    x = bf(rng.standard_normal((3, 64)))
    cs = rng.uniform(0.5, 2.0, 64).astype(np.float32)
    xf = synth.bf16_bits_to_f32(x)
    assert np.array_equal(oracle.rotate(x, 1), xf)
    assert np.array_equal(oracle.rotate(x, 1, cs), xf * cs)


# ------------------------------------------------------------------ P5 --

def _cases():
    with open(GOLDEN) as f:
        return {c["name"]: c for c in json.load(f)["cases"]}


@pytest.mark.parametrize("name", ["g4_ramp", "g1_rne_ties", "g1_multiply_by_reciprocal", "g4_stage_order",
                                  "g1_tiny_row"])
def test_hand_worked_rows(name):
    c = _cases()[name]
    x = bf(np.array([c["x"]], np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(x)[0], np.array(c["x"], np.float32))
    y = oracle.rotate(x, c["g"])
    assert np.array_equal(y[0], np.array(c["rotated"], np.float32))
    q, s = oracle.rotate_quantize(x, c["g"])
    assert q[0].tolist() == c["codes"]
    expect = nearest_f32(Fraction(*c["scale_rational"]))
    assert f32_bits(expect) == int(c["scale_bits"], 16)
    assert f32_bits(s[0]) == int(c["scale_bits"], 16)


def test_hand_worked_stage_order_in_a_256_block():
    """The butterfly's stage order is visible in binary32: ascending stages give
    2^-24 where descending ones give the exact 2^-23 (derivation in the fixture)."""
    c = _cases()["g256_stage_order"]
    x = np.zeros((1, c["cols"]), np.float32)
    x[0, :4] = c["x_head"]
    xb = bf(x)
    assert np.array_equal(synth.bf16_bits_to_f32(xb), x)
    y = oracle.rotate(xb, c["g"])
    assert np.array_equal(y[0], np.tile(np.array(c["rotated_period"], np.float32), c["cols"] // 4))
    q, s = oracle.rotate_quantize(xb, c["g"])
    assert np.array_equal(q[0], np.tile(np.array(c["codes_period"], np.int8), c["cols"] // 4))
    assert f32_bits(nearest_f32(Fraction(*c["scale_rational"]))) == int(c["scale_bits"], 16)
    assert f32_bits(s[0]) == int(c["scale_bits"], 16)


def test_hand_worked_constant_block():
    c = _cases()["g256_constant_block"]
    x = bf(np.full((1, c["cols"]), c["x_constant"], np.float32))
    y = oracle.rotate(x, c["g"])
    assert y[0, 0] == c["rotated_first"] and np.all(y[0, 1:] == 0)
    q, s = oracle.rotate_quantize(x, c["g"])
    assert q[0, 0] == c["codes_first"] and np.all(q[0, 1:] == 0)
    assert f32_bits(nearest_f32(Fraction(*c["scale_rational"]))) == int(c["scale_bits"], 16)
    assert f32_bits(s[0]) == int(c["scale_bits"], 16)


@pytest.mark.parametrize("g", [64, 128, 256])
def test_one_hot_codes_follow_the_hadamard_sign_pattern(g):
    """P5: x = e_j gives codes +-127 in j's block with sign (-1)^popcount(i & j_local),
    zeros elsewhere; s = fl32(c_g / 127)."""
    cols, hot = 512, 300
    x = np.zeros((1, cols), np.float32)
    x[0, hot] = 1.0
    q, s = oracle.rotate_quantize(bf(x), g)
    b0 = (hot // g) * g
    jl = hot - b0
    sign = np.array([1 if bin(i & jl).count("1") % 2 == 0 else -1 for i in range(g)])
    expect = np.zeros(cols, np.int64)
    expect[b0:b0 + g] = 127 * sign
    assert np.array_equal(q[0].astype(np.int64), expect)
    c = oracle.norm_const(g)
    assert s[0] == np.float32(c) / np.float32(127)
    if g == 256:
        case = _cases()["g256_one_hot"]
        assert f32_bits(s[0]) == int(case["scale_bits"], 16)


def test_zero_row_gives_zero_scale_and_codes():
    q, s = oracle.rotate_quantize(np.zeros((2, 256), np.uint16), 256)
    assert np.all(q == 0) and np.all(s == 0)


def test_g1_is_textbook_per_row_absmax_on_integer_grid_rows():
    """g = 1 on rows whose absmax is 127: r = 1, codes are the round-half-even
    of the values (numpy's rint is round-half-even)."""
    rng = np.random.default_rng(6)
    v = (rng.integers(-254, 255, size=(4, 64)) / 2.0).astype(np.float32)
    v[:, 0] = 127.0
    q, s = oracle.rotate_quantize(bf(v), 1)
    assert np.all(s == 1.0)
    assert np.array_equal(q.astype(np.int64), np.rint(v).astype(np.int64))


# ------------------------------------------------------------------ P6 --

@pytest.mark.parametrize("b_layout", [0, 1])
def test_gemm_brute_force_python_loops(b_layout):
    rng = np.random.default_rng(7)
    m, n, k = 3, 5, 70
    a = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
    b = rng.integers(-128, 128, size=(n, k) if b_layout == 0 else (k, n)).astype(np.int8)
    c = oracle.gemm_i8(a, b, b_layout)
    for i in range(m):
        for j in range(n):
            s = 0
            for t in range(k):
                bv = int(b[j, t]) if b_layout == 0 else int(b[t, j])
                s += int(a[i, t]) * bv
            assert c[i, j] == s


def test_gemm_int32_range_check():
    k_ok, k_bad = 133144, 133145
    a = np.full((1, k_ok), 127, np.int8)
    assert oracle.gemm_i8(a, a, 0)[0, 0] == 127 * 127 * k_ok
    a = np.full((1, k_bad), 127, np.int8)
    with pytest.raises(OverflowError):
        oracle.gemm_i8(a, a, 0)


def test_tiny_config_accumulators_equal_int64_matmul():
    d = synth.make_config("tiny")
    qw, sw = oracle.rotate_quantize(d["w"], 256)
    out = oracle.qlinear_forward(d["x"], qw, sw, 256)
    ref = out["qx"].astype(np.int64) @ qw.astype(np.int64).T
    assert np.array_equal(out["acc"].astype(np.int64), ref)
    q, s = oracle.rotate_quantize(d["x"], 256)
    assert np.array_equal(q, out["qx"]) and np.array_equal(s, out["sx"])


# ------------------------------------------------------------------ P7 --

@pytest.mark.parametrize("g", [1, 64, 128, 256])
def test_quantization_error_bound_and_full_scale_code(g):
    d = synth.make_config("tiny")
    y = oracle.rotate(d["x"], g).astype(np.float64)
    q, s = oracle.rotate_quantize(d["x"], g)
    s64 = s.astype(np.float64)[:, None]
    err = np.abs(y - q.astype(np.float64) * s64)
    assert np.all(err <= 0.5 * s64 * (1 + 1e-6) + 1e-6 * np.abs(y))
    assert np.all(np.abs(q.astype(np.int64)).max(axis=1) == 127)
    assert q.min() >= -127


# ------------------------------------------------------------------ P8 --

def test_rotation_reduces_quantization_error_on_outlier_inputs():
    """The method's premise ("ConvRot can reduce quantization damage"): on
    outlier-channel activations the rotated int8 product is closer to the fp64
    product than the unrotated one."""
    d = synth.make_config("tiny")
    xf = synth.bf16_bits_to_f32(d["x"]).astype(np.float64)
    wf = synth.bf16_bits_to_f32(d["w"]).astype(np.float64)
    ref = xf @ wf.T
    errs = {}
    for g in (1, 64, 128, 256):
        qw, sw = oracle.rotate_quantize(d["w"], g)
        base = oracle.qlinear_forward(d["x"], qw, sw, g)["base"].astype(np.float64)
        errs[g] = np.linalg.norm(base - ref) / np.linalg.norm(ref)
    assert errs[256] < 0.5 * errs[1]
    assert errs[64] < 0.5 * errs[1] and errs[128] < 0.5 * errs[1]
    assert errs[256] < 2e-2


# ------------------------------------------------------ forward output --

@pytest.mark.parametrize("g", [64, 256])
def test_forward_dequant_matches_fp64_scaled_codes(g):
    """O9: base = acc * s_x * s_w within binary32 rounding (catches a transposed
    or mis-indexed scale), and y = bf16(base) exactly without LoRA."""
    rng = np.random.default_rng(8)
    m, k, n = 9, 512, 40
    x = bf(rng.standard_normal((m, k)))
    w = bf(rng.standard_normal((n, k)) * 0.02)
    qw, sw = oracle.rotate_quantize(w, g)
    out = oracle.qlinear_forward(x, qw, sw, g)
    ref = (out["qx"].astype(np.float64) * out["sx"][:, None]) @ (qw.astype(np.float64) * sw[:, None]).T
    assert np.all(np.abs(out["base"] - ref) <= 3e-7 * np.abs(ref) + 1e-30)
    assert np.array_equal(out["y"], torch.from_numpy(out["base"]).to(torch.bfloat16).view(torch.int16)
                          .numpy().view(np.uint16))


def test_forward_lora_term_against_torch_fp64():
    rng = np.random.default_rng(9)
    m, k, n, r = 6, 256, 48, 8
    x = bf(rng.standard_normal((m, k)))
    w = bf(rng.standard_normal((n, k)) * 0.02)
    la = bf(rng.standard_normal((k, r)) * 0.3)
    lb = bf(rng.standard_normal((r, n)) * 0.3)
    qw, sw = oracle.rotate_quantize(w, 256)
    scale = 0.75
    out = oracle.qlinear_forward(x, qw, sw, 256, la, lb, scale)
    t = lambda a: torch.from_numpy(synth.bf16_bits_to_f32(a).astype(np.float64))
    lora = (t(x) @ t(la) @ t(lb) * scale).numpy()
    expect = oracle.bf16_from_f64(out["base"].astype(np.float64) + lora)
    assert np.array_equal(out["y"], expect)
    # the LoRA term is not negligible in this case
    assert np.abs(lora).mean() > 0.5 * np.abs(out["base"]).mean()


# ------------------------------------------------------------- backward --

@pytest.mark.parametrize("g", [64, 256])
def test_backward_base_matches_fp64_dense(g):
    """B1-B5 on a non-square weight: z = (q_dy s_dy) qw, then the normalized block
    rotation (fp64 dense with scipy's Hadamard) equals the oracle's dxbase within
    binary32 rounding; the fold multiplies dY by s_w column-wise."""
    rng = np.random.default_rng(10)
    m, n, k = 7, 384, 512
    dy = bf(rng.standard_normal((m, n)) * 1e-3)
    w = bf(rng.standard_normal((n, k)) * 0.02)
    qw, sw = oracle.rotate_quantize(w, g)
    out = oracle.qlinear_backward_input(dy, qw, sw, g)
    q2, s2 = oracle.rotate_quantize(dy, 1, col_scale=sw)
    assert np.array_equal(q2, out["qdy"]) and np.array_equal(s2, out["sdy"])
    acc = out["qdy"].astype(np.int64) @ qw.astype(np.int64)
    assert np.array_equal(acc, out["acc"].astype(np.int64))
    z = acc.astype(np.float64) * out["sdy"].astype(np.float64)[:, None]
    r = np.kron(np.eye(k // g), scipy.linalg.hadamard(g) / np.sqrt(g))
    ref = z @ r.T
    assert np.abs(out["dxbase"] - ref).max() <= 1e-5 * np.abs(ref).max()


def test_backward_approximates_unquantized_input_gradient():
    """P9: dX ~ dY W (original, unrotated bf16 weight) up to quantization error."""
    d = synth.make_linear(32, 768, 512, seed=11, backward=True)
    qw, sw = oracle.rotate_quantize(d["w"], 256)
    out = oracle.qlinear_backward_input(d["dy"], qw, sw, 256)
    ref = synth.bf16_bits_to_f32(d["dy"]).astype(np.float64) @ synth.bf16_bits_to_f32(d["w"]).astype(np.float64)
    dx = synth.bf16_bits_to_f32(out["dx"]).astype(np.float64)
    assert np.linalg.norm(dx - ref) / np.linalg.norm(ref) < 2e-2


def test_lora_gradients_against_torch_autograd():
    """dA, dB and the LoRA part of dX equal torch autograd (fp64) of
    sum(dY * ((x A) B * scale)) up to the final bf16 rounding."""
    d = synth.make_linear(24, 256, 128, seed=12, lora_rank=16, backward=True)
    scale = 2.0
    qw, sw = oracle.rotate_quantize(d["w"], 64)
    out = oracle.qlinear_backward_input(d["dy"], qw, sw, 64, d["x"], d["lora_a"], d["lora_b"], scale)
    t = lambda a, grad=False: torch.tensor(synth.bf16_bits_to_f32(a).astype(np.float64), requires_grad=grad)
    x, A, B, dY = t(d["x"], True), t(d["lora_a"], True), t(d["lora_b"], True), t(d["dy"])
    ((x @ A @ B * scale) * dY).sum().backward()
    for name, ref in (("grad_a", A.grad), ("grad_b", B.grad)):
        assert np.array_equal(out[name], oracle.bf16_from_f64(ref.numpy())), name
    dx_expect = oracle.bf16_from_f64(out["dxbase"].astype(np.float64) + x.grad.numpy())
    assert np.array_equal(out["dx"], dx_expect)


def test_lora_gradients_only_call_matches_the_full_call():
    d = synth.make_linear(40, 256, 192, seed=15, lora_rank=32, backward=True)
    qw, sw = oracle.rotate_quantize(d["w"], 128)
    full = oracle.qlinear_backward_input(d["dy"], qw, sw, 128, d["x"], d["lora_a"], d["lora_b"], 0.5)
    only = oracle.qlinear_backward_input(d["dy"], qw, sw, 128, d["x"], d["lora_a"], d["lora_b"], 0.5,
                                         want_dx=False)
    assert only["dx"] is None
    assert np.array_equal(full["grad_a"], only["grad_a"]) and np.array_equal(full["grad_b"], only["grad_b"])


# ------------------------------------------------------------- bf16 rounding --

def test_bf16_encoder_matches_torch_on_binary32_values():
    rng = np.random.default_rng(13)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
                        # exact ties: 8 significant bits plus a half ulp
                        (1.0 + (2 * rng.integers(0, 128, 2000) + 1) * 2.0 ** -8).astype(np.float32)])
    v = v.astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_from_f64(v.astype(np.float64)), ref)


def test_bf16_encoder_single_rounding_and_specials():
    cases = [
        (1.0 + 2.0 ** -8, 0x3F80),                  # tie -> even
        (1.0 + 3 * 2.0 ** -8, 0x3F82),              # tie -> even (up)
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),     # just above the tie (binary32 first would give 0x3F80)
        (-(1.0 + 2.0 ** -8 + 2.0 ** -40), 0xBF81),
        (0.0, 0x0000), (-0.0, 0x8000),
        (2.0 ** -133, 0x0001),                      # smallest subnormal
        (2.0 ** -134, 0x0000),                      # tie with zero -> even
        (3 * 2.0 ** -134, 0x0002),                  # tie -> even
        ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),     # largest finite
        ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),     # tie at the top rounds to infinity
        (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
    ]
    got = oracle.bf16_from_f64(np.array([v for v, _ in cases], np.float64))
    assert got.tolist() == [b for _, b in cases]


def test_synth_bf16_rounding_agrees_with_torch():
    """The input generator's rounding is torch's binary32 -> bf16 (ties to even)."""
    rng = np.random.default_rng(14)
    v = (rng.standard_normal(50000) * 30).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.to_bf16_bits(v), ref)


def test_argument_errors():
    with pytest.raises(ValueError):
        oracle.rotate_quantize(np.zeros((2, 100), np.uint16), 64)    # cols % g != 0
    with pytest.raises(ValueError):
        oracle.rotate_quantize(np.zeros((2, 96), np.uint16), 96)     # g not a power of two


# ------------------------------------------------------------ FP8 (E4M3) --
# The FP8 variant of the quantized matmul (float8_e4m3fn, listed next to INT8 in
# the SDNQ README's feature list and SDNQConfig example): the same rotation and
# absmax with a /448 scale and OCP E4M3 codes, round half to even.

def torch_e4m3(v) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_e4m3_value(c) -> np.ndarray:
    return torch.from_numpy(np.asarray(c, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


FINITE_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def test_e4m3_decode_matches_torch_and_closed_form():
    got = oracle.e4m3_decode(FINITE_CODES)
    assert np.array_equal(got, torch_e4m3_value(FINITE_CODES))
    d = dict(zip(FINITE_CODES.tolist(), got.tolist()))
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0       # largest finite
    assert d[0x08] == 2.0 ** -6 and d[0x01] == 2.0 ** -9  # smallest normal, smallest subnormal
    assert d[0x38] == 1.0 and d[0x00] == 0.0


def test_e4m3_encode_matches_torch_on_codes_midpoints_and_neighbours():
    vals = np.sort(np.unique(np.abs(oracle.e4m3_decode(FINITE_CODES))))
    mids = (vals[:-1] + vals[1:]) / 2                        # exact in binary32
    pts = np.concatenate([vals, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                          np.nextafter(mids.astype(np.float32), np.float32(1e9))]).astype(np.float32)
    pts = pts[np.abs(pts) <= 448]
    pts = np.concatenate([pts, -pts])
    rng = np.random.default_rng(8)
    rnd = (rng.uniform(-1, 1, 20000) * np.exp2(rng.integers(-14, 9, 20000))).astype(np.float32)
    rnd = rnd[np.abs(rnd) <= 448]
    for v in (pts, rnd):
        assert np.array_equal(oracle.e4m3_encode(v), torch_e4m3(v))


def test_e4m3_ties_go_to_even_codes():
    # 1 + 1/16 lies halfway between 1 (0x38, even) and 1.125 (0x39); 3 * 2^-10
    # halfway between 2^-9 (0x01) and 2^-8 (0x02); 248 between 240 (0x77) and 256 (0x78).
    assert oracle.e4m3_encode(np.array([1.0625, 3 * 2.0 ** -10, 248.0], np.float32)).tolist() == [0x38, 0x02, 0x78]


@pytest.mark.parametrize("g", [1, 64, 256])
def test_fp8_quantization_matches_a_library_encoder_of_the_rotated_row(g):
    """Codes = torch's e4m3 encoding of fl32(y * fl32(448 / a)), y the oracle's
    (separately pinned) rotation; scales = fl32(a / 448)."""
    rng = np.random.default_rng(g)
    x = bf(rng.standard_normal((7, 512)) * np.exp2(rng.integers(-8, 8, (7, 1))))
    q, s = oracle.rotate_quantize_fp8(x, g)
    y = oracle.rotate(x, g)
    a = np.abs(y).max(axis=1).astype(np.float32)
    assert np.array_equal(s, (a / np.float32(448)).astype(np.float32))
    r = (np.float32(448) / a).astype(np.float32)
    t = np.clip((y * r[:, None]).astype(np.float32), -448, 448) + np.float32(0)  # exact zeros as +0
    assert np.array_equal(q, torch_e4m3(t))


@pytest.mark.parametrize("g", [64, 128, 256])
def test_fp8_quantization_error_bound_and_full_scale_code(g):
    rng = np.random.default_rng(3 + g)
    x = bf(synth.outlier_activations(rng, 16, 1024, channels=(5, 700)))
    q, s = oracle.rotate_quantize_fp8(x, g)
    y = oracle.rotate(x, g).astype(np.float64)
    deq = oracle.e4m3_decode(q) * s[:, None].astype(np.float64)
    # half an E4M3 ulp: 2^-4 relative for normals, 2^-10 of the row scale in the subnormal range
    bound = np.maximum(np.abs(y) * 2.0 ** -4, s[:, None] * 2.0 ** -10) * (1 + 1e-6) + 1e-30
    assert np.all(np.abs(deq - y) <= bound)
    assert np.all(np.any((q & 0x7F) == 0x7E, axis=1))     # every row reaches +-448


def test_fp8_exact_zeros_are_stored_as_positive_zero():
    """A block of -0 inputs rotates to zeros of both signs; every code is 0x00.
    A small negative value that rounds to zero keeps its sign (0x80)."""
    x = np.full((1, 256), 0x8000, np.uint16)                  # bf16 -0.0
    x[0, 0] = bf(np.array([1.0], np.float32))[0]
    x[0, 1] = bf(np.array([-1.0], np.float32))[0]            # y has exact zeros from cancellation
    q, s = oracle.rotate_quantize_fp8(x, 2)
    assert set(q[0, 2:].tolist()) == {0x00}
    x = bf(np.array([[448.0, -1e-4] + [0.0] * 14], np.float32))
    q, s = oracle.rotate_quantize_fp8(x, 1)
    assert q[0, 1] == 0x80 and q[0, 2] == 0x00


def test_fp8_all_zero_and_tiny_rows():
    x = np.zeros((2, 256), np.uint16)
    x[1, 3] = bf(np.array([2.0 ** -120], np.float32))[0]      # absmax below 2^-100
    x[1, 5] = bf(np.array([2.0 ** -121], np.float32))[0]
    q, s = oracle.rotate_quantize_fp8(x, 256)
    assert s[0] == 0 and np.all(q[0] == 0)
    # rotated values are (+-2^-120 +- 2^-121) / 16: magnitudes a = 3 * 2^-125 and a / 3
    a = np.float32(3 * 2.0 ** -125)
    assert s[1] == np.float32(a / np.float32(448))
    # the row is scaled by 2^100 (exact) before r = 448 / a, so 448 / 3 stays finite
    small = np.float32(np.float32(a * np.float32(2.0 ** 100) / 3) * np.float32(np.float32(448) / np.float32(a * np.float32(2.0 ** 100))))
    assert sorted(set((q[1] & 0x7F).tolist())) == sorted({0x7E, int(torch_e4m3([small])[0])})


def test_gemm_fp8_brute_force_python_loops():
    rng = np.random.default_rng(11)
    codes = FINITE_CODES
    a = rng.choice(codes, (5, 24))
    b = rng.choice(codes, (4, 24))
    c = oracle.gemm_fp8(a, b)
    av, bv = torch_e4m3_value(a), torch_e4m3_value(b)
    for i in range(5):
        for j in range(4):
            exact = sum(Fraction(float(av[i, t])) * Fraction(float(bv[j, t])) for t in range(24))
            assert Fraction(float(c[i, j])) == exact


def test_fp8_forward_dequant_and_lora_terms():
    inp = synth.make_linear(12, 512, 48, seed=4, lora_rank=16)
    qw, sw = oracle.rotate_quantize_fp8(inp["w"], 128)
    out = oracle.qlinear_forward_fp8(inp["x"], qw, sw, 128, inp["lora_a"], inp["lora_b"], 0.5)
    qx, sx = oracle.rotate_quantize_fp8(inp["x"], 128)
    assert np.array_equal(out["qx"], qx) and np.array_equal(out["sx"], sx)
    assert np.array_equal(out["acc"], oracle.gemm_fp8(qx, qw))
    base = (out["acc"].astype(np.float32) * (sx[:, None] * sw[None, :]).astype(np.float32)).astype(np.float32)
    assert np.array_equal(out["base"], base)
    xf = torch.from_numpy(synth.bf16_bits_to_f32(inp["x"]).astype(np.float64))
    la = torch.from_numpy(synth.bf16_bits_to_f32(inp["lora_a"]).astype(np.float64))
    lb = torch.from_numpy(synth.bf16_bits_to_f32(inp["lora_b"]).astype(np.float64))
    ref = base.astype(np.float64) + 0.5 * (xf @ la @ lb).numpy()
    assert np.array_equal(out["y"], oracle.bf16_from_f64(ref))
    # the quantized product approximates the unquantized fp64 product
    wf = synth.bf16_bits_to_f32(inp["w"]).astype(np.float64)
    exact = synth.bf16_bits_to_f32(inp["x"]).astype(np.float64) @ wf.T
    assert np.linalg.norm(base - exact) / np.linalg.norm(exact) < 0.06


@pytest.mark.parametrize("g", [1, 64, 256])
def test_fp8_backward_steps_against_independent_computations(g):
    """The FP8 input gradient, step by step: the fold and per-token E4M3 codes
    equal the (separately pinned) FP8 quantizer with the weight scales as the
    column scale and g = 1; the accumulators equal the exact sum of torch's E4M3
    values; dxbase equals the fp64 dense normalized block Hadamard product of
    fl32(fl32(acc) * s_dy) within binary32 rounding; dx is its bf16 rounding."""
    rng = np.random.default_rng(40 + g)
    m, n, k = 6, 320, 512
    dy = bf(rng.standard_normal((m, n)) * 1e-3)
    w = bf(rng.standard_normal((n, k)) * 0.02)
    qw, sw = oracle.rotate_quantize_fp8(w, g)
    out = oracle.qlinear_backward_input_fp8(dy, qw, sw, g)
    q2, s2 = oracle.rotate_quantize_fp8(dy, 1, col_scale=sw)
    assert np.array_equal(q2, out["qdy"]) and np.array_equal(s2.view(np.uint32), out["sdy"].view(np.uint32))
    av, wv = torch_e4m3_value(out["qdy"]), torch_e4m3_value(qw)
    for i, kk in [(0, 0), (2, 17), (5, k - 1), (3, 300)]:
        exact = sum(Fraction(float(av[i, j])) * Fraction(float(wv[j, kk])) for j in range(n))
        assert Fraction(float(out["acc"][i, kk])) == exact
    assert np.allclose(out["acc"], av @ wv, rtol=0, atol=1e-9 * np.abs(av @ wv).max())
    z = (out["acc"].astype(np.float32) * out["sdy"][:, None]).astype(np.float32).astype(np.float64)
    if g > 1:
        r = np.kron(np.eye(k // g), scipy.linalg.hadamard(g) / np.sqrt(g))
        ref = z @ r.T
        assert np.abs(out["dxbase"] - ref).max() <= 1e-5 * np.abs(ref).max()
    else:
        assert np.array_equal(out["dxbase"], z.astype(np.float32))
    assert np.array_equal(out["dx"], oracle.bf16_from_f64(out["dxbase"].astype(np.float64)))


def test_fp8_backward_lora_terms_against_torch_autograd():
    """The LoRA part of the FP8 dX and the LoRA gradients equal torch autograd
    (fp64) of sum(dY * ((x A) B * scale)) up to the final bf16 rounding."""
    d = synth.make_linear(20, 256, 128, seed=13, lora_rank=16, backward=True)
    scale = 0.5
    qw, sw = oracle.rotate_quantize_fp8(d["w"], 64)
    out = oracle.qlinear_backward_input_fp8(d["dy"], qw, sw, 64, d["x"], d["lora_a"], d["lora_b"], scale)
    t = lambda a, grad=False: torch.tensor(synth.bf16_bits_to_f32(a).astype(np.float64), requires_grad=grad)
    x, A, B, dY = t(d["x"], True), t(d["lora_a"], True), t(d["lora_b"], True), t(d["dy"])
    ((x @ A @ B * scale) * dY).sum().backward()
    for name, ref in (("grad_a", A.grad), ("grad_b", B.grad)):
        assert np.array_equal(out[name], oracle.bf16_from_f64(ref.numpy())), name
    assert np.array_equal(out["dx"], oracle.bf16_from_f64(out["dxbase"].astype(np.float64) + x.grad.numpy()))
    # with all-zero weight codes the LoRA term is the whole input gradient
    zero = oracle.qlinear_backward_input_fp8(d["dy"], np.zeros_like(qw), np.zeros_like(sw), 64, None, d["lora_a"],
                                            d["lora_b"], scale)
    assert np.array_equal(zero["dx"], oracle.bf16_from_f64(x.grad.numpy()))


def test_fp8_backward_approximates_unquantized_input_gradient():
    """dX ~ dY W (original bf16 weight) up to the E4M3 quantization error (3 mantissa
    bits: about 2^-5 relative per code, twice over)."""
    d = synth.make_linear(32, 768, 512, seed=14, backward=True)
    qw, sw = oracle.rotate_quantize_fp8(d["w"], 256)
    out = oracle.qlinear_backward_input_fp8(d["dy"], qw, sw, 256)
    ref = synth.bf16_bits_to_f32(d["dy"]).astype(np.float64) @ synth.bf16_bits_to_f32(d["w"]).astype(np.float64)
    dx = synth.bf16_bits_to_f32(out["dx"]).astype(np.float64)
    err = np.linalg.norm(dx - ref) / np.linalg.norm(ref)
    assert err < 0.06
    out8 = oracle.qlinear_backward_input(d["dy"], *oracle.rotate_quantize(d["w"], 256), 256)
    err8 = np.linalg.norm(synth.bf16_bits_to_f32(out8["dx"]).astype(np.float64) - ref) / np.linalg.norm(ref)
    assert err8 < err  # int8 keeps more bits than E4M3 on these rows


# ----------------------------------------------------------- weight gradient --
# Full fine-tuning through the quantized matmul ("SDNQ: SD.Next Quantization
# Engine": quantized matmul in the backward pass, full-parameter quantized
# training): dW = dY^T x contracts over the tokens, so both operands are
# quantized per feature along the tokens, rotated with block g along the tokens.

def _wgrad_inputs(m, n, k, seed):
    rng = np.random.default_rng(seed)
    dy = bf(rng.standard_normal((m, n)) * 1e-3)
    x = bf(synth.outlier_activations(rng, m, k, channels=(3, k - 5)))
    return dy, x


@pytest.mark.parametrize("g", [1, 64, 256])
def test_weight_grad_approximates_the_exact_product(g):
    dy, x = _wgrad_inputs(512, 48, 80, 21 + g)
    out = oracle.qlinear_weight_grad(dy, x, g)
    exact = synth.bf16_bits_to_f32(dy).astype(np.float64).T @ synth.bf16_bits_to_f32(x).astype(np.float64)
    got = synth.bf16_bits_to_f32(out["dw"]).astype(np.float64)
    assert np.linalg.norm(got - exact) / np.linalg.norm(exact) < 0.03


def test_weight_grad_rotation_along_tokens_cancels():
    """(dY^T H)(x^T H)^T = dY^T x: the unquantized rotated operands give the exact
    product up to binary32 rounding."""
    dy, x = _wgrad_inputs(256, 32, 48, 5)
    ry = oracle.rotate(np.ascontiguousarray(dy.T), 256).astype(np.float64)
    rx = oracle.rotate(np.ascontiguousarray(x.T), 256).astype(np.float64)
    exact = synth.bf16_bits_to_f32(dy).astype(np.float64).T @ synth.bf16_bits_to_f32(x).astype(np.float64)
    assert np.abs(ry @ rx.T - exact).max() <= 1e-5 * np.abs(exact).max()


def test_weight_grad_brute_force_on_codes():
    """Python loops over the per-feature codes of the transposed operands."""
    dy, x = _wgrad_inputs(64, 5, 6, 9)
    out = oracle.qlinear_weight_grad(dy, x, 64, intermediates=True)
    qd, sd = oracle.rotate_quantize(np.ascontiguousarray(dy.T), 64)
    qx, sx = oracle.rotate_quantize(np.ascontiguousarray(x.T), 64)
    assert np.array_equal(out["q_dy"], qd) and np.array_equal(out["q_x"], qx)
    for i in range(5):
        for j in range(6):
            acc = sum(int(qd[i, t]) * int(qx[j, t]) for t in range(64))
            v = np.float32(np.float32(acc) * np.float32(sd[i] * sx[j]))
            assert out["dw"][i, j] == oracle.bf16_from_f64(np.array([float(v)]))[0]


# ------------------------------------------------------ low-rank (SVD) split --
# Reading: randomized range finder with subspace iteration (Halko, Martinsson and
# Tropp 2011); factors bf16(W^T Q) [K, r] and bf16(Q^T) [r, N]; residual in
# binary32 against the rounded factors, then rotate + quantize.

def _exact_rank4_weight(n=96, k=128, seed=3):
    """W = U V^T with U, V entries in {-1, 0, 1} / 8: every entry is a multiple of
    2^-6 no larger than 4 * 2^-6, so W is exactly representable in bf16 and has
    rank 4 (checked)."""
    rng = np.random.default_rng(seed)
    u = rng.integers(-1, 2, (n, 4)).astype(np.float64) / 8
    v = rng.integers(-1, 2, (k, 4)).astype(np.float64) / 8
    w = u @ v.T
    assert np.linalg.matrix_rank(w) == 4
    bits = oracle.bf16_from_f64(w)
    assert np.array_equal(synth.bf16_bits_to_f32(bits).astype(np.float64), w)
    return bits, w


@pytest.mark.parametrize("steps", [0, 3])
def test_svd_recovers_an_exactly_low_rank_weight(steps):
    """range(W omega) = range(W) for a Gaussian omega when rank(W) <= r, so the
    projection Q Q^T W is W itself up to fp64 rounding, with or without iterations."""
    bits, w = _exact_rank4_weight()
    omega = np.random.default_rng(1).standard_normal((w.shape[1], 6))
    q = oracle.svd_lowrank_split(bits, omega, steps)["q"]
    assert np.abs(w - q @ (q.T @ w)).max() <= 1e-12 * np.abs(w).max()


def test_svd_q_is_orthonormal_and_the_residual_orthogonal_to_it():
    d = synth.make_config("tiny")
    w = synth.bf16_bits_to_f32(d["w"]).astype(np.float64)
    omega = np.random.default_rng(2).standard_normal((w.shape[1], 16))
    q = oracle.svd_lowrank_split(d["w"], omega, 2)["q"]
    assert q.shape == (w.shape[0], 16)
    assert np.abs(q.T @ q - np.eye(16)).max() <= 1e-12
    assert np.abs(q.T @ (w - q @ (q.T @ w))).max() <= 1e-12 * np.abs(w).max()


def _planted(n, k, lead, decay, seed, planted=12):
    rng = np.random.default_rng(seed)
    return synth.to_bf16_bits(synth.planted_lowrank_weight(rng, n, k, planted=planted, lead=lead, decay=decay))


def test_svd_with_a_spectral_gap_finds_the_top_singular_subspace():
    """Eckart-Young: no rank-r matrix is closer to W in Frobenius norm than the
    truncated SVD (computed here with LAPACK).  With a clear gap after the planted
    directions the subspace iteration reaches that optimum and that subspace."""
    bits = _planted(256, 320, lead=20.0, decay=0.9, seed=4, planted=8)
    w = synth.bf16_bits_to_f32(bits).astype(np.float64)
    u, s, _ = np.linalg.svd(w)
    assert s[7] > 5 * s[8]
    omega = np.random.default_rng(5).standard_normal((w.shape[1], 8))
    q = oracle.svd_lowrank_split(bits, omega, 8)["q"]
    err = np.linalg.norm(w - q @ (q.T @ w))
    opt = np.sqrt((s[8:] ** 2).sum())
    assert opt <= err <= opt * (1 + 1e-9)
    assert np.abs(q @ q.T - u[:, :8] @ u[:, :8].T).max() <= 1e-8


def test_svd_subspace_iterations_approach_the_optimum():
    """Without a clear gap the range finder alone (steps = 0) is measurably worse
    than the truncated SVD; the iterations close most of that distance."""
    bits = _planted(256, 320, lead=1.5, decay=0.85, seed=6, planted=24)
    w = synth.bf16_bits_to_f32(bits).astype(np.float64)
    s = np.linalg.svd(w, compute_uv=False)
    opt = np.sqrt((s[16:] ** 2).sum())
    omega = np.random.default_rng(7).standard_normal((w.shape[1], 16))
    errs = []
    for steps in (0, 1, 2, 4, 8):
        q = oracle.svd_lowrank_split(bits, omega, steps)["q"]
        errs.append(np.linalg.norm(w - q @ (q.T @ w)))
    assert errs[0] > 1.05 * opt
    assert all(b < a for a, b in zip(errs, errs[1:]))
    assert errs[-1] <= 1.005 * opt


def test_svd_factors_and_residual_add_back_to_the_weight():
    """svd_b^T svd_a^T is the projection Q Q^T W up to the bf16 rounding of the two
    factors, and the binary32 residual is W minus exactly that rounded product
    (one rounding to binary32)."""
    d = synth.make_config("tiny")
    w = synth.bf16_bits_to_f32(d["w"]).astype(np.float64)
    omega = np.random.default_rng(8).standard_normal((w.shape[1], 32))
    out = oracle.svd_lowrank_split(d["w"], omega, 8)
    a = synth.bf16_bits_to_f32(out["svd_a"]).astype(np.float64)
    b = synth.bf16_bits_to_f32(out["svd_b"]).astype(np.float64)
    assert a.shape == (w.shape[1], 32) and b.shape == (32, w.shape[0])
    lr = b.T @ a.T
    proj = out["q"] @ (out["q"].T @ w)
    assert np.linalg.norm(lr - proj) <= 2 ** -7 * np.linalg.norm(proj)
    r = out["residual"].astype(np.float64)
    exact = w - lr
    half_ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64) / 2
    assert np.all(np.abs(r - exact) <= half_ulp + 1e-300)


def test_rotate_quantize_f32_agrees_with_the_bf16_path_on_bf16_values():
    d = synth.make_config("tiny")
    for g in (1, 64, 256):
        q1, s1 = oracle.rotate_quantize(d["w"], g)
        q2, s2 = oracle.rotate_quantize_f32(synth.bf16_bits_to_f32(d["w"]), g)
        assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_rotate_quantize_f32_keeps_binary32_precision():
    """Values that bf16 cannot hold: the codes stay within half a step of the exact
    rotated values (fp64 Sylvester product), so the low mantissa bits are used."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((8, 256)) * (1 + 2.0 ** -12)).astype(np.float32)
    q, s = oracle.rotate_quantize_f32(x, 256)
    h = scipy.linalg.hadamard(256).astype(np.float64) / 16.0
    y = x.astype(np.float64) @ h.T
    for i in range(8):
        assert s[i] == np.float32(np.abs(y[i]).max().astype(np.float32) / np.float32(127)) or \
            abs(float(s[i]) - np.abs(y[i]).max() / 127) <= 1e-6 * float(s[i])
        assert np.abs(q[i] * float(s[i]) - y[i]).max() <= 0.5 * float(s[i]) * (1 + 1e-5)
    # a bf16 truncation of the inputs moves some code
    qt, _ = oracle.rotate_quantize(synth.to_bf16_bits(x), 256)
    assert not np.array_equal(q, qt)


def test_svd_split_lowers_the_forward_error_on_a_planted_weight():
    """With a few dominant singular directions, quantizing only the residual (and
    adding the bf16 factors back) approximates x W^T better than quantizing W."""
    c = synth.CONFIGS["tiny"]
    x = synth.make_config("tiny")["x"]
    bits = _planted(c.n, c.k, lead=20.0, decay=0.6, seed=10, planted=8)
    w = synth.bf16_bits_to_f32(bits).astype(np.float64)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    exact = xf @ w.T
    qw, sw = oracle.rotate_quantize(bits, 256)
    plain = synth.bf16_bits_to_f32(oracle.qlinear_forward(x, qw, sw, 256)["y"]).astype(np.float64)
    omega = np.random.default_rng(11).standard_normal((c.k, 32))
    sv = oracle.svd_quantize_weight(bits, 256, omega, 8)
    y = oracle.qlinear_forward(x, sv["qw"], sv["sw"], 256, sv["svd_a"], sv["svd_b"], 1.0)["y"]
    svd = synth.bf16_bits_to_f32(y).astype(np.float64)
    e_plain = np.linalg.norm(plain - exact) / np.linalg.norm(exact)
    e_svd = np.linalg.norm(svd - exact) / np.linalg.norm(exact)
    assert e_svd < 0.5 * e_plain


# ---------------------------------------------------- int8 attention (QK^T) --
# Reading: per-token int8 Q and K rotated along the head dimension with block
# min(g, D); K smoothed by its per-channel mean over the key tokens; fp64 softmax
# and P V; grouped-query heads h -> h // (Hq / Hkv); top-left causal mask.

def _attn_inputs(b, hq, hkv, sq, sk, d, seed):
    rng = np.random.default_rng(seed)
    q = synth.to_bf16_bits(rng.standard_normal((b, hq, sq, d)).astype(np.float32))
    k = synth.to_bf16_bits((rng.standard_normal((b, hkv, sk, d)) + rng.standard_normal((b, hkv, 1, d)) * 3)
                           .astype(np.float32))
    v = synth.to_bf16_bits(rng.standard_normal((b, hkv, sk, d)).astype(np.float32))
    return q, k, v


def _f64(bits):
    return torch.from_numpy(synth.bf16_bits_to_f32(bits).astype(np.float64))


@pytest.mark.parametrize("causal", [False, True])
def test_attention_core_is_sdpa_on_the_dequantized_codes(causal):
    """Softmax, P V, the scale, the causal mask and the head grouping, against
    torch's scaled_dot_product_attention in fp64 on q_codes * s_q, k_codes * s_k
    (the rotation leaves every score q . k unchanged, so SDPA may see the
    rotated, dequantized operands)."""
    q, k, v = _attn_inputs(2, 4, 2, 40, 56, 64, 12)
    r = oracle.attention_int8(q, k, v, causal, 0.3, True, 64, intermediates=True)
    qh = torch.from_numpy(r["q_codes"].astype(np.float64) * r["q_scales"].astype(np.float64)[..., None])
    kh = torch.from_numpy(r["k_codes"].astype(np.float64) * r["k_scales"].astype(np.float64)[..., None])
    ref = torch.nn.functional.scaled_dot_product_attention(qh, kh, _f64(v), is_causal=causal, scale=0.3,
                                                           enable_gqa=True).numpy()
    assert np.abs(r["o"] - ref).max() <= 1e-12


def test_attention_causal_brute_force():
    q, k, v = _attn_inputs(1, 1, 1, 5, 7, 64, 13)
    r = oracle.attention_int8(q, k, v, True, None, False, 64, intermediates=True)
    vf = synth.bf16_bits_to_f32(v)[0, 0].astype(np.float64)
    for i in range(5):
        s = []
        for j in range(i + 1):
            acc = sum(int(r["q_codes"][0, 0, i, t]) * int(r["k_codes"][0, 0, j, t]) for t in range(64))
            s.append(acc * float(r["q_scales"][0, 0, i]) * float(r["k_scales"][0, 0, j]) / 8.0)
        mx = max(s)
        p = [np.exp(x - mx) for x in s]
        o = sum(p[j] * vf[j] for j in range(i + 1)) / sum(p)
        assert np.abs(o - r["o"][0, 0, i]).max() <= 1e-12


def test_attention_k_mean_is_the_exact_mean_rounded_once():
    """Values n/16 with |n| < 128 (exact in bf16), 150 tokens: the mean is the
    exact rational mean rounded once to binary32 (here fp64's division is exact
    enough that numpy's rounding of it is the same number)."""
    rng = np.random.default_rng(14)
    kf = rng.integers(-127, 128, (1, 2, 150, 64)).astype(np.float64) / 16
    k = oracle.bf16_from_f64(kf)
    assert np.array_equal(synth.bf16_bits_to_f32(k).astype(np.float64), kf)
    mean = oracle.attention_k_mean(k)
    for h in range(2):
        for c in range(64):
            exact = Fraction(int(round(kf[0, h, :, c].sum() * 16)), 16 * 150)
            assert mean[0, h, c] == np.float32(float(exact))


def _nearest_f32_brute(exact: Fraction) -> np.float32:
    """Binary32 nearest to a rational, ties to even, by comparing the neighbours of
    a first guess exactly."""
    f = np.float32(float(exact))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda x: (abs(Fraction(float(x)) - exact), int(np.array(x).view(np.uint32)) & 1))


def test_attention_k_mean_does_not_depend_on_a_summation_order():
    """Keys 2^60, 1, -2^60 repeated over 192 tokens: any binary64 running sum
    loses the ones (2^60 + 1 rounds to 2^60), whatever the blocking; the exact
    mean is 64 / 192 = 1/3, rounded once."""
    v = np.zeros((1, 1, 192, 16))
    v[0, 0, 0::3] = 2.0 ** 60
    v[0, 0, 1::3] = 1.0
    v[0, 0, 2::3] = -(2.0 ** 60)
    v[0, 0, :, 5] = np.roll(v[0, 0, :, 5], 1)          # another token order, the same mean
    mean = oracle.attention_k_mean(oracle.bf16_from_f64(v))
    assert np.all(mean == _nearest_f32_brute(Fraction(1, 3)))


def test_attention_k_mean_rounds_ties_to_even():
    """16 tokens (14 ones, a 2, one small key): the exact means 1 + 2^-24 and
    1 + 3 * 2^-24 lie halfway between binary32 neighbours; ties go to the even
    significand (1 and 1 + 2^-22)."""
    v = np.ones((1, 1, 16, 2))
    v[0, 0, 14] = 2.0
    v[0, 0, 15, 0] = 2.0 ** -20
    v[0, 0, 15, 1] = 3 * 2.0 ** -20
    mean = oracle.attention_k_mean(oracle.bf16_from_f64(v))
    assert mean[0, 0, 0] == np.float32(1.0)
    assert mean[0, 0, 1] == np.float32(1.0 + 2.0 ** -22)


def test_attention_k_mean_random_and_subnormal_keys_against_exact_rationals():
    """Keys of every magnitude class, from bf16 subnormals up to 2^100, against the
    exact Fraction mean rounded by comparing neighbours."""
    rng = np.random.default_rng(21)
    s, d = 80, 24
    mag = 2.0 ** rng.integers(-140, 100, (s, d))
    kf = rng.standard_normal((s, d)) * mag
    kf[:, :4] = rng.integers(-255, 256, (s, 4)) * 2.0 ** -133    # bf16 subnormals (and zeros)
    kf[:, 4] = rng.standard_normal(s) * 2.0 ** -128                # around the normal boundary
    k = oracle.bf16_from_f64(kf.reshape(1, 1, s, d))
    exact_keys = synth.bf16_bits_to_f32(k).astype(np.float64)[0, 0]
    mean = oracle.attention_k_mean(k)[0, 0]
    for c in range(d):
        exact = sum((Fraction(float(x)) for x in exact_keys[:, c]), Fraction(0)) / s
        want = _nearest_f32_brute(exact)
        assert mean[c].view(np.uint32) == want.view(np.uint32) or (want == 0 and mean[c] == 0), c


def test_attention_smoothing_ignores_a_key_offset_common_to_all_tokens():
    """Adding the same per-channel constant to every key token leaves the smoothed
    K, so its codes and the output, unchanged.  With 64 tokens of values n/16 and
    integer offsets every step is exact (the mean divides by a power of two), so
    the invariance holds bit for bit."""
    rng = np.random.default_rng(15)
    kf = rng.integers(-64, 64, (1, 2, 64, 64)).astype(np.float64) / 16
    off = rng.integers(-7, 8, (1, 2, 1, 64)).astype(np.float64)
    q, _, v = _attn_inputs(1, 2, 2, 24, 64, 64, 16)
    a = oracle.attention_int8(q, oracle.bf16_from_f64(kf), v, False, None, True, 64, intermediates=True)
    b = oracle.attention_int8(q, oracle.bf16_from_f64(kf + off), v, False, None, True, 64, intermediates=True)
    assert np.array_equal(a["k_codes"], b["k_codes"]) and np.array_equal(a["k_scales"], b["k_scales"])
    assert np.array_equal(a["out"], b["out"])
    c = oracle.attention_int8(q, oracle.bf16_from_f64(kf + off), v, False, None, False, 64, intermediates=True)
    assert not np.array_equal(a["k_codes"], c["k_codes"])


def test_attention_gqa_equals_repeated_key_value_heads():
    q, k, v = _attn_inputs(1, 6, 2, 30, 40, 64, 17)
    a = oracle.attention_int8(q, k, v, True, None, True, 64)["out"]
    b = oracle.attention_int8(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), True, None, True, 64)["out"]
    assert np.array_equal(a, b)


def test_attention_approximates_exact_attention_and_rotation_and_smoothing_help():
    """The method's premise on the outlier workload: against fp64 SDPA on the bf16
    inputs, the Hadamard rotation lowers the error and K smoothing lowers it
    further; the full method stays within 3 %."""
    d = synth.make_attention("attn_tiny")
    c = synth.ATTENTION_CONFIGS["attn_tiny"]
    ref = torch.nn.functional.scaled_dot_product_attention(_f64(d["q"]), _f64(d["k"]), _f64(d["v"]),
                                                           is_causal=c.causal, enable_gqa=True).numpy()

    def err(g, smooth):
        o = synth.bf16_bits_to_f32(oracle.attention_int8(d["q"], d["k"], d["v"], c.causal, None, smooth, g)["out"])
        return np.linalg.norm(o.astype(np.float64) - ref) / np.linalg.norm(ref)
    e_plain, e_rot, e_full = err(1, False), err(256, False), err(256, True)
    assert e_full < e_rot < e_plain
    assert e_full < 0.03


@pytest.mark.parametrize("d", [64, 128])
def test_attention_rotation_block_is_the_whole_head(d):
    """g = 256 rotates each head row as one block of D (min(g, D)): a one-hot row
    becomes flat, so all D codes are +-127; with g = 1 only one code is nonzero."""
    q = np.zeros((1, 1, 2, d), np.float64)
    q[0, 0, 0, 3] = 1.0
    q[0, 0, 1, d - 1] = -2.0
    bits = oracle.bf16_from_f64(q)
    codes, _ = oracle.attention_prep(bits, 256)
    assert np.all(np.abs(codes[0, 0]) == 127)
    codes1, _ = oracle.attention_prep(bits, 1)
    assert np.count_nonzero(codes1[0, 0, 0]) == 1 and np.count_nonzero(codes1[0, 0, 1]) == 1
