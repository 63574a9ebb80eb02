"""GPU parity of the low-rank (SVD) split against the oracle.

What is unique and compared:
  * the span of Q (the projector Q Q^T), to fp64 rounding;
  * the bf16 factors: Q is an orthonormal basis of that span, fixed up to the
    sign of each column (CholeskyQR here, Householder QR in the oracle), so
    svd_a[:, c] and svd_b[c, :] are compared up to one sign per c;
  * the binary32 residual, to one binary32 ulp (its fp64 sum may round the other
    way where the two sums differ in their last bits);
  * the codes and scales of the residual, bit for bit, against the oracle's
    quantizer applied to the GPU's own residual (the quantizer's decisions are
    taken on identical binary32 inputs on both sides);
  * the layer's output with the factors as the LoRA term, within 1e-2 relative L2.
"""
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
    oracle.set_num_threads(16)
    yield
    torch.cuda.synchronize()


def d_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def h_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_split(w_bits, omega, g, steps):
    n, k = w_bits.shape
    r = omega.shape[1]
    say(f"  svd split n={n} k={k} rank={r} steps={steps} g={g}")
    ws = torch.empty(h.sdnq_svd_workspace_bytes(n, k, r), dtype=torch.uint8, device=DEV)
    qw, sw, a, b = h.sdnq_svd_quantize_weight(d_bf16(w_bits), g, torch.from_numpy(omega).to(DEV), steps,
                                              workspace=ws)
    torch.cuda.synchronize()
    res = ws[: n * k * 4].view(torch.float32).view(n, k).cpu().numpy()
    qo = h.sdnq_svd_workspace_q_offset(n, k, r)
    q = ws[qo: qo + n * r * 8].view(torch.float64).view(n, r).cpu().numpy()
    return dict(qw=qw.cpu().numpy(), sw=sw.cpu().numpy(), svd_a=h_bits(a), svd_b=h_bits(b), residual=res, q=q)


def column_signs(got_a, ref_a):
    """+1 / -1 per column c such that got_a[:, c] = sign * ref_a[:, c] (in value)."""
    ga = synth.bf16_bits_to_f32(got_a).astype(np.float64)
    ra = synth.bf16_bits_to_f32(ref_a).astype(np.float64)
    return np.where((ga * ra).sum(axis=0) >= 0, 1.0, -1.0)


def check_against_oracle(w_bits, omega, g, steps, proj_tol=1e-8):
    got = run_split(w_bits, omega, g, steps)
    ref = oracle.svd_quantize_weight(w_bits, g, omega.astype(np.float64), steps)
    n, k = w_bits.shape
    r = omega.shape[1]
    assert np.all(np.isfinite(got["q"])) and np.all(np.isfinite(got["residual"]))
    # span of Q
    qg, qr = got["q"], ref["q"]
    assert np.abs(qg.T @ qg - np.eye(r)).max() <= 1e-10
    proj = np.abs(qg @ qg.T - qr @ qr.T).max()
    say(f"    projector max diff {proj:.2e}")
    assert proj <= proj_tol
    # factors up to one sign per column
    sg = column_signs(got["svd_a"], ref["svd_a"])
    flip_a = np.where(sg < 0, 0x8000, 0).astype(np.uint16)
    a_ref = ref["svd_a"] ^ flip_a[None, :]
    b_ref = ref["svd_b"] ^ flip_a[:, None]
    diff_a = np.count_nonzero(got["svd_a"] != a_ref)
    diff_b = np.count_nonzero(got["svd_b"] != b_ref)
    say(f"    factor elements differing: svd_a {diff_a}/{a_ref.size}, svd_b {diff_b}/{b_ref.size}")
    assert diff_a <= 1e-4 * a_ref.size and diff_b <= 1e-4 * b_ref.size
    # residual within one binary32 ulp where the factors agree
    same_rows = np.all(got["svd_b"] == b_ref, axis=0)      # rows n of the weight with equal svd_b
    same_cols = np.all(got["svd_a"] == a_ref, axis=1)      # columns k with equal svd_a
    rg = got["residual"][np.ix_(same_rows, same_cols)].astype(np.float64)
    ro = ref["residual"][np.ix_(same_rows, same_cols)].astype(np.float64)
    ulp = np.spacing(np.abs(ref["residual"][np.ix_(same_rows, same_cols)])).astype(np.float64)
    assert np.all(np.abs(rg - ro) <= ulp)
    say(f"    residual elements differing: {np.count_nonzero(rg != ro)}/{rg.size}")
    # the quantizer on the GPU's own residual: bit for bit
    q_o, s_o = oracle.rotate_quantize_f32(got["residual"], g)
    bad = np.nonzero(np.any(got["qw"] != q_o, axis=1))[0]
    assert bad.size == 0, f"codes differ in rows {bad[:8]}"
    assert np.array_equal(got["sw"].view(np.uint32), s_o.view(np.uint32)), "scales"
    return got, ref


def tiny_planted(n=512, k=512, seed=1, lead=6.0):
    rng = np.random.default_rng(seed)
    w = synth.to_bf16_bits(synth.planted_lowrank_weight(rng, n, k, lead=lead))
    return w


@pytest.mark.parametrize("g", [1, 64, 128, 256])
def test_split_tiny_all_blocks(g):
    w = tiny_planted()
    omega = synth.gaussian_test_matrix(np.random.default_rng(2), 512, 32)
    check_against_oracle(w, omega, g, 8)


@pytest.mark.parametrize("rank,steps", [(16, 0), (16, 3), (64, 8), (32, 0)])
def test_split_ranks_and_steps(rank, steps):
    w = tiny_planted(seed=3)
    omega = synth.gaussian_test_matrix(np.random.default_rng(4), 512, rank)
    check_against_oracle(w, omega, 256, steps)


def test_split_ragged_tiles():
    """n and k not multiples of the 64-wide tiles, k not a multiple of 256 (g = 64)."""
    w = tiny_planted(n=208, k=320, seed=5)
    omega = synth.gaussian_test_matrix(np.random.default_rng(6), 320, 16)
    check_against_oracle(w, omega, 64, 4)


def test_split_exactly_low_rank_weight():
    """An exactly rank-4 bf16 weight with rank 16: W omega is rank-deficient, the
    shifted CholeskyQR leaves the missing directions near zero, and the projection
    still reproduces W; the residual is then only the bf16 rounding of the factors."""
    rng = np.random.default_rng(7)
    u = rng.integers(-1, 2, (256, 4)).astype(np.float64) / 8
    v = rng.integers(-1, 2, (256, 4)).astype(np.float64) / 8
    wf = u @ v.T
    w = oracle.bf16_from_f64(wf)
    assert np.array_equal(synth.bf16_bits_to_f32(w).astype(np.float64), wf)
    omega = synth.gaussian_test_matrix(np.random.default_rng(8), 256, 16)
    got = run_split(w, omega, 256, 2)
    assert np.all(np.isfinite(got["q"])) and np.all(np.isfinite(got["residual"]))
    q = got["q"]
    assert np.abs(wf - q @ (q.T @ wf)).max() <= 1e-9 * np.abs(wf).max()
    assert np.linalg.norm(got["residual"]) <= 2 ** -7 * np.linalg.norm(wf)
    q_o, s_o = oracle.rotate_quantize_f32(got["residual"], 256)
    assert np.array_equal(got["qw"], q_o) and np.array_equal(got["sw"].view(np.uint32), s_o.view(np.uint32))


def test_split_full_size_and_forward():
    """The workload: W [3072, 3072] with planted directions, rank 32, 8 steps, g = 256;
    then the layer on x [4096, 3072] with the factors as the LoRA term (scale 1),
    checked on sampled token rows, and its error against the exact x W^T compared
    with the plain int8 layer's."""
    c = synth.CONFIGS["svd"]
    inp = synth.make_config("svd")
    got, ref = check_against_oracle(inp["w"], inp["omega"], 256, c.extra["steps"], proj_tol=1e-6)
    m = c.m
    ws = torch.empty(h.sdnq_workspace_bytes(m, c.n, c.k, c.extra["rank"], False), dtype=torch.uint8, device=DEV)
    x = d_bf16(inp["x"])
    y = h.sdnq_qlinear_forward(x, torch.from_numpy(got["qw"]).to(DEV), torch.from_numpy(got["sw"]).to(DEV), 256,
                               d_bf16(got["svd_a"]), d_bf16(got["svd_b"]), 1.0, workspace=ws)
    qw_p, sw_p = h.sdnq_rotate_quantize_weight(d_bf16(inp["w"]), 256)
    y_plain = h.sdnq_qlinear_forward(x, qw_p, sw_p, 256)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(m - 8, m), rng.choice(m, 48, replace=False)]))
    yo = oracle.qlinear_forward(inp["x"][rows], ref["qw"], ref["sw"], 256, ref["svd_a"], ref["svd_b"], 1.0,
                                intermediates=False)["y"]
    yg = synth.bf16_bits_to_f32(h_bits(y)[rows]).astype(np.float64)
    yr = synth.bf16_bits_to_f32(yo).astype(np.float64)
    err = np.linalg.norm(yg - yr) / np.linalg.norm(yr)
    say(f"    forward rel-L2 vs oracle {err:.3e}")
    assert err < 1e-2
    exact = synth.bf16_bits_to_f32(inp["x"][rows]).astype(np.float64) @ \
        synth.bf16_bits_to_f32(inp["w"]).astype(np.float64).T
    e_svd = np.linalg.norm(yg - exact) / np.linalg.norm(exact)
    e_plain = np.linalg.norm(synth.bf16_bits_to_f32(h_bits(y_plain)[rows]).astype(np.float64) - exact) / \
        np.linalg.norm(exact)
    say(f"    error vs exact: svd {e_svd:.3e}, plain int8 {e_plain:.3e}")
    assert e_svd < e_plain
