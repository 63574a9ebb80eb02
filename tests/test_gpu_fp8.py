"""GPU parity of the FP8 (E4M3) variant against the CPU oracle, through the C ABI.

Bars: E4M3 codes and fp32 scales bit-exact; the MFMA GEMM within 2^-9 of
sum |a b| of the exact fp64 sum.  The fp8 dot-product unit does not round like a
sequential fp32 sum: on random codes spanning the whole E4M3 range (2^-9 .. 448,
so products over 35 binades) its error reached 3.2e-4 of sum |a b|, where a
sequential fp32 sum stays near 5e-7; it does not flush subnormal codes.  A layout
or indexing slip gives errors of order one.  bf16 outputs within 1e-2 relative L2
(the layer's stated tolerance).
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
FINITE_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def say(*a):
    print(*a, flush=True)


def d_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def d(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def h_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def rel_l2(got_bits, ref_bits):
    g = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    r = synth.bf16_bits_to_f32(ref_bits).astype(np.float64)
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    h.lib()
    yield
    torch.cuda.synchronize()


def assert_rq8_exact(x_bits, g, col_scale=None):
    say(f"  rotate_quantize_act_fp8 {x_bits.shape} g={g} colscale={col_scale is not None}")
    q, s = h.sdnq_rotate_quantize_act_fp8(d_bf16(x_bits), g, None if col_scale is None else d(col_scale))
    torch.cuda.synchronize()
    qo, so = oracle.rotate_quantize_fp8(x_bits, g, col_scale)
    q = q.cpu().numpy()
    bad = np.nonzero(np.any(q != qo, axis=1))[0]
    if bad.size:
        y = oracle.rotate(x_bits[bad[:4]], g, col_scale)
        for n, row in enumerate(bad[:4]):
            cols = np.nonzero(q[row] != qo[row])[0][:6]
            a = np.float32(np.abs(y[n]).max())
            r = np.float32(np.float32(448) / a)
            say(f"    row {row} cols {cols.tolist()} gpu {q[row, cols].tolist()} oracle {qo[row, cols].tolist()} "
                f"y*r {[float(np.float32(y[n, c] * r)) for c in cols]} a {float(a)!r}")
    assert bad.size == 0, f"codes differ in rows {bad[:8]}"
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32)), "scales differ"


@pytest.mark.parametrize("g,m,k", [(256, 64, 512), (256, 37, 3072), (128, 19, 1152), (64, 33, 320),
                                   (1, 40, 272), (256, 3, 40960), (64, 2, 65536), (256, 9000, 3840),
                                   (256, 7, 1536), (128, 5, 10240), (64, 9, 1536), (1, 3, 10240),
                                   (256, 2, 98304), (64, 3, 133120)])
def test_fp8_rotate_quantize_bit_exact(g, m, k):
    assert_rq8_exact(synth.make_linear(m, k, 16, seed=300 + g + m)["x"], g)


@pytest.mark.parametrize("k", [272, 1536, 3072, 10240])
def test_fp8_rotate_quantize_column_scale_bit_exact(k):
    rng = np.random.default_rng(12)
    dy = synth.to_bf16_bits(rng.standard_normal((29, k)).astype(np.float32) * 1e-3)
    cs = (rng.uniform(0.5, 2.0, k) * 1e-3).astype(np.float32)
    assert_rq8_exact(dy, 1, cs)


@pytest.mark.parametrize("k", [512, 1536])   # 4 and 8 lanes per superblock
@pytest.mark.parametrize("g", [1, 64, 128, 256])
def test_fp8_rotate_quantize_stress_rows(g, k):
    rng = np.random.default_rng(9)
    rows = [np.zeros(k, np.float32)]
    r = rng.standard_normal(k).astype(np.float32); r[17] = 1e30; rows.append(r)
    rows.append((rng.standard_normal(k) * 1e-38).astype(np.float32))      # a below 2^-100
    rows.append((rng.standard_normal(k) * 1e-36).astype(np.float32))
    r = np.zeros(k, np.float32); r[300] = 1.0; rows.append(r)              # one-hot: every code +-448
    rows.append(np.full(k, 3.0, np.float32))
    # values that land on E4M3 ties after scaling: a = 448, r = 1
    codes = FINITE_CODES[(FINITE_CODES & 0x7F) < 0x7E]
    v = np.sort(np.abs(oracle.e4m3_decode(codes)))
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    r = np.resize(np.where(rng.random(mids.size) < 0.5, mids, -mids), k).astype(np.float32); r[0] = 448.0
    rows.append(r)
    x = synth.to_bf16_bits(np.stack(rows))
    assert_rq8_exact(x, g)


def test_fp8_weight_prep_bit_exact():
    w = synth.make_config("tiny")["w"]
    qw, sw = h.sdnq_rotate_quantize_weight_fp8(d_bf16(w), 256)
    torch.cuda.synchronize()
    qo, so = oracle.rotate_quantize_fp8(w, 256)
    assert np.array_equal(qw.cpu().numpy(), qo)
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), so.view(np.uint32))


def abs_sum(a, b):
    return np.abs(oracle.e4m3_decode(a)) @ np.abs(oracle.e4m3_decode(b)).T + 1e-30


# 4000 x 3840 selects 256-column tiles, 4000 x 5104 320-column tiles, the small
# grids 192-column tiles (on 256 CUs)
@pytest.mark.parametrize("m,n,k", [(64, 512, 512), (300, 640, 400), (1, 16, 16), (257, 272, 4096),
                                   (40, 48, 144), (4000, 3840, 80), (4000, 5104, 80)])
def test_fp8_gemm_within_accumulation_bound(m, n, k):
    rng = np.random.default_rng(m + n + k)
    a = rng.choice(FINITE_CODES, (m, k))
    b = rng.choice(FINITE_CODES, (n, k))
    say(f"  gemm_fp8_f32 m={m} n={n} k={k}")
    c = h.sdnq_gemm_fp8_f32(d(a), d(b))
    torch.cuda.synchronize()
    exact = oracle.gemm_fp8(a, b)
    err = np.abs(c.cpu().numpy().astype(np.float64) - exact) / abs_sum(a, b)
    say(f"    max error / sum|ab| = {err.max():.3e}")
    assert np.all(err <= 2.0 ** -9)


def forward8_case(m, k, n, g, rank=0, seed=0, scale=1.0):
    inp = synth.make_linear(m, k, n, seed=seed, lora_rank=rank)
    qwo, swo = oracle.rotate_quantize_fp8(inp["w"], g)
    say(f"  qlinear_forward_fp8 m={m} k={k} n={n} g={g} rank={rank}")
    qw, sw = h.sdnq_rotate_quantize_weight_fp8(d_bf16(inp["w"]), g)
    la = d_bf16(inp["lora_a"]) if rank else None
    lb = d_bf16(inp["lora_b"]) if rank else None
    ws = torch.empty(h.sdnq_workspace_bytes(m, n, k, rank, False), dtype=torch.uint8, device=DEV)
    y = h.sdnq_qlinear_forward_fp8(d_bf16(inp["x"]), qw, sw, g, la, lb, scale, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(qw.cpu().numpy(), qwo)
    ref = oracle.qlinear_forward_fp8(inp["x"], qwo, swo, g, inp.get("lora_a"), inp.get("lora_b"), scale)
    qx = ws[: m * k].view(m, k).cpu().numpy()
    assert np.array_equal(qx, ref["qx"]), "activation codes"
    return h_bits(y), ref


@pytest.mark.parametrize("g", [1, 64, 128, 256])
@pytest.mark.parametrize("m,k,n", [(64, 512, 512), (300, 768, 640), (7, 256, 16)])
def test_fp8_forward(m, k, n, g):
    y, ref = forward8_case(m, k, n, g, seed=m + g)
    err = rel_l2(y, ref["y"])
    say(f"    rel-L2 {err:.3e}, bf16 outputs equal: {np.mean(y == ref['y']):.4f}")
    assert err < REL_L2


@pytest.mark.parametrize("g,rank,scale", [(64, 32, 1.0), (256, 16, 2.0), (128, 64, 0.5)])
def test_fp8_forward_with_lora(g, rank, scale):
    y, ref = forward8_case(300, 768, 640, g, rank=rank, seed=rank + g, scale=scale)
    err = rel_l2(y, ref["y"])
    say(f"    rel-L2 {err:.3e}")
    assert err < REL_L2


@pytest.mark.parametrize("m,n", [(4000, 3840), (4000, 5104)])
def test_fp8_forward_every_tile_width(m, n):
    y, ref = forward8_case(m, 256, n, 256, seed=m + n)
    assert rel_l2(y, ref["y"]) < REL_L2
    y, ref = forward8_case(m, 256, n, 128, rank=32, seed=m + n + 1, scale=0.5)
    assert rel_l2(y, ref["y"]) < REL_L2


def test_fp8_forward_quantized_entry_matches_forward():
    inp = synth.make_linear(200, 512, 384, seed=13)
    x = d_bf16(inp["x"])
    qw, sw = h.sdnq_rotate_quantize_weight_fp8(d_bf16(inp["w"]), 256)
    y1 = h.sdnq_qlinear_forward_fp8(x, qw, sw, 256)
    qx, sx = h.sdnq_rotate_quantize_act_fp8(x, 256)
    y2 = h.sdnq_qlinear_forward_fp8_quantized(qx, sx, qw, sw)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_fp8_mlp_pair_full_size():
    """The FP8 benchmark rows: both MLP layers at 4096 tokens, codes and scales in
    full, outputs on sampled token rows."""
    inp = synth.make_config("mlp")
    oracle.set_num_threads(16)
    for xk, wk in (("x", "w_up"), ("h", "w_down")):
        say(f"  fp8 {xk} -> {wk}")
        qw, sw = h.sdnq_rotate_quantize_weight_fp8(d_bf16(inp[wk]), 256)
        qx, sx = h.sdnq_rotate_quantize_act_fp8(d_bf16(inp[xk]), 256)
        y = h.sdnq_qlinear_forward_fp8_quantized(qx, sx, qw, sw)
        torch.cuda.synchronize()
        qwo, swo = oracle.rotate_quantize_fp8(inp[wk], 256)
        qxo, sxo = oracle.rotate_quantize_fp8(inp[xk], 256)
        assert np.array_equal(qw.cpu().numpy(), qwo) and np.array_equal(qx.cpu().numpy(), qxo)
        assert np.array_equal(sw.cpu().numpy().view(np.uint32), swo.view(np.uint32))
        assert np.array_equal(sx.cpu().numpy().view(np.uint32), sxo.view(np.uint32))
        rows = np.array(sorted(set(range(8)) | set(range(4088, 4096)) | {1000, 2047, 3333}))
        ref = oracle.qlinear_forward_fp8(inp[xk][rows], qwo, swo, 256, intermediates=False)
        err = rel_l2(h_bits(y)[rows], ref["y"])
        say(f"    rel-L2 {err:.3e}")
        assert err < REL_L2


# ------------------------------------------------------------ FP8 backward --
# The input gradient through the E4M3 weight codes.  The dY fold and its E4M3
# codes are bit-exact (the entry point's workspace); dX is within 1e-2 relative
# L2 of the oracle over the tensor and for every token row (the GPU sums the
# decoded products with the fp32-accumulating MFMA, the oracle exactly); the LoRA
# term is checked alone with all-zero weight codes; the LoRA gradients as in the
# int8 path.

def max_token_rel(got_bits, ref_bits):
    g = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    r = synth.bf16_bits_to_f32(ref_bits).astype(np.float64)
    return float((np.linalg.norm(g - r, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-30)).max())


def backward8_case(m, n, k, g, rank=0, seed=0, scale=0.5, zero_weight=False, rows=None):
    inp = synth.make_linear(m, k, n, seed=seed, lora_rank=rank, backward=True)
    if zero_weight:
        inp["w"] = np.zeros_like(inp["w"])
    say(f"  qlinear_backward_input_fp8 m={m} n={n} k={k} g={g} rank={rank} zero_weight={zero_weight}")
    qw, sw = h.sdnq_rotate_quantize_weight_fp8(d_bf16(inp["w"]), g)
    la = d_bf16(inp["lora_a"]) if rank else None
    lb = d_bf16(inp["lora_b"]) if rank else None
    ws = torch.empty(h.sdnq_workspace_bytes(m, n, k, rank, True), dtype=torch.uint8, device=DEV)
    dx, ga, gb = h.sdnq_qlinear_backward_input_fp8(d_bf16(inp["dy"]), qw, sw, g, d_bf16(inp["x"]) if rank else None,
                                                   la, lb, scale, workspace=ws)
    torch.cuda.synchronize()
    qwo, swo = oracle.rotate_quantize_fp8(inp["w"], g)
    assert np.array_equal(qw.cpu().numpy(), qwo)
    qdy = ws[: m * n].view(m, n).cpu().numpy()
    off = (m * n + 255) // 256 * 256
    sdy = ws[off: off + 4 * m].cpu().numpy().view(np.float32)
    qo, so = oracle.rotate_quantize_fp8(inp["dy"], 1, swo)
    assert np.array_equal(qdy, qo), "dY' E4M3 codes"
    assert np.array_equal(sdy.view(np.uint32), so.view(np.uint32)), "dY' scales"
    rows = np.arange(m) if rows is None else rows
    ref = oracle.qlinear_backward_input_fp8(inp["dy"][rows], qwo, swo, g, None, inp.get("lora_a"),
                                            inp.get("lora_b"), scale, intermediates=False)
    got = h_bits(dx)[rows]
    err, tok = rel_l2(got, ref["dx"]), max_token_rel(got, ref["dx"])
    say(f"    dx rel-L2 {err:.3e}  max-token {tok:.3e}")
    assert err < REL_L2 and tok < REL_L2
    if rank and not zero_weight:
        grads = oracle.qlinear_backward_input(inp["dy"], np.zeros((n, k), np.int8), swo, g, inp["x"], inp["lora_a"],
                                              inp["lora_b"], scale, want_dx=False)
        for name, got_g in (("grad_a", ga), ("grad_b", gb)):
            e = rel_l2(h_bits(got_g), grads[name])
            say(f"    {name} rel-L2 {e:.3e}")
            assert e < REL_L2


@pytest.mark.parametrize("g", [1, 64, 128, 256])
def test_fp8_backward(g):
    backward8_case(300, 640, 768 if g != 256 else 512, g, seed=g)


@pytest.mark.parametrize("g,rank", [(256, 64), (64, 32), (128, 24)])
def test_fp8_backward_with_lora(g, rank):
    backward8_case(260, 384, 512, g, rank=rank, seed=rank + g)
    backward8_case(260, 384, 512, g, rank=rank, seed=rank + g + 1, zero_weight=True)


def test_fp8_backward_ragged_tiles():
    """Token rows and dX columns past the last full tile (384 = 1.5 column tiles)."""
    backward8_case(33, 272, 384, 128, rank=16, seed=5)


def test_fp8_backward_peft_size_sampled_rows():
    """16384 tokens x 3072 x 3072, g = 256, rank 64: every dY' code and scale, and
    sampled rows of dX."""
    c = synth.CONFIGS["peft"]
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(c.m - 8, c.m), rng.choice(c.m, 32, replace=False)]))
    backward8_case(c.m, c.n, c.k, 256, rank=c.lora_rank, seed=0, scale=c.lora_scale, rows=rows)
