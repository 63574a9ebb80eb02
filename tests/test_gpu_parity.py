"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same
seeded inputs.

Bars: bit-exact int8 codes, fp32 scales and int32 accumulators; the forward output
without LoRA is also bit-exact (both sides round fl32(fl32(acc) * fl32(s_x * s_w))
to bf16), and so is the input gradient without LoRA (both sides form
fl32(acc) * s_dy, run the butterfly's stages in ascending order, multiply by
fl32(1/sqrt(g)) and round once to bf16).  bf16 outputs with LoRA and the LoRA
gradients are within 1e-2 relative L2 of the oracle (the layer's stated
tolerance), over the whole tensor and for every token row on its own: both
sides round the same sums to bf16 (a flip moves an element by at most 2^-8 of
its value), and the GPU's extra bf16 roundings of the LoRA intermediates touch
only the LoRA term's share of each row.  The LoRA term itself is checked with an
all-zero weight, where it is the whole output.
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


def d(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def h_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def rel_l2(got_bits, ref_bits):
    g, r = f32(got_bits), f32(ref_bits)
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))


def max_token_rel(got_bits, ref_bits):
    g, r = f32(got_bits), f32(ref_bits)
    num = np.linalg.norm(g - r, axis=1)
    den = np.maximum(np.linalg.norm(r, axis=1), 1e-30)
    return float((num / den).max())


def assert_close(got_bits, ref_bits, what="", per_token=True):
    """Relative L2 over the tensor and, for outputs whose rows are tokens (y, dx),
    for the worst token row, both below 1e-2.  The LoRA weight gradients are sums
    over all tokens; their rows are features, compared as one tensor."""
    err, tok = rel_l2(got_bits, ref_bits), max_token_rel(got_bits, ref_bits)
    say(f"    {what} rel-L2 {err:.3e}  max-row {tok:.3e}")
    assert err < REL_L2, f"{what} rel-L2 {err:.3e}"
    if per_token:
        assert tok < REL_L2, f"{what} worst token rel-L2 {tok:.3e}"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    h.lib()
    yield
    torch.cuda.synchronize()


def rq_gpu(x_bits, g, col_scale=None):
    say(f"  rotate_quantize_act {x_bits.shape} g={g} colscale={col_scale is not None}")
    q, s = h.sdnq_rotate_quantize_act(d_bf16(x_bits), g, None if col_scale is None else d(col_scale))
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def assert_rq_exact(x_bits, g, col_scale=None):
    q, s = rq_gpu(x_bits, g, col_scale)
    qo, so = oracle.rotate_quantize(x_bits, g, col_scale)
    bad = np.nonzero(np.any(q != qo, axis=1))[0]
    assert bad.size == 0, f"codes differ in rows {bad[:8]}"
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), "scales differ"


# ----------------------------------------------------------------- G1 --

@pytest.mark.parametrize("g,m,k", [
    (256, 64, 512), (256, 37, 3072), (256, 3, 256), (256, 130, 768),
    (128, 37, 384), (128, 19, 1152), (128, 64, 3072),
    (64, 33, 320), (64, 5, 64), (64, 70, 3072), (64, 9, 192),
    (1, 11, 16), (1, 21, 48), (1, 40, 272), (1, 64, 3072),
    # rows of 1536, 10240 and 14336 values: 8 lanes per 256-value superblock, a
    # row group of 4 rows (1536) or 1 row, with a partial last group
    (256, 7, 1536), (128, 13, 1536), (64, 5, 1536), (1, 9, 1536),
    (128, 3, 10240), (64, 6, 10240), (1, 4, 10240), (256, 5, 14336),
    (256, 3, 40960), (64, 2, 65536),        # rows longer than 32768 values: 1024-thread workgroups
    # rows longer than 65536 values, quantized in 2, 3 and 4 segments of whole blocks
    (256, 3, 98304), (128, 2, 65664), (64, 2, 133120), (1, 3, 100000),
])
def test_rotate_quantize_bit_exact(g, m, k):
    x = synth.make_linear(m, k, 16, seed=100 + g + m)["x"]
    assert_rq_exact(x, g)


@pytest.mark.parametrize("g,m,k", [(64, 20000, 3072), (256, 9000, 10240), (1, 30000, 512)])
def test_rotate_quantize_many_rows_bit_exact(g, m, k):
    """Enough rows that every persistent workgroup walks several row groups."""
    x = synth.make_linear(m, k, 16, seed=7 + g)["x"]
    assert_rq_exact(x, g)


@pytest.mark.parametrize("k", [16, 272, 1536, 3072, 10240, 100000])
def test_rotate_quantize_column_scale_bit_exact(k):
    rng = np.random.default_rng(5 + k)
    dy = synth.to_bf16_bits(rng.standard_normal((29, k)).astype(np.float32) * 1e-3)
    cs = (rng.uniform(0.5, 2.0, k) * 1e-3).astype(np.float32)
    assert_rq_exact(dy, 1, cs)


@pytest.mark.parametrize("k", [512, 1536])   # 4 and 8 lanes per superblock
@pytest.mark.parametrize("g", [1, 64, 128, 256])
def test_rotate_quantize_stress_rows(g, k):
    rng = np.random.default_rng(7)
    rows = []
    rows.append(np.zeros(k, np.float32))                                   # all-zero row
    r = rng.standard_normal(k).astype(np.float32); r[17] = 1e30; rows.append(r)   # one huge channel
    r = rng.standard_normal(k).astype(np.float32); r[rng.permutation(k)[:5]] *= 1000; rows.append(r)
    rows.append((rng.standard_normal(k) * 1e-38).astype(np.float32))      # tiny values (normal and subnormal)
    rows.append((rng.standard_normal(k) * 1e-36).astype(np.float32))
    r = np.zeros(k, np.float32); r[:4] = [1.0, 2.0 ** -24, -1.0, 2.0 ** -24]; rows.append(r)  # stage-order case
    r = (rng.integers(-254, 255, k) / 2.0).astype(np.float32); r[3] = 127.0; rows.append(r)  # rne ties
    r = np.zeros(k, np.float32); r[:2] = [1.125, 0.5625]; rows.append(r)  # reciprocal case
    r = np.full(k, 3.0, np.float32); rows.append(r)                        # constant blocks
    r = np.zeros(k, np.float32); r[300] = 1.0; rows.append(r)              # one-hot
    r = -np.abs(rng.standard_normal(k)).astype(np.float32); rows.append(r)
    x = synth.to_bf16_bits(np.stack(rows))
    assert_rq_exact(x, g)


@pytest.mark.parametrize("g", [64, 128, 256])
def test_weight_prep_bit_exact(g):
    w = synth.make_config("tiny")["w"]
    say(f"  rotate_quantize_weight g={g}")
    qw, sw = h.sdnq_rotate_quantize_weight(d_bf16(w), g)
    torch.cuda.synchronize()
    qo, so = oracle.rotate_quantize(w, g)
    assert np.array_equal(qw.cpu().numpy(), qo)
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), so.view(np.uint32))


def test_empty_batch_is_a_no_op():
    say("  empty batch")
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)
    q, s = h.sdnq_rotate_quantize_act(x, 256)
    assert q.shape == (0, 256) and s.shape == (0,)
    w = d_bf16(synth.make_linear(4, 256, 32)["w"])
    qw, sw = h.sdnq_rotate_quantize_weight(w, 256)
    y = h.sdnq_qlinear_forward(x, qw, sw, 256)
    assert y.shape == (0, 32)
    la = torch.ones((256, 16), dtype=torch.bfloat16, device=DEV)
    lb = torch.ones((16, 32), dtype=torch.bfloat16, device=DEV)
    dy = torch.zeros((0, 32), dtype=torch.bfloat16, device=DEV)
    dx, ga, gb = h.sdnq_qlinear_backward_input(dy, qw, sw, 256, x, la, lb, 1.0)
    torch.cuda.synchronize()
    assert dx.shape == (0, 256)
    assert torch.count_nonzero(ga).item() == 0 and torch.count_nonzero(gb).item() == 0


# ----------------------------------------------------------------- G2 --

@pytest.mark.parametrize("b_layout", [0, 1])
@pytest.mark.parametrize("m,n,k", [(64, 512, 512), (300, 640, 400), (1, 16, 16), (257, 272, 4096),
                                   (513, 256, 128), (40, 48, 144)])
def test_gemm_int32_bit_exact(m, n, k, b_layout):
    rng = np.random.default_rng(m * 7 + n + k)
    a = rng.integers(-128, 128, (m, k)).astype(np.int8)
    b = rng.integers(-128, 128, (n, k) if b_layout == 0 else (k, n)).astype(np.int8)
    say(f"  gemm_i8_i32 m={m} n={n} k={k} layout={b_layout}")
    c = h.sdnq_gemm_i8_i32(d(a), d(b), b_layout)
    torch.cuda.synchronize()
    ref = oracle.gemm_i8(a, b, b_layout)
    assert np.array_equal(c.cpu().numpy(), ref)


# Shapes that select each output tile width on a 256-CU device (the launch picks
# the width with the fewest column-rounds): small grids take 192 columns,
# 4000 x 3840 takes 256 (240 tiles) and 4000 x 5104 takes 320 (256 tiles), all
# with ragged row, column and K tails.
TILE_WIDTH_SHAPES = [(4000, 3840, 80), (4000, 5104, 80), (260, 400, 48)]


@pytest.mark.parametrize("b_layout", [0, 1])
@pytest.mark.parametrize("m,n,k", TILE_WIDTH_SHAPES)
def test_gemm_int32_every_tile_width(m, n, k, b_layout):
    rng = np.random.default_rng(m + n + k + b_layout)
    a = rng.integers(-128, 128, (m, k)).astype(np.int8)
    b = rng.integers(-128, 128, (n, k) if b_layout == 0 else (k, n)).astype(np.int8)
    say(f"  gemm_i8_i32 m={m} n={n} k={k} layout={b_layout}")
    c = h.sdnq_gemm_i8_i32(d(a), d(b), b_layout)
    torch.cuda.synchronize()
    ref = oracle.gemm_i8(a, b, b_layout)
    assert np.array_equal(c.cpu().numpy(), ref)


@pytest.mark.parametrize("m,n", [(4000, 3840), (4000, 5104), (260, 400)])
def test_forward_every_tile_width(m, n):
    y, ref = forward_case(m, 256, n, 256, seed=m + n)
    assert np.array_equal(y, ref["y"]), f"rel-L2 {rel_l2(y, ref['y']):.3e}"
    y, ref = forward_case(m, 256, n, 128, rank=32, seed=m + n + 1, scale=0.5)
    assert_close(y, ref["y"], "y")
    # the LoRA epilogue of this tile width alone: with an all-zero weight it is the output
    y, ref = forward_case(m, 256, n, 128, rank=32, seed=m + n + 2, scale=0.5, zero_weight=True)
    assert_close(y, ref["y"], "LoRA term")


def test_gemm_int32_extreme_values():
    k = 4096
    a = np.full((32, k), -128, np.int8)
    b = np.full((32, k), -128, np.int8)
    say("  gemm_i8_i32 extremes")
    c = h.sdnq_gemm_i8_i32(d(a), d(b), 0)
    torch.cuda.synchronize()
    assert np.all(c.cpu().numpy() == 128 * 128 * k)


# ------------------------------------------------------------ forward --

def forward_case(m, k, n, g, rank=0, seed=0, scale=1.0, zero_weight=False):
    inp = synth.make_linear(m, k, n, seed=seed, lora_rank=rank)
    if zero_weight:  # codes and scales all zero: the output is the LoRA term alone
        inp["w"] = np.zeros_like(inp["w"])
    qwo, swo = oracle.rotate_quantize(inp["w"], g)
    say(f"  qlinear_forward m={m} k={k} n={n} g={g} rank={rank}")
    qw, sw = h.sdnq_rotate_quantize_weight(d_bf16(inp["w"]), g)
    la = d_bf16(inp["lora_a"]) if rank else None
    lb = d_bf16(inp["lora_b"]) if rank else None
    y = h.sdnq_qlinear_forward(d_bf16(inp["x"]), qw, sw, g, la, lb, scale)
    torch.cuda.synchronize()
    assert np.array_equal(qw.cpu().numpy(), qwo)
    ref = oracle.qlinear_forward(inp["x"], qwo, swo, g, inp.get("lora_a"), inp.get("lora_b"), scale)
    return h_bits(y), ref


@pytest.mark.parametrize("g", [1, 64, 128, 256])
@pytest.mark.parametrize("m,k,n", [(64, 512, 512), (300, 768, 640), (7, 256, 16)])
def test_forward_without_lora_is_bit_exact(m, k, n, g):
    y, ref = forward_case(m, k, n, g, seed=m + g)
    assert np.array_equal(y, ref["y"]), f"rel-L2 {rel_l2(y, ref['y']):.3e}"


# More tiles than CUs (two rounds: 512 tiles of 256 x 320 and of 256 x 192, 480
# of 256 x 256), with short contractions of even and odd k-tile counts and a
# partial last k-tile, so the oracle can check every output of the large grids.
@pytest.mark.parametrize("m,k,n,g", [(4096, 256, 10240, 256), (4096, 384, 10240, 128), (4096, 272, 10240, 1),
                                     (8192, 128, 3072, 64), (8192, 256, 3840, 256)])
def test_forward_two_rounds_of_tiles_bit_exact(m, k, n, g):
    y, ref = forward_case(m, k, n, g, seed=m + k + n)
    assert np.array_equal(y, ref["y"]), f"rel-L2 {rel_l2(y, ref['y']):.3e}"


@pytest.mark.parametrize("g,rank,scale", [(64, 32, 1.0), (128, 32, 1.0), (256, 16, 2.0), (128, 64, 0.5),
                                          (64, 128, 0.25)])
def test_forward_with_lora(g, rank, scale):
    y, ref = forward_case(300, 768, 640, g, rank=rank, seed=rank + g, scale=scale)
    assert_close(y, ref["y"], "y")
    y, ref = forward_case(300, 768, 640, g, rank=rank, seed=rank + g + 1, scale=scale, zero_weight=True)
    assert_close(y, ref["y"], "LoRA term")


@pytest.mark.parametrize("rank", [48, 128])
def test_forward_with_lora_many_tokens(rank):
    """16400 tokens: the LoRA down-projection's wide-workgroup variant with a ragged last workgroup."""
    y, ref = forward_case(16400, 320, 256, 64, rank=rank, seed=5 + rank, scale=0.75)
    assert_close(y, ref["y"], "y")
    y, ref = forward_case(16400, 320, 256, 64, rank=rank, seed=6 + rank, scale=0.75, zero_weight=True)
    assert_close(y, ref["y"], "LoRA term")


def test_forward_quantized_entry_matches_forward():
    inp = synth.make_linear(200, 512, 384, seed=3, lora_rank=32)
    say("  forward_quantized vs forward")
    x, la, lb = d_bf16(inp["x"]), d_bf16(inp["lora_a"]), d_bf16(inp["lora_b"])
    qw, sw = h.sdnq_rotate_quantize_weight(d_bf16(inp["w"]), 128)
    y1 = h.sdnq_qlinear_forward(x, qw, sw, 128, la, lb, 1.0)
    qx, sx = h.sdnq_rotate_quantize_act(x, 128)
    t = (x.float() @ la.float()).to(torch.bfloat16)
    y2 = h.sdnq_qlinear_forward_quantized(qx, sx, qw, sw, t, lb, 1.0)
    y3 = h.sdnq_qlinear_forward_quantized(qx, sx, qw, sw)
    y4 = h.sdnq_qlinear_forward(x, qw, sw, 128)
    torch.cuda.synchronize()
    assert rel_l2(h_bits(y2), h_bits(y1)) < 1e-2
    assert torch.equal(y3, y4)


# ----------------------------------------------------------- backward --

def backward_case(m, n, k, g, rank=0, seed=0, scale=0.5, grads=True, zero_weight=False):
    inp = synth.make_linear(m, k, n, seed=seed, lora_rank=rank, backward=True)
    if zero_weight:  # s_w = 0 folds dY to zero: dX is the LoRA term g_r A^T alone
        inp["w"] = np.zeros_like(inp["w"])
    qwo, swo = oracle.rotate_quantize(inp["w"], g)
    say(f"  qlinear_backward_input m={m} n={n} k={k} g={g} rank={rank}")
    qw, sw = h.sdnq_rotate_quantize_weight(d_bf16(inp["w"]), g)
    la = d_bf16(inp["lora_a"]) if rank else None
    lb = d_bf16(inp["lora_b"]) if rank else None
    x = d_bf16(inp["x"]) if (rank and grads) else None
    dx, ga, gb = h.sdnq_qlinear_backward_input(d_bf16(inp["dy"]), qw, sw, g, x, la, lb, scale)
    torch.cuda.synchronize()
    ref = oracle.qlinear_backward_input(inp["dy"], qwo, swo, g, inp["x"] if grads else None, inp.get("lora_a"),
                                        inp.get("lora_b"), scale)
    return inp, (h_bits(dx), None if ga is None else h_bits(ga), None if gb is None else h_bits(gb)), ref, swo


@pytest.mark.parametrize("m,n,k,g", [(m, n, k, g) for (m, n, k) in [(300, 640, 768), (260, 208, 512), (33, 272, 384),
                                                                    (7, 16, 256)]
                                     for g in (1, 64, 128, 256) if k % g == 0])
def test_backward_without_lora_is_bit_exact(m, n, k, g):
    """Ragged token and column tiles included (768 and 384 leave the last 256-column
    tile partly past K)."""
    inp, (dx, _, _), ref, swo = backward_case(m, n, k, g, seed=g + m)
    assert np.array_equal(dx, ref["dx"]), f"dx rel-L2 {rel_l2(dx, ref['dx']):.3e}"
    assert_rq_exact(inp["dy"], 1, swo)   # the backward's dY quantization, bit-exact


def assert_lora_grads(dx, ga, gb, ref):
    assert_close(dx, ref["dx"], "dx")
    assert_close(ga, ref["grad_a"], "grad_a", per_token=False)
    assert_close(gb, ref["grad_b"], "grad_b", per_token=False)


@pytest.mark.parametrize("g,rank", [(256, 64), (64, 32), (128, 16)])
def test_backward_with_lora_grads(g, rank):
    inp, (dx, ga, gb), ref, _ = backward_case(300, 640, 768, g, rank=rank, seed=rank, scale=0.5)
    assert_lora_grads(dx, ga, gb, ref)
    inp, (dx, _, _), ref, _ = backward_case(300, 640, 768, g, rank=rank, seed=rank + 1, scale=0.5, grads=False,
                                            zero_weight=True)
    assert_close(dx, ref["dx"], "LoRA dx term")


@pytest.mark.parametrize("m,rank", [(100, 16), (2000, 40), (5000, 64)])
def test_backward_one_lora_gradient(m, rank):
    """grad_a alone and grad_b alone (the C ABI's nullable outputs): each equals
    the two-gradient call bit for bit (same token splits, independent jobs) and
    the oracle within the tolerance.  m spans one split per 64 tokens up to the
    split count the workgroup target sets; rank 40 is zero-padded to 48."""
    import ctypes
    n, k, g = 640, 768, 128
    inp = synth.make_linear(m, k, n, seed=m + rank, lora_rank=rank, backward=True)
    say(f"  one LoRA gradient m={m} n={n} k={k} rank={rank}")
    qw, sw = h.sdnq_rotate_quantize_weight(d_bf16(inp["w"]), g)
    dy, x = d_bf16(inp["dy"]), d_bf16(inp["x"])
    la, lb = d_bf16(inp["lora_a"]), d_bf16(inp["lora_b"])
    ws = torch.empty(h.sdnq_workspace_bytes(m, n, k, rank, True), dtype=torch.uint8, device=DEV)
    L = h.lib()
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call(want_a, want_b):
        dx = torch.empty((m, k), dtype=torch.bfloat16, device=DEV)
        ga = torch.empty((k, rank), dtype=torch.bfloat16, device=DEV) if want_a else None
        gb = torch.empty((rank, n), dtype=torch.bfloat16, device=DEV) if want_b else None
        rc = L.sdnq_qlinear_backward_input(P(dy), m, n, P(qw), P(sw), k, g, P(x), P(la), P(lb), rank, 0.5, P(dx),
                                           P(ga), P(gb), P(ws), ws.numel(), sp)
        assert rc == 0, h.status_string(rc)
        torch.cuda.synchronize()
        return dx, ga, gb

    dx2, ga2, gb2 = call(True, True)
    dxa, ga1, _ = call(True, False)
    dxb, _, gb1 = call(False, True)
    assert torch.equal(dxa.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(dxb.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(ga1.view(torch.int16), ga2.view(torch.int16))
    assert torch.equal(gb1.view(torch.int16), gb2.view(torch.int16))
    qwo, swo = oracle.rotate_quantize(inp["w"], g)
    ref = oracle.qlinear_backward_input(inp["dy"], qwo, swo, g, inp["x"], inp["lora_a"], inp["lora_b"], 0.5)
    assert_lora_grads(h_bits(dx2), h_bits(ga1), h_bits(gb1), ref)


@pytest.mark.parametrize("g,k", [(128, 384), (64, 320), (256, 512)])
def test_backward_partial_column_tile(g, k):
    """The last 256-column tile of dX is partly past K; the rotation blocks stay whole."""
    inp, (dx, ga, gb), ref, _ = backward_case(260, 208, k, g, rank=16, seed=k + g, scale=0.25)
    assert_lora_grads(dx, ga, gb, ref)
    inp, (dx, _, _), ref, _ = backward_case(260, 208, k, g, rank=16, seed=k + g + 1, scale=0.25, grads=False,
                                            zero_weight=True)
    assert_close(dx, ref["dx"], "LoRA dx term")


def test_backward_ragged_tokens_and_tiles():
    inp, (dx, ga, gb), ref, _ = backward_case(33, 272, 512, 256, rank=32, seed=9)
    assert_lora_grads(dx, ga, gb, ref)


@pytest.mark.parametrize("rank,g", [(48, 128), (200, 64)])
def test_backward_many_tokens_with_lora(rank, g):
    """16400 tokens: the down-projections of g_r and t run as one launch of the
    LDS-staged kernel (128 tokens per workgroup, a ragged last workgroup of 16),
    rank 48 with a half-empty 32-rank block, rank 200 as slices of 128 and 80;
    272 columns leave the last 128-byte k-tile partly past the row."""
    inp, (dx, ga, gb), ref, _ = backward_case(16400, 272, 256, g, rank=rank, seed=11 + rank, scale=0.5)
    assert_lora_grads(dx, ga, gb, ref)


# ---------------------------------------------------------- LoRA ranks --
# Any rank in [1, 256]: ranks off the multiple of 16 run on zero-padded factors,
# ranks above 128 in two slices of the down-projection.

@pytest.mark.parametrize("rank", [1, 8, 33, 200, 256])
def test_forward_any_lora_rank(rank):
    y, ref = forward_case(300, 512, 640, 128, rank=rank, seed=rank + 300, scale=32.0 / rank)
    assert_close(y, ref["y"], f"rank {rank} y")
    y, ref = forward_case(300, 512, 640, 128, rank=rank, seed=rank + 301, scale=32.0 / rank, zero_weight=True)
    assert_close(y, ref["y"], f"rank {rank} LoRA term")


@pytest.mark.parametrize("rank", [1, 8, 33, 200, 256])
def test_backward_any_lora_rank(rank):
    inp, (dx, ga, gb), ref, _ = backward_case(260, 384, 512, 256, rank=rank, seed=rank + 400, scale=32.0 / rank)
    assert ga.shape == (512, rank) and gb.shape == (rank, 384)
    assert_lora_grads(dx, ga, gb, ref)
    inp, (dx, _, _), ref, _ = backward_case(260, 384, 512, 256, rank=rank, seed=rank + 401, scale=32.0 / rank,
                                            grads=False, zero_weight=True)
    assert_close(dx, ref["dx"], f"rank {rank} LoRA dx term")


@pytest.mark.parametrize("rank", [1, 33, 200])
def test_forward_quantized_any_lora_rank(rank):
    """The caller's t [m, rank] (rows not 16-byte multiples) goes through the
    padded copy; the result equals the full forward's up to the rounding of t."""
    inp = synth.make_linear(200, 512, 384, seed=rank, lora_rank=rank)
    say(f"  forward_quantized rank={rank}")
    x, la, lb = d_bf16(inp["x"]), d_bf16(inp["lora_a"]), d_bf16(inp["lora_b"])
    qw, sw = h.sdnq_rotate_quantize_weight(d_bf16(inp["w"]), 128)
    qx, sx = h.sdnq_rotate_quantize_act(x, 128)
    t = (x.float() @ la.float()).to(torch.bfloat16)
    y = h.sdnq_qlinear_forward_quantized(qx, sx, qw, sw, t, lb, 1.0)
    torch.cuda.synchronize()
    qwo, swo = oracle.rotate_quantize(inp["w"], 128)
    ref = oracle.qlinear_forward(inp["x"], qwo, swo, 128, inp["lora_a"], inp["lora_b"], 1.0)
    assert_close(h_bits(y), ref["y"], f"rank {rank} y")


# ------------------------------------------------- transposed weight codes --

@pytest.mark.parametrize("fp8", [False, True])
def test_backward_with_transposed_codes_is_the_same_call(fp8):
    """qw_t made once by sdnq_transpose_codes gives the backward's results bit for bit."""
    inp = synth.make_linear(300, 768, 640, seed=21, lora_rank=32, backward=True)
    quant = h.sdnq_rotate_quantize_weight_fp8 if fp8 else h.sdnq_rotate_quantize_weight
    say(f"  transposed codes fp8={fp8}")
    qw, sw = quant(d_bf16(inp["w"]), 128)
    qwt = h.sdnq_transpose_codes(qw)
    torch.cuda.synchronize()
    assert torch.equal(qwt.cpu(), qw.cpu().t().contiguous())
    f, ft = ((h.sdnq_qlinear_backward_input_fp8, h.sdnq_qlinear_backward_input_fp8_wt) if fp8 else
             (h.sdnq_qlinear_backward_input, h.sdnq_qlinear_backward_input_wt))
    dy, x, la, lb = (d_bf16(inp[k]) for k in ("dy", "x", "lora_a", "lora_b"))
    a = f(dy, qw, sw, 128, x, la, lb, 0.5)
    b = ft(dy, qwt, sw, 128, x, la, lb, 0.5)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ------------------------------------------------- the int32 bound on K --

def test_forward_at_the_largest_contraction_is_bit_exact():
    """K = 133120 (the largest multiple of 256 with 127 * 127 * K < 2^31): the
    rows are quantized in segments and the int32 accumulators stay exact."""
    y, ref = forward_case(64, 133120, 256, 256, seed=31)
    assert np.array_equal(y, ref["y"]), f"rel-L2 {rel_l2(y, ref['y']):.3e}"


def test_backward_with_rows_above_65536_is_bit_exact():
    """n = 100000: dY rows are folded and quantized in two segments, and n is the
    GEMM's contraction."""
    inp, (dx, _, _), ref, swo = backward_case(48, 100000, 256, 64, seed=32)
    assert np.array_equal(dx, ref["dx"]), f"dx rel-L2 {rel_l2(dx, ref['dx']):.3e}"
    assert_rq_exact(inp["dy"], 1, swo)
