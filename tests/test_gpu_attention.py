"""GPU parity of the int8-QK^T attention against the oracle.

Bit-exact: the q and k codes and scales and the K mean that the entry point
leaves in its workspace (both sides take every rounding decision on the same
binary32 values in the same order).  The oracle's K mean is the exact mean
rounded once; the GPU's binary64 sum reproduces it wherever that sum is exact
(every realistic key tensor), and elsewhere stays within the summation's error
bound.  Within 1e-2 relative L2 per head: the
output (the GPU accumulates P V in fp32 from bf16 P with exp2; the oracle
computes softmax and P V in fp64).
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


def run(q, k, v, causal, smooth, g, scale=None):
    b, hq, sq, d = q.shape
    hkv, sk = k.shape[1], k.shape[2]
    say(f"  attention B={b} Hq={hq} Hkv={hkv} Sq={sq} Sk={sk} D={d} causal={causal} smooth={smooth} g={g}")
    ws = torch.empty(h.sdnq_attention_workspace_bytes(b, hq, hkv, sq, sk, d), dtype=torch.uint8, device=DEV)
    out = h.sdnq_attention_int8(d_bf16(q), d_bf16(k), d_bf16(v), causal, scale, smooth, g, workspace=ws)
    torch.cuda.synchronize()
    off = [h.sdnq_attention_workspace_offset(b, hq, hkv, sq, sk, d, i) for i in range(5)]
    nq, nk = b * hq * sq, b * hkv * sk
    res = {
        "out": h_bits(out),
        "q_codes": ws[off[0]: off[0] + nq * d].cpu().numpy().view(np.int8).reshape(b, hq, sq, d),
        "q_scales": ws[off[1]: off[1] + 4 * nq].cpu().numpy().view(np.float32).reshape(b, hq, sq),
        "k_codes": ws[off[2]: off[2] + nk * d].cpu().numpy().view(np.int8).reshape(b, hkv, sk, d),
        "k_scales": ws[off[3]: off[3] + 4 * nk].cpu().numpy().view(np.float32).reshape(b, hkv, sk),
        "k_mean": ws[off[4]: off[4] + 4 * b * hkv * d].cpu().numpy().view(np.float32).reshape(b, hkv, d),
    }
    so = h.sdnq_attention_workspace_offset(b, hq, hkv, sq, sk, d, 5)
    assert int(ws[so: so + 4].cpu().numpy().view(np.uint32)[0]) == 0, "split-tile hand-over status"
    return res


def rel_l2_per_head(got_bits, ref_bits):
    g = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    r = synth.bf16_bits_to_f32(ref_bits).astype(np.float64)
    num = np.sqrt(((g - r) ** 2).sum(axis=(-2, -1)))
    den = np.sqrt((r ** 2).sum(axis=(-2, -1)))
    return (num / den).max()


def kmean_exact_domain(k_bits):
    """[B, H, D] mask of the channels whose binary64 partial sums are exact in any
    order: sum|k| < 2^53 * q, q the finest quantum (last place) among the nonzero
    keys.  There the GPU's mean is the exactly rounded mean (a binary64 sum, one
    division, one rounding to binary32)."""
    kf = synth.bf16_bits_to_f32(k_bits).astype(np.float64)
    e = ((np.asarray(k_bits, np.uint16) >> 7) & 0xFF).astype(np.int64)
    quantum = np.where(kf != 0, np.exp2(np.maximum(e, 1) - 134.0), np.inf).min(axis=2)
    return np.abs(kf).sum(axis=2) < 2.0 ** 53 * quantum


def kmean_error_bound(k_bits, got_mean):
    """Bound on |GPU mean - exact mean| for any inputs: the blocked binary64 sum
    (64-token blocks, then the block sums) errs by at most
    (63 + blocks) u sum|k| with u = 2^-53, the division by u |S / Sk|, and the
    binary32 rounding by half a unit in the last place."""
    kf = synth.bf16_bits_to_f32(k_bits).astype(np.float64)
    sk = kf.shape[2]
    n = 63 + (sk + 63) // 64 + 2
    ulp = np.spacing(np.abs(got_mean.astype(np.float32))).astype(np.float64)
    return n * 2.0 ** -53 * np.abs(kf).sum(axis=2) / sk + ulp


def check(q, k, v, causal, smooth, g, q_rows=None, scale=None):
    got = run(q, k, v, causal, smooth, g, scale)
    ref = oracle.attention_int8(q, k, v, causal, scale, smooth, g, intermediates=True, q_rows=q_rows)
    rows = slice(None) if q_rows is None else np.asarray(q_rows)
    same_mean = np.ones(k.shape[:2], bool)
    if smooth:
        dom = kmean_exact_domain(k)
        eq = got["k_mean"].view(np.uint32) == ref["k_mean"].view(np.uint32)
        assert np.all(eq[dom]), "k mean (exact domain)"
        err = np.abs(got["k_mean"].astype(np.float64) - ref["k_mean"].astype(np.float64))
        assert np.all(err <= kmean_error_bound(k, got["k_mean"])), "k mean (outside the exact domain)"
        same_mean = eq.all(axis=2)
        if not dom.all():
            say(f"    {int((~dom).sum())} channels outside the exact-sum domain, {int((~eq).sum())} means differ")
    # K codes follow from the mean: bit-exact for every head whose mean agrees
    assert np.array_equal(got["k_codes"][same_mean], ref["k_codes"][same_mean]), "k codes"
    assert np.array_equal(got["k_scales"][same_mean].view(np.uint32), ref["k_scales"][same_mean].view(np.uint32)), \
        "k scales"
    assert np.array_equal(got["q_codes"][:, :, rows], ref["q_codes"]), "q codes"
    assert np.array_equal(got["q_scales"][:, :, rows].view(np.uint32), ref["q_scales"].view(np.uint32)), "q scales"
    err = rel_l2_per_head(got["out"][:, :, rows], ref["out"])
    say(f"    output rel-L2 (worst head) {err:.3e}")
    assert np.all(np.isfinite(synth.bf16_bits_to_f32(got["out"])))
    assert err < REL_L2
    return got, ref


def inputs(b, hq, hkv, sq, sk, d, seed, bias=3.0):
    rng = np.random.default_rng(seed)
    q = synth.to_bf16_bits(rng.standard_normal((b, hq, sq, d)).astype(np.float32))
    k = synth.to_bf16_bits((rng.standard_normal((b, hkv, sk, d)) + rng.standard_normal((b, hkv, 1, d)) * bias)
                           .astype(np.float32))
    v = synth.to_bf16_bits(rng.standard_normal((b, hkv, sk, d)).astype(np.float32))
    return q, k, v


def test_attention_tiny_config():
    c = synth.ATTENTION_CONFIGS["attn_tiny"]
    d = synth.make_attention("attn_tiny")
    check(d["q"], d["k"], d["v"], c.causal, True, 256)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("smooth,g", [(True, 256), (False, 256), (True, 64), (True, 1), (False, 0)])
def test_attention_options(d, causal, smooth, g):
    q, k, v = inputs(1, 4, 2, 150, 208, d, 30 + d + int(causal))
    check(q, k, v, causal, smooth, g)


@pytest.mark.parametrize("sq,sk", [(1, 16), (17, 16), (128, 64), (129, 80), (300, 1024)])
def test_attention_ragged_and_tiny_lengths(sq, sk):
    q, k, v = inputs(2, 2, 1, sq, sk, 128, 40 + sq)
    check(q, k, v, True, True, 256)
    check(q, k, v, False, True, 256, scale=0.05)


def test_attention_text_encoder_config():
    c = synth.ATTENTION_CONFIGS["attn_te"]
    d = synth.make_attention("attn_te")
    rows = np.unique(np.concatenate([np.arange(4), np.arange(c.seq_q - 4, c.seq_q),
                                     np.random.default_rng(5).choice(c.seq_q, 24, replace=False)]))
    check(d["q"], d["k"], d["v"], True, True, 256, q_rows=rows)


def test_attention_flux_full_size():
    """flux.1 joint attention (24 heads x 128, 4608 tokens): every code and scale,
    and the output on sampled query rows of every head; then the error against
    exact fp64 attention on the same sampled rows."""
    c = synth.ATTENTION_CONFIGS["attn_flux"]
    d = synth.make_attention("attn_flux")
    rows = np.unique(np.concatenate([np.arange(4), np.arange(c.seq_q - 4, c.seq_q),
                                     np.random.default_rng(6).choice(c.seq_q, 24, replace=False)]))
    got, ref = check(d["q"], d["k"], d["v"], False, True, 256, q_rows=rows)
    f = lambda b: torch.from_numpy(synth.bf16_bits_to_f32(b).astype(np.float64))
    exact = torch.nn.functional.scaled_dot_product_attention(f(d["q"][:, :, rows]), f(d["k"]), f(d["v"])).numpy()
    o = synth.bf16_bits_to_f32(got["out"][:, :, rows]).astype(np.float64)
    err = np.linalg.norm(o - exact) / np.linalg.norm(exact)
    say(f"    error vs exact attention {err:.3e}")
    assert err < 0.03


@pytest.mark.parametrize("causal", [False, True])
def test_attention_row_maximum_keeps_growing(causal):
    """Scores that rise along the keys: every query has a component along one
    direction u and key j carries t_j u with t_j increasing, so a row's maximum
    grows by about 2^3 per 32-key step (2^42 over the row) and the softmax
    offset, which moves when the maximum passes it by 2^8, has to follow it
    several times; a late key then jumps 2^22 above the rest.  The output must
    still match the oracle."""
    rng = np.random.default_rng(77)
    b, hq, hkv, s, d = 1, 2, 1, 320, 128
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((b, hq, s, d)) * 0.3 + 4.0 * u
    t = np.linspace(0.0, 60.0, s)
    k = rng.standard_normal((b, hkv, s, d)) * 0.3 + t[None, None, :, None] * u
    k[:, :, s - 40, :] += 40.0 * u  # one late key far above the rest
    v = rng.standard_normal((b, hkv, s, d))
    qb, kb, vb = (synth.to_bf16_bits(a.astype(np.float32)) for a in (q, k, v))
    check(qb, kb, vb, causal, True, 256)
    check(qb, kb, vb, causal, False, 128)


@pytest.mark.parametrize("heads,s,d", [(22, 4608, 128), (25, 4096, 128), (52, 2048, 64), (28, 4608, 128)])
def test_attention_more_tiles_than_resident_workgroups(heads, s, d):
    """Non-causal shapes whose query tiles overfill the resident workgroups
    (3 per CU, 768 on 256 CUs): by a little (792, 800 and 832 tiles: the key
    tiles of most query tiles are split between two workgroups and their
    softmax states merged) or by a third (1 008 tiles: whole tiles, a second
    round).  Sampled rows of every head, spread over all query tiles, against
    the oracle."""
    q, k, v = inputs(1, heads, heads, s, s, d, heads + s + d)
    nq = (s + 127) // 128
    rng = np.random.default_rng(heads)
    rows = np.unique(np.concatenate([np.arange(nq) * 128 + rng.integers(0, 128, nq), [s - 1]]))
    rows = rows[rows < s]
    check(q, k, v, False, True, 256, q_rows=rows)


@pytest.mark.parametrize("heads,causal", [(24, False), (21, False), (8, True)])
def test_attention_repeat_runs_are_bit_identical(heads, causal):
    """The kernels are deterministic by construction (no atomics; split tiles
    merge their two halves in one fixed order), so repeated calls on the same
    inputs must give identical bits.  Catches races between the LDS refills and
    the fragment reads of the previous key tile, which show as a few wavefronts'
    rows off by a few per cent in some runs and not in others."""
    b, s, d = 1, 4608, 128
    g = torch.Generator(device=DEV).manual_seed(heads)
    q = torch.randn((b, heads, s, d), device=DEV, generator=g).to(torch.bfloat16)
    k = (torch.randn((b, heads, s, d), device=DEV, generator=g) +
         3.0 * torch.randn((b, heads, 1, d), device=DEV, generator=g)).to(torch.bfloat16)
    v = torch.randn((b, heads, s, d), device=DEV, generator=g).to(torch.bfloat16)
    say(f"  attention B={b} H={heads} S={s} D={d} causal={causal}, 4 runs")
    ws = torch.empty(h.sdnq_attention_workspace_bytes(b, heads, heads, s, s, d), dtype=torch.uint8, device=DEV)
    first = h.sdnq_attention_int8(q, k, v, causal, workspace=ws).clone()
    for _ in range(3):
        again = h.sdnq_attention_int8(q, k, v, causal, workspace=ws)
        torch.cuda.synchronize()
        diff = (again.view(torch.int16) != first.view(torch.int16))
        assert not diff.any().item(), f"{int(diff.any(-1).sum().item())} rows differ between runs"


def test_attention_handover_give_up_is_flagged():
    """The shared-tile wait bounded from the host.  With a bound of 0 the waiting
    workgroup gives up before its first poll: every call must set the status word,
    and every launch still ends.  With a bound of 1 it gives up only if its
    partner's share is not yet published: each call's output is the normal call's
    bit for bit, or its status word is set.  The default bound, restored, gives the
    normal output and a clear status word."""
    b, heads, s, d = 1, 24, 4608, 128  # 864 query tiles on 768 resident workgroups: shared tiles
    g = torch.Generator(device=DEV).manual_seed(99)
    q = torch.randn((b, heads, s, d), device=DEV, generator=g).to(torch.bfloat16)
    k = torch.randn((b, heads, s, d), device=DEV, generator=g).to(torch.bfloat16)
    v = torch.randn((b, heads, s, d), device=DEV, generator=g).to(torch.bfloat16)
    ws = torch.empty(h.sdnq_attention_workspace_bytes(b, heads, heads, s, s, d), dtype=torch.uint8, device=DEV)
    so = h.sdnq_attention_workspace_offset(b, heads, heads, s, s, d, 5)

    def status():
        return int(ws[so: so + 4].cpu().numpy().view(np.uint32)[0])

    normal = h.sdnq_attention_int8(q, k, v, False, workspace=ws).clone()
    torch.cuda.synchronize()
    assert status() == 0
    flagged = 0
    try:
        h.sdnq_attention_set_handover_polls(0)
        for _ in range(2):
            h.sdnq_attention_int8(q, k, v, False, workspace=ws)
            torch.cuda.synchronize()
            assert status() != 0, "a wait that gave up left the status word clear"
        h.sdnq_attention_set_handover_polls(1)
        for _ in range(3):
            out = h.sdnq_attention_int8(q, k, v, False, workspace=ws)
            torch.cuda.synchronize()
            st = status()
            same = torch.equal(out.view(torch.int16), normal.view(torch.int16))
            assert st != 0 or same, "output changed without a status"
            flagged += st != 0
    finally:
        h.sdnq_attention_set_handover_polls(h.SDNQ_ATTENTION_HANDOVER_POLLS)
    say(f"    one-poll bound: {flagged} of 3 calls flagged")
    out = h.sdnq_attention_int8(q, k, v, False, workspace=ws)
    torch.cuda.synchronize()
    assert status() == 0
    assert torch.equal(out.view(torch.int16), normal.view(torch.int16))


def stress_rows(d, n, seed):
    """n rows of d values: the quantizer's edge cases (as the linear layer's stress
    rows, with the large channel kept at 1e15 so that scores stay finite), then
    normal rows."""
    rng = np.random.default_rng(seed)
    rows = [np.zeros(d, np.float32)]                                        # all-zero row
    r = rng.standard_normal(d).astype(np.float32); r[17] = 1e15; rows.append(r)   # one large channel
    r = rng.standard_normal(d).astype(np.float32); r[rng.permutation(d)[:5]] *= 1000; rows.append(r)
    rows.append((rng.standard_normal(d) * 1e-38).astype(np.float32))      # tiny (normal and subnormal)
    rows.append((rng.standard_normal(d) * 1e-36).astype(np.float32))
    r = np.zeros(d, np.float32); r[:4] = [1.0, 2.0 ** -24, -1.0, 2.0 ** -24]; rows.append(r)  # stage order
    r = (rng.integers(-254, 255, d) / 2.0).astype(np.float32); r[3] = 127.0; rows.append(r)  # ties
    r = np.zeros(d, np.float32); r[:2] = [1.125, 0.5625]; rows.append(r)  # reciprocal case
    rows.append(np.full(d, 3.0, np.float32))                               # constant
    r = np.zeros(d, np.float32); r[d // 2] = 1.0; rows.append(r)           # one-hot
    rows.append(-np.abs(rng.standard_normal(d)).astype(np.float32))
    while len(rows) < n:
        rows.append(rng.standard_normal(d).astype(np.float32))
    return np.stack(rows[:n])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("smooth", [False, True])
def test_attention_prep_stress_rows(d, smooth):
    """Q and K rows at the quantizer's edge cases: codes, scales and the K mean
    bit-exact against the oracle, the output within the tolerance."""
    q = synth.to_bf16_bits(np.stack([stress_rows(d, 24, 50), stress_rows(d, 24, 51)])[None])
    k = synth.to_bf16_bits(stress_rows(d, 32, 52)[None, None])
    v = synth.to_bf16_bits(np.random.default_rng(53).standard_normal((1, 1, 32, d)).astype(np.float32))
    for g in (256, 1):
        check(q, k, v, False, smooth, g)


def test_attention_k_mean_outside_the_exact_sum_domain():
    """Keys for which a binary64 running sum rounds (2^60, 1, -2^60 patterns,
    2^100 next to ones, bf16 subnormals next to large keys), 256 tokens in four
    summation blocks: the oracle's mean is exact, the GPU's within the bound of
    its blocked binary64 sum; a second head of ordinary keys stays bit-exact."""
    rng = np.random.default_rng(91)
    b, hkv, s, d = 1, 2, 256, 64
    k = rng.standard_normal((b, hkv, s, d)) + 3.0 * rng.standard_normal((b, hkv, 1, d))
    odd = k[0, 1]
    odd[0::3, 0], odd[1::3, 0], odd[2::3, 0] = 2.0 ** 60, 1.0, -(2.0 ** 60)
    odd[:, 1] = np.where(np.arange(s) % 2 == 0, 2.0 ** 100, 1.0)
    odd[:, 2] = rng.integers(-255, 256, s) * 2.0 ** -133
    odd[7, 2] = 1.0e20
    odd[:, 3] = rng.standard_normal(s) * 2.0 ** rng.integers(-120, 60, s)
    kb = synth.to_bf16_bits(k.astype(np.float32))
    q = synth.to_bf16_bits(rng.standard_normal((b, 2, 64, d)).astype(np.float32))
    v = synth.to_bf16_bits(rng.standard_normal((b, hkv, s, d)).astype(np.float32))
    dom = kmean_exact_domain(kb)
    assert dom[0, 0].all() and not dom[0, 1, :4].any()
    got = run(q, kb, v, False, True, 256)
    ref = oracle.attention_int8(q, kb, v, False, None, True, 256, intermediates=True)
    eq = got["k_mean"].view(np.uint32) == ref["k_mean"].view(np.uint32)
    assert eq[dom].all()
    err = np.abs(got["k_mean"].astype(np.float64) - ref["k_mean"].astype(np.float64))
    bound = kmean_error_bound(kb, got["k_mean"])
    say(f"    outside the domain: {int((~eq).sum())} means differ, worst error / bound "
        f"{float((err / bound).max()):.3e}")
    assert np.all(err <= bound)
    assert np.array_equal(got["k_codes"][0, 0], ref["k_codes"][0, 0])
