"""Seeded synthetic inputs for the Hadamard-rotated INT8 linear layer.

This module holds only input generation (random draws and their rounding to
bfloat16).  None of the layer's arithmetic is here, so the GPU path, the CPU
oracle, the tests and the benchmark can all read the same bytes from it.

Workload model.  The pages measure real diffusion transformers, which are not
available here; these inputs stand in for them:
  * activations are N(0, 1) with a few "outlier" input channels scaled by 20,
    following the observation that activations concentrate their energy in a
    few input channels (SD.Next dev-branch commit log, the LoRA svd-calibration
    commit) and the extreme-activation stress rows of the benchmark commits;
  * weights are N(0, 0.02); LoRA factors N(0, 0.01); the upstream gradient of
    the PEFT step is N(0, 1e-3);
  * the 3072 x 3072 shape is the flux.1 attention linear named in the same
    commit log's benchmark shape list.
N(0, s) means standard deviation s.  "1 % of channels" means round(0.01 * K)
channels picked by a seeded permutation, scaled before the bf16 rounding.
Every config draws from one ``numpy.random.default_rng(seed)`` in a fixed order.

bf16 tensors are returned as ``numpy.uint16`` arrays of raw bfloat16 bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> binary32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gaussian(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def outlier_activations(rng: np.random.Generator, m: int, k: int, channels=None,
                        frac: float = 0.01, factor: float = 20.0) -> np.ndarray:
    """x ~ N(0, 1) [m, k] (binary32) with some input channels scaled by ``factor``.
    ``channels`` fixes them; otherwise round(frac * k) channels come from a seeded
    permutation drawn right after x."""
    x = rng.standard_normal((m, k), dtype=np.float32)
    if channels is None:
        count = int(round(frac * k))
        channels = np.sort(rng.permutation(k)[:count])
    x[:, np.asarray(channels, dtype=np.int64)] *= np.float32(factor)
    return x


def planted_lowrank_weight(rng: np.random.Generator, n: int, k: int, std: float = 0.02, planted: int = 16,
                           lead: float = 4.0, decay: float = 0.7) -> np.ndarray:
    """W [n, k] (binary32) = N(0, std) plus a planted part sum_i s_i u_i v_i^T with
    u_i ~ N(0, 1/n) [n], v_i ~ N(0, 1/k) [k] (nearly unit, nearly orthogonal) and
    s_i = lead * std * (sqrt(n) + sqrt(k)) * decay^i: a few singular directions well
    above the noise's edge, std * (sqrt(n) + sqrt(k)), then decaying into it.
    Drawn in the order noise, u, v."""
    w = gaussian(rng, (n, k), std)
    u = rng.standard_normal((n, planted), dtype=np.float32) / np.float32(np.sqrt(n))
    v = rng.standard_normal((k, planted), dtype=np.float32) / np.float32(np.sqrt(k))
    s = (lead * std * (np.sqrt(n) + np.sqrt(k)) * decay ** np.arange(planted)).astype(np.float32)
    return w + (u * s) @ v.T


def gaussian_test_matrix(rng: np.random.Generator, k: int, rank: int) -> np.ndarray:
    """The random test matrix of the low-rank split: N(0, 1) [k, rank], binary32."""
    return rng.standard_normal((k, rank), dtype=np.float32)


@dataclass(frozen=True)
class AttentionConfig:
    """One attention workload in SDPA's layout: q [batch, heads_q, seq_q, head_dim],
    k and v [batch, heads_kv, seq_k, head_dim]."""
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seq_q: int
    seq_k: int
    head_dim: int
    causal: bool = False
    note: str = ""


# flux.1 joint attention: 3072 wide = 24 heads of 128, 4608 joint tokens (the SD.Next
# dev-branch commit log's block geometry); a causal grouped-query text-encoder
# stand-in for the commit log's causal gqa text-encoder preset; a small case.
ATTENTION_CONFIGS = {
    "attn_tiny": AttentionConfig("attn_tiny", 1, 4, 2, 200, 176, 128, causal=True,
                                 note="ragged tiles, gqa, causal"),
    "attn_flux": AttentionConfig("attn_flux", 1, 24, 24, 4608, 4608, 128,
                                 note="flux.1 joint attention: 24 heads x 128, 4608 tokens"),
    "attn_te": AttentionConfig("attn_te", 2, 16, 4, 1024, 1024, 128, causal=True,
                               note="causal gqa text encoder: 16 query heads over 4 key/value heads"),
}


def make_attention(name: str, seed: int = 0) -> dict:
    """q, k, v (bf16 bits) of a named attention workload, drawn in the order q, k, v:
    q ~ N(0, 1) with 1 % of the head channels x20 (outlier channels, as for the
    linear layer's activations); k the same plus a per-(head, channel) offset
    N(0, 4) shared by all tokens (the channel-wise bias that K smoothing removes);
    v ~ N(0, 1)."""
    c = ATTENTION_CONFIGS[name]
    rng = np.random.default_rng(seed)

    def act(heads, seq):
        x = rng.standard_normal((c.batch, heads, seq, c.head_dim), dtype=np.float32)
        count = max(1, int(round(0.01 * c.head_dim)))
        ch = np.sort(rng.permutation(c.head_dim)[:count])
        x[..., ch] *= np.float32(20.0)
        return x
    q = act(c.heads_q, c.seq_q)
    k = act(c.heads_kv, c.seq_k)
    k += rng.standard_normal((c.batch, c.heads_kv, 1, c.head_dim), dtype=np.float32) * np.float32(4.0)
    v = rng.standard_normal((c.batch, c.heads_kv, c.seq_k, c.head_dim), dtype=np.float32)
    return {"q": to_bf16_bits(q), "k": to_bf16_bits(k), "v": to_bf16_bits(v)}


@dataclass(frozen=True)
class LinearConfig:
    """One workload: activation rows m, in-features k, out-features n."""
    name: str
    m: int
    k: int
    n: int
    groups: tuple = (256,)
    lora_rank: int = 0
    lora_alpha: float = 0.0
    backward: bool = False
    outlier_channels: tuple | None = None
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def lora_scale(self) -> float:
        return self.lora_alpha / self.lora_rank if self.lora_rank else 0.0


# The five workloads of the layer.  "mlp" is two layers: up (k=3840 -> n=10240)
# and down (k=10240 -> n=3840) on a synthetic hidden activation h.
CONFIGS = {
    "tiny": LinearConfig("tiny", 64, 512, 512, outlier_channels=(7, 300),
                         note="x [64,512] N(0,1), channels 7 and 300 x20; W [512,512] N(0,0.02)"),
    "attn": LinearConfig("attn", 4096, 3072, 3072,
                         note="attention projection: x [4096,3072], W [3072,3072]"),
    "mlp_up": LinearConfig("mlp_up", 4096, 3840, 10240, note="MLP up: x [4096,3840], W [10240,3840]"),
    "mlp_down": LinearConfig("mlp_down", 4096, 10240, 3840, note="MLP down: h [4096,10240], W [3840,10240]"),
    "quarot": LinearConfig("quarot", 8192, 3072, 3072, groups=(64, 128), lora_rank=32, lora_alpha=32.0,
                           note="QuaRot-style blocks + LoRA r=32: x [8192,3072], W [3072,3072]"),
    "peft": LinearConfig("peft", 16384, 3072, 3072, lora_rank=64, lora_alpha=32.0, backward=True,
                         note="PEFT step: x, dY [16384,3072], W [3072,3072], LoRA r=64"),
    "svd": LinearConfig("svd", 4096, 3072, 3072, extra={"rank": 32, "steps": 8},
                        note="low-rank split r=32, 8 steps (the SDNQConfig defaults) on the attention "
                             "shape: x [4096,3072]; W [3072,3072] N(0,0.02) + 16 planted directions"),
}


def make_linear(m: int, k: int, n: int, seed: int = 0, outlier_channels=None, lora_rank: int = 0,
                backward: bool = False, dy_std: float = 1e-3) -> dict:
    """Inputs for one linear layer, drawn in the order x, W, [A, B], [dY]."""
    rng = np.random.default_rng(seed)
    out = {"x": to_bf16_bits(outlier_activations(rng, m, k, outlier_channels)),
           "w": to_bf16_bits(gaussian(rng, (n, k), 0.02))}
    if lora_rank:
        out["lora_a"] = to_bf16_bits(gaussian(rng, (k, lora_rank), 0.01))
        out["lora_b"] = to_bf16_bits(gaussian(rng, (lora_rank, n), 0.01))
    if backward:
        out["dy"] = to_bf16_bits(gaussian(rng, (m, n), dy_std))
    return out


def make_config(name: str, seed: int = 0) -> dict:
    """Inputs of a named workload.  For the MLP pair both layers come from one
    stream: x, W_up, h, W_down."""
    if name in ("mlp", "mlp_up", "mlp_down"):
        rng = np.random.default_rng(seed)
        up, down = CONFIGS["mlp_up"], CONFIGS["mlp_down"]
        x = to_bf16_bits(outlier_activations(rng, up.m, up.k))
        w_up = to_bf16_bits(gaussian(rng, (up.n, up.k), 0.02))
        h = to_bf16_bits(outlier_activations(rng, down.m, down.k))
        w_down = to_bf16_bits(gaussian(rng, (down.n, down.k), 0.02))
        if name == "mlp_up":
            return {"x": x, "w": w_up}
        if name == "mlp_down":
            return {"x": h, "w": w_down}
        return {"x": x, "w_up": w_up, "h": h, "w_down": w_down}
    if name == "svd":
        c = CONFIGS["svd"]
        rng = np.random.default_rng(seed)
        x = to_bf16_bits(outlier_activations(rng, c.m, c.k))
        w = to_bf16_bits(planted_lowrank_weight(rng, c.n, c.k))
        omega = gaussian_test_matrix(rng, c.k, c.extra["rank"])
        return {"x": x, "w": w, "omega": omega}
    c = CONFIGS[name]
    return make_linear(c.m, c.k, c.n, seed, c.outlier_channels, c.lora_rank, c.backward)
