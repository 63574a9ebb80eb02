"""Mutation check of the oracle pins (CPU only).

Each case plants one plausible mistake in a scratch copy of the oracle source,
compiles it, and runs the pin suite against that build: the suite must fail.
The clamp bound is left out on purpose: |fl32(y * r)| <= 127 (1 + 2^-23) for
every element, so clamping at -128 instead of -127 changes no output.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "sub_swapped": ("v[i + h] = a - b;", "v[i + h] = b - a;"),
    "stage_order_descending": ("for (int h = 1; h < g; h <<= 1) {", "for (int h = g / 2; h >= 1; h >>= 1) {"),
    "divide_by_scale": ("float t = nearbyintf((y[i] * up) * r);", "float t = nearbyintf(y[i] / *s);"),
    "round_half_away": ("float t = nearbyintf((y[i] * up) * r);", "float t = roundf((y[i] * up) * r);"),
    "no_tiny_row_rescale": ("float up = (a < 0x1p-100f) ? 0x1p100f : 1.0f;", "float up = 1.0f;"),
    "no_normalization": ("y[i] = y[i] * c;", "y[i] = y[i];"),
    "no_column_scale": ("y[i] = y[i] * col_scale[i];", "y[i] = y[i];"),
    "backward_weight_transposed": ("acc[kk] += qv * (int64_t)wr[kk];", "acc[kk] += qv * (int64_t)qw[kk * n + j];"),
    "backward_no_inverse_rotation": ("for (int64_t b = 0; b < k; b += g)\n                        fwht_block(z + b, g);",
                                     "for (int64_t b = 0; b < 0; b += g)\n                        fwht_block(z + b, g);"),
    "scale_over_128": ("*s = a / 127.0f;", "*s = a / 128.0f;"),
    "lora_b_transposed": ("l += t[r] * (double)bf16_decode(lora_b[(int64_t)r * n + j]);",
                          "l += t[r] * (double)bf16_decode(lora_b[(int64_t)j * rank + r]);"),
    "grad_b_unscaled": ("bf16_encode_f64(acc[(int64_t)r * (j_hi - j_lo) + (j - j_lo)] * lora_scale);",
                        "bf16_encode_f64(acc[(int64_t)r * (j_hi - j_lo) + (j - j_lo)]);"),
    "grad_a_wrong_factor": ("acc[(kk - k_lo) * rank + r] += xv * gr[i * rank + r];",
                            "acc[(kk - k_lo) * rank + r] += xv * gr[i * rank + (rank - 1 - r)];"),
    "bf16_truncation": ("double rq = nearbyint(q);", "double rq = floor(q);"),
    "weight_scale_index": ("float base = (float)(int32_t)acc * (sx * sw[j]);",
                           "float base = (float)(int32_t)acc * (sx * sw[i % n]);"),
    "e4m3_truncation": ("double r = nearbyint(ldexp(a, 3 - eu));", "double r = floor(ldexp(a, 3 - eu));"),
    "e4m3_subnormal_step": ("double r = nearbyint(ldexp(a, 9));", "double r = nearbyint(ldexp(a, 10));"),
    "e4m3_exponent_bias": ("(uint8_t)((eu + 7) << 3)", "(uint8_t)((eu + 8) << 3)"),
    "fp8_scale_over_240": ("*s = a / 448.0f;", "*s = a / 240.0f;"),
    "fp8_no_tiny_row_rescale": ("float up = (a < 0x1p-100f) ? 0x1p100f : 1.0f;\n    float as = a * up;\n    float r = (as > 0.0f) ? 448.0f / as : 0.0f;",
                                "float up = 1.0f;\n    float as = a * up;\n    float r = (as > 0.0f) ? 448.0f / as : 0.0f;"),
    "fp8_weight_index": ("acc += dq[kk] * e4m3_decode(wr[kk]);", "acc += dq[kk] * e4m3_decode(wr[(kk + 1) % k]);"),
    "fp8_signed_zero": ("float t = (y[i] * up) * r + 0.0f;", "float t = (y[i] * up) * r;"),
    "fp8_backward_no_fold": ("rotate_row(dy + i * n, n, 1, sw, yr);\n                quantize_row_fp8",
                             "rotate_row(dy + i * n, n, 1, NULL, yr);\n                quantize_row_fp8"),
    "fp8_backward_weight_transposed": ("acc[kk] += dq[j] * e4m3_decode(wr[kk]);",
                                       "acc[kk] += dq[j] * e4m3_decode(qw[kk * n + j]);"),
    "fp8_backward_no_inverse_rotation": ("z[kk] = (float)acc[kk] * sdy;\n                }\n                if (g > 1) {",
                                         "z[kk] = (float)acc[kk] * sdy;\n                }\n                if (0) {"),
    "fp8_backward_scale_dropped": ("z[kk] = (float)acc[kk] * sdy;", "z[kk] = (float)acc[kk];"),
    "fp8_backward_lora_b_transposed": (
        "s += (double)bf16_decode(dy[i * n + j]) * (double)bf16_decode(lora_b[(int64_t)r * n + j]);",
        "s += (double)bf16_decode(dy[i * n + j]) * (double)bf16_decode(lora_b[(int64_t)j * rank + r]);"),
    "f32_input_no_normalization": ("                    for (int64_t i = 0; i < cols; i++)\n                        y[i] = y[i] * c;",
                                   "                    for (int64_t i = 0; i < cols; i++)\n                        y[i] = y[i];"),
}

# Mistakes planted in the Python part of the oracle (the low-rank split).
PY_MUTANTS = {
    "svd_no_subspace_iteration": ("    for _ in range(steps):", "    for _ in range(0):"),
    "svd_residual_against_unrounded_factors": (
        "    lr = f32_from_bf16(b_bits).astype(np.float64).T @ f32_from_bf16(a_bits).astype(np.float64).T",
        "    lr = q @ (q.T @ w)"),
    "svd_residual_sign": ('"residual": (w - lr).astype(np.float32)', '"residual": (lr - w).astype(np.float32)'),
    "svd_one_sided_iteration": ("        z = _orth(w.T @ q)\n        q = _orth(w @ z)",
                                "        z = _orth(w.T @ q)\n        q = _orth(w @ om)"),
    "svd_factor_b_not_orthonormal": ("    b_bits = bf16_from_f64(np.ascontiguousarray(q.T))",
                                     "    b_bits = bf16_from_f64(np.ascontiguousarray((w @ om).T))"),
    "attn_mean_divides_by_head_dim": ("    den = s << 133", "    den = d << 133"),
    "attn_mean_truncates": ("    if 2 * r > d or (2 * r == d and qi & 1):", "    if False:"),
    "attn_mean_ties_away": ("    if 2 * r > d or (2 * r == d and qi & 1):", "    if 2 * r >= d:"),
    "attn_mean_subnormal_keys_get_the_hidden_bit": ("np.where(e > 0, 128, 0)", "128"),
    "attn_mean_binary64_sum": ("    return out.reshape(b, hh, d)\n",
                               "    return (f32_from_bf16(kb).astype(np.float64).sum(axis=2) / s).astype(np.float32)\n"),
    "attn_causal_off_by_one": ("    mask = (np.arange(sk)[None, :] > rows[:, None]) if is_causal else None",
                               "    mask = (np.arange(sk)[None, :] >= rows[:, None]) if is_causal else None"),
    "attn_gqa_modulo": ("            hk = h // rep", "            hk = h % hkv"),
    "attn_smoothing_adds": ("        xf = f32_from_bf16(x_bf16) - np.asarray(offset, np.float32)[:, :, None, :]",
                            "        xf = f32_from_bf16(x_bf16) + np.asarray(offset, np.float32)[:, :, None, :]"),
    "attn_half_head_block": ("    return 1 if g <= 1 else min(g, d)", "    return 1 if g <= 1 else min(g, d) // 2"),
    "attn_scale_dropped": ("                                          ks[b, hk].astype(np.float64)[None, :]) * scale",
                           "                                          ks[b, hk].astype(np.float64)[None, :])"),
}


def _run(name, tmp):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) >= 1, name
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new, 1))
    lib = oracle.build(force=True, src=path, out=os.path.join(tmp, f"lib{name}.so"))
    env = dict(os.environ, SDNQ_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def _run_py(name, tmp):
    """Copy the oracle package with one planted mistake in its Python source and run
    the pins against the copy (it loads the unmodified C library)."""
    old, new = PY_MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert src.count(old) == 1, name
    pkg = os.path.join(tmp, name, "oracle")
    os.makedirs(pkg)
    with open(os.path.join(pkg, "__init__.py"), "w") as f:
        f.write(src.replace(old, new, 1))
    env = dict(os.environ, SDNQ_ORACLE_LIB=oracle.build(force=False), OMP_NUM_THREADS="1",
               PYTHONPATH=os.pathsep.join([os.path.join(tmp, name), ROOT]))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=os.path.join(tmp, name), env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


@pytest.mark.slow
def test_every_planted_python_mistake_is_caught(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = dict(ex.map(lambda n: _run_py(n, str(tmp_path)), sorted(PY_MUTANTS)))
    survivors = [n for n, rc in results.items() if rc == 0]
    assert not survivors, f"pins did not catch: {survivors}"


@pytest.mark.slow
def test_every_planted_mistake_is_caught(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = dict(ex.map(lambda n: _run(n, str(tmp_path)), sorted(MUTANTS)))
    survivors = [n for n, rc in results.items() if rc == 0]
    assert not survivors, f"pins did not catch: {survivors}"
