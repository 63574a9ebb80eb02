"""Throughput of the Hadamard-rotated INT8 linear layer on one MI355X.

Workload (one step): the MLP pair of a transformer block at 4096 tokens,
  up:   x [4096, 3840] bf16 -> rotate (g = 256) + per-token int8 -> GEMM with
        W_up [10240, 3840] int8 -> y_up [4096, 10240] bf16
  down: h [4096, 10240] bf16 -> rotate (g = 256) + per-token int8 -> GEMM with
        W_down [3840, 10240] int8 -> y_down [4096, 3840] bf16
Inputs are seeded synthetic (outlier-channel activations, N(0, 0.02) weights),
resident in HBM before the timed region; the weights are rotated and quantized
once, outside it (offline preparation).

value = int8 ops of both GEMMs (2 M N K each) / wall time per step, in TOPS,
with the activation rotate+quantize kernels inside the step (the timed region
holds nothing else).  Per-kernel launch durations come first, from HIP events on
the launch stream (cold launches, back-to-back launches of each kernel, and whole
steps with an event between the kernels), which also brings the GPU's clock to
its steady state under this load before the warmup steps and the timed region;
the GEMM's back-to-back durations feed the roofline object.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--copy-probe]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0     # MI355X dense INT8 MFMA, 5.0 POP/s
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
M, K_UP, N_UP = 4096, 3840, 10240
K_DOWN, N_DOWN = 10240, 3840
G = 256


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target duration of the CPU oracle sample")
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row timings of the other workloads")
    ap.add_argument("--no-smi", action="store_true",
                    help="do not start rocm-smi for the clock record (under a profiler that preloads into children)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one 256 MiB device-to-device copy first (scales the HBM byte counters)")
    ap.add_argument("--k-sweep", action="store_true",
                    help="also time the GEMM kernel (product and MFMA-only) over K at one and two rounds of tiles")
    return ap.parse_args()


CSRC = os.path.join(ROOT, "hadamard_rotated_int8_amd", "csrc")
# committed rocprofv3 FETCH_SIZE + WRITE_SIZE summaries, and the sources of the
# kernel each was taken on (its own file and the shared device header)
GEMM_TRAFFIC = (os.path.join(ROOT, "profiles", "gemm_i8_mlp_4096tok_hbm_traffic.txt"),
                [os.path.join(CSRC, f) for f in ("gemm_i8.hip", "sdnq_internal.hpp")])
ROTQ_TRAFFIC = (os.path.join(ROOT, "profiles", "rotq_mlp_4096tok_hbm_traffic.txt"),
                [os.path.join(CSRC, f) for f in ("rotq.hip", "sdnq_internal.hpp")])


def source_sha256(files) -> str:
    import hashlib
    return hashlib.sha256(b"".join(open(f, "rb").read() for f in files)).hexdigest()


def measured_traffic(which):
    """HBM bytes per launch (up, down) from a committed rocprofv3 counter summary,
    or None when the kernel's sources have changed since it was taken.  The file
    holds `key: value` lines: source_sha256, up_bytes, down_bytes."""
    path, sources = which
    try:
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("source_sha256") != source_sha256(sources):
            return None
        return [int(kv["up_bytes"]), int(kv["down_bytes"])]
    except (OSError, KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def environment(torch, query_smi: bool = True) -> dict:
    """Device, ROCm and clock information recorded with the numbers (rocm-smi's
    current clocks, read after the timed region; None where unavailable)."""
    props = torch.cuda.get_device_properties(0)
    env = {"device": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
           "compute_units": props.multi_processor_count, "hip": torch.version.hip, "torch": torch.__version__}
    if not query_smi:
        env["clocks"] = None
        return env
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        card = next(iter(json.loads(r.stdout).values())) if r.returncode == 0 else {}
        env["clocks"] = {k: v for k, v in card.items() if "clock" in k.lower() and ("sclk" in k or "mclk" in k
                                                                                   or "fclk" in k)}
    except Exception:  # the tool may be missing or print something else
        env["clocks"] = None
    return env


def to_dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def cpu_baseline(inp, target_s: float) -> dict:
    """The oracle (plain C, OpenMP over rows) on a bounded sample of the same
    workload: the first R token rows of both layers, weights prepared outside;
    on all the threads the oracle uses, then again on one thread."""
    import oracle
    qwu, swu = oracle.rotate_quantize(inp["w_up"], G)
    qwd, swd = oracle.rotate_quantize(inp["w_down"], G)

    def run(rows):
        t0 = time.perf_counter()
        oracle.qlinear_forward(inp["x"][:rows], qwu, swu, G, intermediates=False)
        oracle.qlinear_forward(inp["h"][:rows], qwd, swd, G, intermediates=False)
        return time.perf_counter() - t0

    def sample(target, probe_rows):
        # size the sample from a small probe, then repeat it until about `target` has passed
        probe = run(probe_rows)
        rows = int(min(M, max(probe_rows, probe_rows * target / max(probe, 1e-3))))
        t, reps = 0.0, 0
        while reps == 0 or t < 0.6 * target:
            t += run(rows)
            reps += 1
        ops = 2.0 * rows * reps * (N_UP * K_UP + N_DOWN * K_DOWN)
        return ops / t / 1e12, rows, reps, t

    threads = oracle.num_threads()
    tops, rows, reps, t = sample(target_s, 64)
    oracle.set_num_threads(1)
    try:
        tops1, rows1, reps1, t1 = sample(0.5 * target_s, 8)
    finally:
        oracle.set_num_threads(threads)
    return {"value": round(tops, 6), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
            "sample": f"first {rows} of {M} token rows through both layers, {reps} time(s) (rotate+quantize, "
                      f"exact int GEMM, fp32 dequant, bf16 out); weights prepared outside; {t:.1f} s",
            "seconds": round(t, 2),
            "value_1_thread": round(tops1, 6),
            "sample_1_thread": f"first {rows1} token rows, {reps1} time(s), {t1:.1f} s"}


def measure_rows(torch, h, synth, reps: int = 100, warmup: int = 10) -> dict:
    """Whole-call timings of the other steps of the layer, each on its own
    workload: weight preparation, the attention projection forward, the
    QuaRot-style forward with LoRA (g = 64 and 128), the PEFT backward (input
    gradient + LoRA gradients), the full fine-tuning weight gradient, the FP8
    (E4M3) variant of the MLP step, the low-rank (SVD) split with the forward
    that uses it, and the int8-QK^T attention.  Each is `reps` calls after
    `warmup` untimed ones, every call between two HIP events on the launch
    stream; `us` is the median, `us_min` the minimum."""
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    rows = {}

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        us = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps)])
        return float(np.median(us)), float(us.min())

    def row(key, fn, ops=None, extra=None, peak=INT8_PEAK_TOPS, unit="TOPS"):
        us, us_min = timed(fn)
        r = {"us": round(us, 2), "us_min": round(us_min, 2)}
        if ops is not None:
            r.update({unit: round(ops / us / 1e6, 1), "pct_of_peak": round(ops / us / 1e6 / peak * 100, 2)})
        r.update(extra or {})
        rows[key] = r
        return us

    a = synth.make_config("attn")
    x, w = to_dev_bf16(torch, a["x"]), to_dev_bf16(torch, a["w"])
    nb = 3072 * 3072 * 3 + 3072 * 4
    us = row("a0_weight_prep_3072x3072_g256", lambda: h.sdnq_rotate_quantize_weight(w, 256))
    rows["a0_weight_prep_3072x3072_g256"]["GB/s"] = round(nb / us / 1e3, 1)
    qw, sw = h.sdnq_rotate_quantize_weight(w, 256)
    ws = torch.empty(h.sdnq_workspace_bytes(4096, 3072, 3072, 0, False), dtype=torch.uint8, device=dev)
    y = torch.empty((4096, 3072), dtype=torch.bfloat16, device=dev)
    row("attn_forward_4096x3072x3072_g256", lambda: h.sdnq_qlinear_forward(x, qw, sw, 256, out=y, workspace=ws),
        2.0 * 4096 * 3072 * 3072)
    del x, w, ws, y
    q = synth.make_config("quarot")
    c = synth.CONFIGS["quarot"]
    x, w = to_dev_bf16(torch, q["x"]), to_dev_bf16(torch, q["w"])
    la, lb = to_dev_bf16(torch, q["lora_a"]), to_dev_bf16(torch, q["lora_b"])
    ws = torch.empty(h.sdnq_workspace_bytes(c.m, c.n, c.k, c.lora_rank, False), dtype=torch.uint8, device=dev)
    y = torch.empty((c.m, c.n), dtype=torch.bfloat16, device=dev)
    for g in (64, 128):
        qw, sw = h.sdnq_rotate_quantize_weight(w, g)
        row(f"quarot_lora_forward_8192x3072x3072_g{g}_r32",
            lambda: h.sdnq_qlinear_forward(x, qw, sw, g, la, lb, c.lora_scale, out=y, workspace=ws),
            2.0 * c.m * c.n * c.k)
    del x, w, la, lb, ws, y
    p = synth.make_config("peft")
    c = synth.CONFIGS["peft"]
    x, w, dy = to_dev_bf16(torch, p["x"]), to_dev_bf16(torch, p["w"]), to_dev_bf16(torch, p["dy"])
    la, lb = to_dev_bf16(torch, p["lora_a"]), to_dev_bf16(torch, p["lora_b"])
    qw, sw = h.sdnq_rotate_quantize_weight(w, 256)
    ws = torch.empty(h.sdnq_workspace_bytes(c.m, c.n, c.k, c.lora_rank, True), dtype=torch.uint8, device=dev)
    ops = 2.0 * c.m * c.n * c.k
    # the frozen weight's codes are transposed once, at weight preparation
    qwt = h.sdnq_transpose_codes(qw)
    per_call = timed(lambda: h.sdnq_qlinear_backward_input(dy, qw, sw, 256, x, la, lb, c.lora_scale, workspace=ws))
    row("peft_backward_16384x3072x3072_g256_r64",
        lambda: h.sdnq_qlinear_backward_input_wt(dy, qwt, sw, 256, x, la, lb, c.lora_scale, workspace=ws), ops,
        {"note": "dX through the int8 weight + LoRA dX, dA, dB; weight codes transposed once at preparation",
         "us_codes_transposed_per_call": round(per_call[0], 2)})
    qw8, sw8 = h.sdnq_rotate_quantize_weight_fp8(w, 256)
    qwt8 = h.sdnq_transpose_codes(qw8)
    row("fp8_peft_backward_16384x3072x3072_g256_r64",
        lambda: h.sdnq_qlinear_backward_input_fp8_wt(dy, qwt8, sw8, 256, x, la, lb, c.lora_scale, workspace=ws),
        ops, {"note": "dX through the E4M3 weight + LoRA dX, dA, dB; weight codes transposed once at preparation; "
                      "fp8 dense peak 5.0 PFLOP/s"},
        peak=5000.0, unit="TFLOP/s")
    del qw8, sw8, qwt, qwt8
    wws = torch.empty(h.sdnq_weight_grad_workspace_bytes(c.m, c.n, c.k), dtype=torch.uint8, device=dev)
    dw = torch.empty((c.n, c.k), dtype=torch.bfloat16, device=dev)
    row("weight_grad_16384x3072x3072_g256", lambda: h.sdnq_qlinear_weight_grad(dy, x, 256, out=dw, workspace=wws),
        ops, {"note": "dW = dY^T x, both quantized per feature along the tokens"})
    del wws, dw
    del x, w, dy, la, lb, ws
    # FP8 variant of the MLP step (same workload, E4M3 codes, fp32 MFMA accumulation)
    inp = synth.make_config("mlp")
    x, hh = to_dev_bf16(torch, inp["x"]), to_dev_bf16(torch, inp["h"])
    qwu, swu = h.sdnq_rotate_quantize_weight_fp8(to_dev_bf16(torch, inp["w_up"]), 256)
    qwd, swd = h.sdnq_rotate_quantize_weight_fp8(to_dev_bf16(torch, inp["w_down"]), 256)
    qx = torch.empty((M, K_UP), dtype=torch.uint8, device=dev)
    sx = torch.empty((M,), dtype=torch.float32, device=dev)
    qh = torch.empty((M, K_DOWN), dtype=torch.uint8, device=dev)
    sh = torch.empty((M,), dtype=torch.float32, device=dev)
    yu = torch.empty((M, N_UP), dtype=torch.bfloat16, device=dev)
    yd = torch.empty((M, N_DOWN), dtype=torch.bfloat16, device=dev)
    L = h.lib()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    gemm_up = lambda: L.sdnq_qlinear_forward_fp8_quantized(P(qx), P(sx), M, K_UP, P(qwu), P(swu), N_UP, None, None,
                                                           0, 0.0, P(yu), None, 0, sp)
    gemm_down = lambda: L.sdnq_qlinear_forward_fp8_quantized(P(qh), P(sh), M, K_DOWN, P(qwd), P(swd), N_DOWN,
                                                             None, None, 0, 0.0, P(yd), None, 0, sp)

    def step8():
        L.sdnq_rotate_quantize_act_fp8(P(x), M, K_UP, G, None, P(qx), P(sx), sp)
        gemm_up()
        L.sdnq_rotate_quantize_act_fp8(P(hh), M, K_DOWN, G, None, P(qh), P(sh), sp)
        gemm_down()
    ops = 2.0 * M * (N_UP * K_UP + N_DOWN * K_DOWN)
    (t_up, _), (t_down, _) = timed(gemm_up), timed(gemm_down)
    gemm_tflops = ops / (t_up + t_down) / 1e6
    row("fp8_mlp_step_4096tok_g256", step8, ops,
        {"gemm_up_us": round(t_up, 2), "gemm_down_us": round(t_down, 2), "gemm_TFLOP/s": round(gemm_tflops, 1),
         "gemm_pct_of_fp8_peak": round(gemm_tflops / 50.0, 2),
         "note": "E4M3 codes, fp32 MFMA accumulation; GEMM medians timed alone; fp8 dense peak 5.0 PFLOP/s"},
        peak=5000.0, unit="TFLOP/s")
    del x, hh, qwu, qwd, qx, qh, yu, yd
    # low-rank (SVD) split: offline preparation of W [3072, 3072] (rank 32, 8 steps),
    # then the forward with the factors as the LoRA term
    sv = synth.make_config("svd")
    c = synth.CONFIGS["svd"]
    r, steps = c.extra["rank"], c.extra["steps"]
    x, w = to_dev_bf16(torch, sv["x"]), to_dev_bf16(torch, sv["w"])
    omega = torch.from_numpy(sv["omega"]).to(dev)
    sws = torch.empty(h.sdnq_svd_workspace_bytes(c.n, c.k, r), dtype=torch.uint8, device=dev)
    row("svd_split_prep_3072x3072_r32_s8_g256", lambda: h.sdnq_svd_quantize_weight(w, 256, omega, steps, workspace=sws),
        extra={"note": "offline: randomized range finder, 8 subspace iterations, fp64 thin products"})
    qw, sw, sa, sb = h.sdnq_svd_quantize_weight(w, 256, omega, steps, workspace=sws)
    del sws
    ws = torch.empty(h.sdnq_workspace_bytes(c.m, c.n, c.k, r, False), dtype=torch.uint8, device=dev)
    y = torch.empty((c.m, c.n), dtype=torch.bfloat16, device=dev)
    row("svd_forward_4096x3072x3072_g256_r32",
        lambda: h.sdnq_qlinear_forward(x, qw, sw, 256, sa, sb, 1.0, out=y, workspace=ws), 2.0 * c.m * c.n * c.k,
        {"note": "int8 residual + bf16 rank-32 factors in the epilogue"})
    del x, w, omega, qw, sw, sa, sb, ws, y
    # int8-QK^T attention: flux.1 joint attention and a causal grouped-query text encoder
    for name in ("attn_flux", "attn_te"):
        ac = synth.ATTENTION_CONFIGS[name]
        ai = synth.make_attention(name)
        q, k, v = (to_dev_bf16(torch, ai[t]) for t in ("q", "k", "v"))
        aws = torch.empty(h.sdnq_attention_workspace_bytes(ac.batch, ac.heads_q, ac.heads_kv, ac.seq_q, ac.seq_k,
                                                           ac.head_dim), dtype=torch.uint8, device=dev)
        o = torch.empty_like(q)
        pairs = ac.seq_q * ac.seq_k * (0.5 if ac.causal else 1.0)
        ops = 4.0 * ac.batch * ac.heads_q * pairs * ac.head_dim
        ref_us, _ = timed(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=ac.causal,
                                                                                   enable_gqa=True))
        us, us_min = timed(lambda: h.sdnq_attention_int8(q, k, v, ac.causal, None, True, 256, out=o, workspace=aws))
        rows[f"attention_int8_{name[5:]}_{ac.batch}x{ac.heads_q}x{ac.seq_q}x{ac.head_dim}"] = {
            "us": round(us, 2), "us_min": round(us_min, 2), "TOPS": round(ops / us / 1e6, 1),
            "torch_sdpa_bf16_us": round(ref_us, 2),
            "note": "whole call (K mean, rotate+quantize of Q and K, V transpose, int8 QK^T / bf16 PV kernel); "
                    "ops = 2 (QK^T) + 2 (PV) per query-key pair and head dimension"}
        del q, k, v, aws, o
    return rows


def gemm_k_sweep(torch, L, P, sp, stream, check) -> dict:
    """Launch duration of the forward GEMM kernel (sdnq_gemm_i8_ceiling mode 0, the
    product kernel, and mode 2, its MFMA instructions alone) against K, with N = 10240
    (256 x 320 tiles) at M = 2048 (one round of 256 tiles) and 4096 (two rounds);
    a line t = fixed + slope * K through the medians splits each launch into its
    k loop and its per-launch fixed part."""
    dev = torch.device("cuda", 0)
    n, ks, ms = 10240, (1920, 3840, 5760, 7680), (2048, 4096)
    gen = torch.Generator(device="cpu").manual_seed(7)
    a_all = torch.randint(-127, 128, (max(ms), max(ks)), dtype=torch.int8, generator=gen).to(dev)
    b_all = torch.randint(-127, 128, (n, max(ks)), dtype=torch.int8, generator=gen).to(dev)
    sa = (torch.rand(max(ms), generator=gen) * 1e-3 + 1e-4).to(dev)
    sb = (torch.rand(n, generator=gen) * 1e-3 + 1e-4).to(dev)
    y = torch.empty((max(ms), n), dtype=torch.bfloat16, device=dev)
    ops = {k: (a_all[:, :k].contiguous(), b_all[:, :k].contiguous()) for k in ks}
    res = {}
    for p in range(3):
        for mode in ((0, 2) if p % 2 == 0 else (2, 0)):
            for m in ms:
                for k in ks:
                    a, b = ops[k]
                    c = lambda: check(L.sdnq_gemm_i8_ceiling(P(a), P(sa), m, k, P(b), P(sb), n, mode, P(y), sp),
                                      "k sweep")
                    for _ in range(5):
                        c()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    for _ in range(30):
                        c()
                    e1.record(stream)
                    torch.cuda.synchronize()
                    res.setdefault((mode, m, k), []).append(e0.elapsed_time(e1) * 1e3 / 30)
    fits = {}
    for mode in (0, 2):
        for m in ms:
            ts = np.array([np.median(res[(mode, m, k)]) for k in ks])
            slope, fixed = np.polyfit(np.array(ks, dtype=float), ts, 1)
            fits[f"mode{mode}_m{m}"] = {"us": [round(float(t), 2) for t in ts], "fixed_us": round(float(fixed), 2),
                                        "us_per_1000_k": round(float(slope) * 1000, 3)}
    del ops, a_all, b_all, y
    return {"n": n, "k": list(ks), "m": list(ms), "rounds_of_tiles": {"2048": 1, "4096": 2}, "fits": fits,
            "timing": "median over 3 passes of the mean over 30 back-to-back launches between two HIP events"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import hadamard_rotated_int8_amd as h
    from hadamard_rotated_int8_amd import synth

    L = h.lib()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    inp = synth.make_config("mlp", seed=0)
    x, hh = to_dev_bf16(torch, inp["x"]), to_dev_bf16(torch, inp["h"])
    w_up, w_down = to_dev_bf16(torch, inp["w_up"]), to_dev_bf16(torch, inp["w_down"])
    qw_up, sw_up = h.sdnq_rotate_quantize_weight(w_up, G)
    qw_down, sw_down = h.sdnq_rotate_quantize_weight(w_down, G)
    del w_up, w_down
    qx = torch.empty((M, K_UP), dtype=torch.int8, device=dev)
    sx = torch.empty((M,), dtype=torch.float32, device=dev)
    qh = torch.empty((M, K_DOWN), dtype=torch.int8, device=dev)
    shh = torch.empty((M,), dtype=torch.float32, device=dev)
    y_up = torch.empty((M, N_UP), dtype=torch.bfloat16, device=dev)
    y_down = torch.empty((M, N_DOWN), dtype=torch.bfloat16, device=dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {h.status_string(rc)}")

    kernels = ["rotq_up", "gemm_up", "rotq_down", "gemm_down"]

    calls = [
        lambda: check(L.sdnq_rotate_quantize_act(P(x), M, K_UP, G, None, P(qx), P(sx), sp), "rotq up"),
        lambda: check(L.sdnq_qlinear_forward_quantized(P(qx), P(sx), M, K_UP, P(qw_up), P(sw_up), N_UP, None, None,
                                                       0, 0.0, P(y_up), None, 0, sp), "gemm up"),
        lambda: check(L.sdnq_rotate_quantize_act(P(hh), M, K_DOWN, G, None, P(qh), P(shh), sp), "rotq down"),
        lambda: check(L.sdnq_qlinear_forward_quantized(P(qh), P(shh), M, K_DOWN, P(qw_down), P(sw_down), N_DOWN,
                                                       None, None, 0, 0.0, P(y_down), None, 0, sp), "gemm down"),
    ]

    def step():
        for c in calls:
            c()

    if args.copy_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Per-kernel characterization, before the warmup and the timed region.  The
    # GPU's power manager needs about 10-15 ms of sustained load to settle (the
    # clock first boosts, then dips below its steady value, then recovers); run
    # after the timed region with a short warmup, the timed steps would fall into
    # that dip.  Here they run at the steady state that a training or serving loop
    # sees, and these per-kernel figures are taken in it too.
    n_char = max(args.steps, 50)

    # cold launches: a 1 GiB read before each one evicts the operands from the
    # 256 MB MALL without leaving dirty lines behind
    scrub = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    cold = np.zeros((20, 4))
    for i in range(cold.shape[0]):
        for j, c in enumerate(calls):
            scrub.max()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            c()
            e1.record(stream)
            torch.cuda.synchronize()
            cold[i, j] = e0.elapsed_time(e1)
    del scrub

    # per-kernel launch duration: HIP events on the launch stream around n_char
    # back-to-back launches of each kernel (same inputs as in the step), in 5
    # passes that alternate the kernel order; the up GEMM of the first and the
    # last pass doubles as a drift sentinel (clock or thermal drift over the run)
    n_pass = 5
    b2b = np.zeros((n_pass, 4))
    for p in range(n_pass):
        for j in (range(4) if p % 2 == 0 else reversed(range(4))):
            c = calls[j]
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for _ in range(5):
                c()
            e0.record(stream)
            for _ in range(n_char):
                c()
            e1.record(stream)
            torch.cuda.synchronize()
            b2b[p, j] = e0.elapsed_time(e1) / n_char
    avg_ms = np.median(b2b, axis=0)

    # GEMM ceiling: the same kernel with the global loads of its k loop removed
    # (mode 1), then also its LDS fragment reads (mode 2: the MFMA instructions
    # alone, on operand bytes of the real codes; mode 3: on loop-index operands),
    # timed like the launches above in 3 passes of alternating order.  Mode 0 is
    # the product launch itself.
    y_ceil = [torch.empty_like(y_up), torch.empty_like(y_down)]
    ceil_args = [(qx, sx, M, K_UP, qw_up, sw_up, N_UP), (qh, shh, M, K_DOWN, qw_down, sw_down, N_DOWN)]

    def ceiling_call(mode, i):
        a, sa, m, k, b, sb, n = ceil_args[i]
        return lambda: check(L.sdnq_gemm_i8_ceiling(P(a), P(sa), m, k, P(b), P(sb), n, mode, P(y_ceil[i]), sp),
                             f"gemm ceiling mode {mode}")

    n_modes = 4
    ceil_jobs = [(mode, i) for mode in range(n_modes) for i in (0, 1)]
    ceil = np.zeros((3, len(ceil_jobs)))
    for p in range(3):
        for j in (range(len(ceil_jobs)) if p % 2 == 0 else reversed(range(len(ceil_jobs)))):
            c = ceiling_call(*ceil_jobs[j])
            for _ in range(5):
                c()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n_char):
                c()
            e1.record(stream)
            torch.cuda.synchronize()
            ceil[p, j] = e0.elapsed_time(e1) / n_char
    ceil_ms = np.median(ceil, axis=0).reshape(n_modes, 2)
    del y_ceil

    # Vendor reference for the GEMM: torch._int_mm (hipBLASLt) on the same operand
    # bytes, int32 out (no scales, no bf16 epilogue), timed the same way.
    vendor_ms = None
    try:
        wt = [qw_up.t(), qw_down.t()]  # [K, N] views of the row-major weights
        vcalls = [lambda: torch._int_mm(qx, wt[0]), lambda: torch._int_mm(qh, wt[1])]
        vend = np.zeros((3, 2))
        for p in range(3):
            for j in ((0, 1) if p % 2 == 0 else (1, 0)):
                for _ in range(5):
                    vcalls[j]()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(n_char):
                    vcalls[j]()
                e1.record(stream)
                torch.cuda.synchronize()
                vend[p, j] = e0.elapsed_time(e1) / n_char
        vendor_ms = np.median(vend, axis=0)
        del wt
    except (RuntimeError, AttributeError) as e:  # torch without the int8 matmul
        vendor_note = f"torch._int_mm unavailable: {e}"
    else:
        vendor_note = ("torch._int_mm (hipBLASLt) on the same int8 operands, int32 out (no scales or bf16 "
                       "epilogue), timed like the kernels")

    # Same-traffic reference for rotate+quantize: a device-to-device copy that
    # moves as many bytes as the kernel does for x and for h (3 bytes per element:
    # 1.5 read and 1.5 written), timed the same way.
    cp_n = [M * K_UP * 3 // 2, M * K_DOWN * 3 // 2]
    cp_src = torch.empty(max(cp_n), dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    cast_calls = [lambda: cp_dst[:cp_n[0]].copy_(cp_src[:cp_n[0]]), lambda: cp_dst[:cp_n[1]].copy_(cp_src[:cp_n[1]])]
    cast = np.zeros((3, 2))
    for p in range(3):
        for j in ((0, 1) if p % 2 == 0 else (1, 0)):
            for _ in range(5):
                cast_calls[j]()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n_char):
                cast_calls[j]()
            e1.record(stream)
            torch.cuda.synchronize()
            cast[p, j] = e0.elapsed_time(e1) / n_char
    cast_ms = np.median(cast, axis=0)
    del cp_src, cp_dst

    # per-kernel times inside steps: n_char steps with HIP events on the launch
    # stream between the kernels (each event pair adds about 5 us to the kernel
    # it brackets)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_char)]
    for i in range(n_char):
        evs[i][0].record(stream)
        for j, c in enumerate(calls):
            c()
            evs[i][j + 1].record(stream)
    torch.cuda.synchronize()
    in_step_all = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(4)]
                            for i in range(n_char)])
    in_step_ms = in_step_all.mean(axis=0)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_per_step = wall * 1e3 / args.steps
    ops_up = 2.0 * M * N_UP * K_UP
    ops_down = 2.0 * M * N_DOWN * K_DOWN
    tops = (ops_up + ops_down) / (ms_per_step * 1e-3) / 1e12

    # Launch durations from the back-to-back passes (median over the passes, so
    # the first one, still in the power manager's settling, does not count): the
    # events' marker processing is amortized over n_char launches, and the
    # kernel trace of the timed steps agrees with these within about 1 %.  An
    # event pair around each launch inside the steps adds 5-15 us to the launch
    # it brackets (in_step figures, reported beside them).
    gemm_tops = (ops_up + ops_down) / ((avg_ms[1] + avg_ms[3]) * 1e-3) / 1e12
    in_step_tops = (ops_up + ops_down) / ((in_step_ms[1] + in_step_ms[3]) * 1e-3) / 1e12
    rot_bytes = (M * K_UP * 3 + M * 4) + (M * K_DOWN * 3 + M * 4)  # bf16 in, int8 out, fp32 scale
    rot_s = (avg_ms[0] + avg_ms[2]) * 1e-3
    rot_gbs = rot_bytes / rot_s / 1e9

    traffic = measured_traffic(GEMM_TRAFFIC)
    rot_traffic = measured_traffic(ROTQ_TRAFFIC)
    out = {
        "metric": "INT8 TOPS of fused Hadamard-quantized linear, % of MI355X INT8 MFMA peak",
        "value": round(tops, 2),
        "unit": "TOPS",
        "pct_of_peak": round(100.0 * tops / INT8_PEAK_TOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "MLP up+down of one block: x[4096,3840] -> W_up[10240,3840], "
                               "h[4096,10240] -> W_down[3840,10240], Hadamard block 256, per-token int8 "
                               "activations, row-wise int8 weights, bf16 out",
                   "tokens": M, "hadamard_group": G},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 1), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "traffic": None if traffic is None else int(sum(traffic) / 2),
                     "traffic_per_launch": traffic,
                     "kernel": "gemm_i8_kernel (forward epilogue)",
                     "timing": "median over 5 passes (alternating kernel order) of the mean launch duration "
                               "over max(K, 50) back-to-back launches between two HIP events on the launch stream",
                     "achieved_in_step_events": round(in_step_tops, 1),
                     "per_launch_frac": [round(ops_up / (avg_ms[1] * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                                         round(ops_down / (avg_ms[3] * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)],
                     "per_launch_ops": [ops_up, ops_down]},
        "rotate_quantize_roofline": {"bound": "hbm", "achieved": round(rot_gbs, 1), "peak": HBM_PEAK_GBS,
                                     "unit": "GB/s", "frac": round(rot_gbs / HBM_PEAK_GBS, 4),
                                     "traffic": None if rot_traffic is None else int(sum(rot_traffic) / 2),
                                     "traffic_per_launch": rot_traffic,
                                     "per_launch_bytes": [M * K_UP * 3 + M * 4, M * K_DOWN * 3 + M * 4],
                                     "kernel": "rotq_kernel (x [4096, 3840], h [4096, 10240])",
                                     "same_traffic_copy_us": [round(float(v) * 1e3, 2) for v in cast_ms],
                                     "same_traffic_copy_frac": round(
                                         (M * K_UP * 3 + M * K_DOWN * 3) / float(cast_ms.sum() * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 4),
                                     "same_traffic_copy_note": "device-to-device copies moving the kernel's bytes "
                                                               "for x and for h (1.5 bytes read and 1.5 written "
                                                               "per element), timed like the kernel",
                                     "timing": "median over 5 passes (alternating kernel order) of the mean launch "
                                               "duration over max(K, 50) back-to-back launches between two "
                                               "HIP events on the launch stream"},
        "gemm_ceiling": {
            "entry_point": "sdnq_gemm_i8_ceiling (the forward GEMM kernel with parts of its k loop removed)",
            "modes": ["0: the product kernel", "1: no global loads in the k loop (MFMA + LDS fragment reads)",
                      "2: no global loads and no LDS reads (MFMA instructions on the first fragments' bytes)",
                      "3: as 2 with operands made of loop indices (few toggling bits)"],
            "us_up_down": [[round(float(v) * 1e3, 2) for v in ceil_ms[mode]] for mode in range(n_modes)],
            "frac_of_peak_up_down": [[round(ops / (float(v) * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)
                                      for ops, v in zip((ops_up, ops_down), ceil_ms[mode])] for mode in range(n_modes)],
            "product_over_mode2": [round(float(ceil_ms[2, i] / ceil_ms[0, i]), 4) for i in range(2)],
            "vendor_int8_gemm_us_up_down": None if vendor_ms is None else [round(float(v) * 1e3, 2)
                                                                           for v in vendor_ms],
            "vendor_int8_gemm_frac_up_down": None if vendor_ms is None else [
                round(ops / (float(v) * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)
                for ops, v in zip((ops_up, ops_down), vendor_ms)],
            "vendor_note": vendor_note,
            "timing": "median over 3 passes (alternating order) of the mean launch duration over max(K, 50) "
                      "back-to-back launches between two HIP events on the launch stream"},
        "kernel_avg_us": {k: round(float(v) * 1e3, 2) for k, v in zip(kernels, avg_ms)},
        "kernel_back_to_back_passes_us": {k: [round(float(v) * 1e3, 2) for v in b2b[:, j]]
                                          for j, k in enumerate(kernels)},
        "drift_sentinel": {"kernel": "gemm_up back-to-back", "first_pass_us": round(float(b2b[0, 1]) * 1e3, 2),
                           "last_pass_us": round(float(b2b[-1, 1]) * 1e3, 2),
                           "ratio": round(float(b2b[-1, 1] / b2b[0, 1]), 4)},
        "kernel_avg_sum_ms": round(float(avg_ms.sum()), 4),
        "kernel_in_step_us": {k: round(float(v) * 1e3, 2) for k, v in zip(kernels, in_step_ms)},
        "kernel_in_step_sum_ms": round(float(in_step_ms.sum()), 4),
        "kernel_in_step_note": "HIP events around every launch inside the steps; each event pair adds several us "
                               "to the launch it brackets, so these overstate the kernels (kernel_avg_us is the "
                               "figure the rooflines use)",
        "kernel_in_step_median_min_us": {k: [round(float(np.median(in_step_all[:, j])) * 1e3, 2),
                                             round(float(in_step_all[:, j].min()) * 1e3, 2)]
                                         for j, k in enumerate(kernels)},
        "kernel_cold_median_min_us": {k: [round(float(np.median(cold[:, j])) * 1e3, 2),
                                          round(float(cold[:, j].min()) * 1e3, 2)]
                                      for j, k in enumerate(kernels)},
        "env": environment(torch, not args.no_smi),
    }
    if args.k_sweep:
        out["gemm_k_sweep"] = gemm_k_sweep(torch, L, P, sp, stream, check)
    if not args.no_rows:
        out["rows"] = measure_rows(torch, h, synth)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
