"""Benchmark of the blockwise-scaled FP8 linear layer on one MI355X.

One step = the FP8 forward of the four Llama-3.1-8B-shaped linear layers at
4096 tokens (QKV 4096->6144, O 4096->4096, gate+up 4096->28672, down
14336->4096): per layer, dynamic 1x128 activation quantization followed by the
block-scaled FP8 GEMM (fp32 accumulation, bf16 output).  The weights are
quantized (128x128 blocks) before the timed region, as they are once per
policy update; the recalibration pass over all 128 linear weights of the
32-layer model is timed separately.  Inputs are seeded synthetic tensors
(no checkpoints, no datasets), resident in HBM when timing starts.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0    # MI355X dense FP8 MFMA, TFLOP/s
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense BF16 MFMA, TFLOP/s
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def act_quant_bytes(M, K):
    """Algorithmic bytes of one 1x128 activation quantization: 2 B read and
    1 B written per element, 4 B per block scale."""
    return M * K * 3 + (M * K // 128) * 4


def weight_quant_bytes(N, K):
    return N * K * 3 + (N // 128) * (K // 128) * 4


GEMM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_dense_llama4096_traffic.txt")
GEMM_SOURCES = ("blockwise_scaled_fp8_quant_amd/csrc/gemm.hip",
                "blockwise_scaled_fp8_quant_amd/csrc/fp8q_device.h")


def gemm_source_digest():
    """sha256 over the GEMM kernel's sources and its compile flags (what
    decides the kernel binary the counters were taken on)."""
    import hashlib
    from blockwise_scaled_fp8_quant_amd import build as hip_build
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    h.update(repr((hip_build.ARCH, hip_build.COMMON)).encode())
    return h.hexdigest()


def gemm_traffic_per_launch():
    """HBM bytes per GEMM launch (average over the four layer shapes) from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, scaled by the
    copy-kernel calibration stored with it; None when the summary is missing
    or was taken on other kernel sources."""
    try:
        with open(GEMM_TRAFFIC_FILE) as f:
            kv = dict(line.split("=", 1) for line in f.read().splitlines()
                      if "=" in line and not line.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if kv.get("source_sha256") != gemm_source_digest():
            return None
        return float(kv["calibrated_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def calibration_copy(torch, dev, nbytes=1 << 30, reps=3):
    """A plain copy of known size (read nbytes, write nbytes) for scaling the
    HBM counters of a profiler run."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def copy_bandwidth(torch, dev, nbytes=1 << 30, reps=10):
    """GB/s (bytes read + written) of a plain 1 GiB elementwise copy: what a
    streaming kernel can reach on this HBM, next to the 8 TB/s spec figure."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    t = time_loop(lambda: torch.neg(src, out=dst), reps, torch, label="copy_1gib")
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / t / 1e9


# Per-launch statistics of every timed figure: label -> mean, median and
# minimum in microseconds over the launches of its loop.
STATS = {}


def _stat(label, mean_s, durs_us):
    """mean_us: the loop's back-to-back mean; median_us, min_us: over the same
    number of launches, each bracketed by its own events."""
    d = sorted(durs_us)
    n = len(d)
    med = d[n // 2] if n % 2 else 0.5 * (d[n // 2 - 1] + d[n // 2])
    STATS[label] = {"mean_us": round(mean_s * 1e6, 2), "median_us": round(med, 2), "min_us": round(d[0], 2),
                    "n": n}


def time_loop(fn, reps, torch, label=None, warmup=2):
    """Average duration (s) of fn() over reps back-to-back launches, HIP events
    on the current stream (the stream the library enqueues on), after warmup
    untimed calls (a kernel's first launch in the process also loads its code
    and sets its attributes).  With a label, a second loop brackets every
    launch with its own events and its median and minimum go to STATS beside
    this mean (the per-launch event records add gaps between launches, so the
    mean comes from the first loop only)."""
    Ev = torch.cuda.Event
    start, end = Ev(enable_timing=True), Ev(enable_timing=True)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    torch.cuda.synchronize()
    mean = start.elapsed_time(end) / 1e3 / reps
    if label:
        evs = [(Ev(enable_timing=True), Ev(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        _stat(label, mean, [a.elapsed_time(b) * 1e3 for a, b in evs])
    return mean


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 50 steps (~50 ms of load): the GPU's clock settles within them; after 5
    # the first timed steps still run ~7% slower
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-rows", type=int, default=64,
                    help="tokens per layer in the oracle's single-thread CPU-baseline sample")
    ap.add_argument("--sections",
                    default="pow2,fused,norm,backward,recal,moe,dispatch,attention,smallm,bf16,power,cpu",
                    help="extra measurements after the step (comma list of pow2, fused, norm, backward, recal, "
                         "moe, dispatch, attention, smallm, bf16, power, cpu)")
    ap.add_argument("--skip-extras", action="store_true",
                    help="only the step (for profiler runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run a 1 GiB copy kernel first (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(it times the kernels on one GPU; a multi-GPU run is not part of it)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import blockwise_scaled_fp8_quant_amd as fp8q
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("library", fp8q.library_path())
    if args.calib_copy:
        calibration_copy(torch, dev)

    # ---- inputs of the step (Llama-3.1-8B-shaped layers, 4096 tokens) ----
    M = synth.LLAMA_TOKENS
    layers = []
    for i, (name, N, K) in enumerate(synth.LLAMA_LAYERS):
        x, w = synth.llama_layer_inputs(i, device=dev)
        bq, bs = fp8q.fp8_quant_weight_128x128(w)
        aq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        as_ = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        layers.append(dict(name=name, N=N, K=K, x=x, w=w, bq=bq, bs=bs, aq=aq, as_=as_, y=y))
    torch.cuda.synchronize()
    step_flops = sum(2.0 * M * l["N"] * l["K"] for l in layers)

    def step():
        for l in layers:
            fp8q.fp8_quant_act_1x128(l["x"], out=(l["aq"], l["as_"]))
            fp8q.fp8_blockscaled_gemm(l["aq"], l["as_"], l["bq"], l["bs"], out=l["y"])

    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region.  HIP events on the current stream (the one the library
    # enqueues on) bracket the whole region and, inside it, every launch, so
    # the per-kernel averages come from the same launches as the step time.
    log("timing", args.steps, "steps")
    Ev = torch.cuda.Event
    marks = [[(Ev(enable_timing=True), Ev(enable_timing=True), Ev(enable_timing=True))
              for _ in layers] for _ in range(args.steps)]
    start, end = Ev(enable_timing=True), Ev(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        for l, (e0, e1, e2) in zip(layers, marks[s]):
            e0.record()
            fp8q.fp8_quant_act_1x128(l["x"], out=(l["aq"], l["as_"]))
            e1.record()
            fp8q.fp8_blockscaled_gemm(l["aq"], l["as_"], l["bq"], l["bs"], out=l["y"])
            e2.record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s = start.elapsed_time(end) / 1e3 / args.steps
    value = step_flops / step_s / 1e12
    log(f"step {step_s * 1e3:.3f} ms  ({wall:.3f} s wall for {args.steps} steps)  {value:.1f} TFLOP/s")
    in_step = {l["name"]: {"quant_s": 0.0, "gemm_s": 0.0} for l in layers}
    for s in range(args.steps):
        for l, (e0, e1, e2) in zip(layers, marks[s]):
            in_step[l["name"]]["quant_s"] += e0.elapsed_time(e1) / 1e3 / args.steps
            in_step[l["name"]]["gemm_s"] += e1.elapsed_time(e2) / 1e3 / args.steps
    _stat("step", step_s, [marks[s][0][0].elapsed_time(marks[s][-1][2]) * 1e3 for s in range(args.steps)])
    for i, l in enumerate(layers):
        _stat(f"step/{l['name']}/gemm", in_step[l["name"]]["gemm_s"],
              [marks[s][i][1].elapsed_time(marks[s][i][2]) * 1e3 for s in range(args.steps)])
        _stat(f"step/{l['name']}/act_quant", in_step[l["name"]]["quant_s"],
              [marks[s][i][0].elapsed_time(marks[s][i][1]) * 1e3 for s in range(args.steps)])

    result = {
        "metric": "block-scaled FP8 GEMM TFLOP/s (% FP8 MFMA peak); quantize GB/s (% HBM)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 x fp8_e4m3 -> fp32 accumulate -> bf16",
        "data": "synthetic (seeded N(0,1) activations with 1% outlier channels x20, N(0,0.02) weights)",
        "config": {
            "workload": "Llama-3.1-8B-shaped FP8 linear layers (QKV, O, gate+up, down), 4096 tokens: "
                        "1x128 activation quantization + block-scaled FP8 GEMM per layer",
            "tokens": M,
            "layers": [[l["name"], l["N"], l["K"]] for l in layers],
            "weight_blocks": "128x128", "activation_blocks": "1x128", "scale_mode": "amax/448",
            "parallelism": "single GPU",
        },
    }

    # ---- per-kernel figures from the timed region ----
    reps = max(20, args.steps)
    gemm_s, gemm_flops, per_layer = 0.0, 0.0, {}
    for l in layers:
        t = in_step[l["name"]]["gemm_s"]
        tq = in_step[l["name"]]["quant_s"]
        f = 2.0 * M * l["N"] * l["K"]
        gemm_s += t
        gemm_flops += f
        per_layer[l["name"]] = {"gemm_us": round(t * 1e6, 2), "gemm_tflops": round(f / t / 1e12, 1),
                                "act_quant_in_step_us": round(tq * 1e6, 2)}
    gemm_tflops = gemm_flops / gemm_s / 1e12
    gemm_avg_us = gemm_s / len(layers) * 1e6
    log(f"gemm {gemm_tflops:.1f} TFLOP/s over the 4 layers (average launch {gemm_avg_us:.2f} us)")

    # activation quantization: rotate through >= 1 GB of distinct inputs so the
    # 256 MB last-level cache cannot hold them
    q_s, q_bytes = 0.0, 0.0
    for l in layers:
        K = l["K"]
        nrot = max(1, int(np.ceil(1.2e9 / (M * K * 3))))
        xs = [l["x"]] + [torch.randn((M, K), device=dev, dtype=torch.float32).to(torch.bfloat16)
                         for _ in range(nrot - 1)]
        ctr = [0]

        def qa(l=l, xs=xs, ctr=ctr):
            fp8q.fp8_quant_act_1x128(xs[ctr[0] % len(xs)], out=(l["aq"], l["as_"]))
            ctr[0] += 1
        t = time_loop(qa, reps * len(xs), torch, label=f"act_quant/{l['name']}")
        b = act_quant_bytes(M, K)
        q_s += t
        q_bytes += b
        per_layer[l["name"]].update(act_quant_us=round(t * 1e6, 2), act_quant_gbs=round(b / t / 1e9, 1))
        del xs
    act_gbs = q_bytes / q_s / 1e9
    log(f"act quant {act_gbs:.1f} GB/s")

    copy_gbs = copy_bandwidth(torch, dev)
    log(f"copy kernel {copy_gbs:.1f} GB/s")

    result["kernels"] = {
        "gemm_tflops": round(gemm_tflops, 1),
        "gemm_frac_fp8_peak": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
        "act_quant_gbs": round(act_gbs, 1),
        "act_quant_frac_hbm": round(act_gbs / HBM_PEAK_GBS, 4),
        "hbm_copy_gbs": round(copy_gbs, 1),
        "act_quant_frac_copy": round(act_gbs / copy_gbs, 4),
        "per_layer": per_layer,
    }
    result["roofline"] = {
        "kernel": "gemm_kernel (dense block-scaled FP8 GEMM), 4 Llama layer shapes",
        "bound": "mfma",
        "achieved": round(gemm_tflops, 1),
        "peak": FP8_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
        "traffic": gemm_traffic_per_launch(),
        "launch_us": round(gemm_avg_us, 2),
        "flops_per_launch": gemm_flops / len(layers),
    }

    sections = set() if args.skip_extras else set(args.sections.split(","))
    if "pow2" in sections:
        result["pow2"] = pow2_gemm(fp8q, layers, torch, M, reps)
    if "fused" in sections:
        result["fused_output_quant"] = fused_output_quant(fp8q, layers, torch, M, reps)
    if "norm" in sections:
        result["rmsnorm_quant"] = rmsnorm_quant(fp8q, torch, dev, M, reps, copy_gbs)
    if "recal" in sections:
        result["recalibration"] = recalibration(fp8q, synth, torch, dev, copy_gbs)
    if "moe" in sections:
        result["moe"] = moe(fp8q, synth, torch, dev, reps)
    if "backward" in sections:
        result["backward"] = backward(fp8q, synth, layers, torch, dev, M, reps)
    if "attention" in sections:
        result["attention_decode"] = attention(fp8q, synth, torch, dev, reps)
    if "dispatch" in sections:
        result["moe_dispatch"] = dispatch(fp8q, synth, torch, dev, reps)
    if "smallm" in sections:
        result["small_m"] = small_m(fp8q, layers, torch, dev, reps)
    if "bf16" in sections:
        result["bf16_reference"] = bf16_compare(layers, torch, M, reps, gemm_tflops)
    if "power" in sections:
        result["power"] = power_under_load(fp8q, layers, torch, step_flops)
    if "cpu" in sections:
        result["cpu_baseline"] = cpu_baseline(layers, synth, M, args.cpu_rows)
    result["timing_stats"] = STATS
    print(json.dumps(result), flush=True)


def small_m(fp8q, layers, torch, dev, reps, M=2048):
    """The four layers at 2048 tokens: O and down then have too few 256x256
    tiles to fill the GPU and run on 128-row tiles."""
    out = {}
    for l in layers:
        x = torch.randn((M, l["K"]), device=dev, dtype=torch.float32).to(torch.bfloat16)
        aq, as_ = fp8q.fp8_quant_act_1x128(x)
        y = torch.empty((M, l["N"]), dtype=torch.bfloat16, device=dev)

        def g(aq=aq, as_=as_, l=l, y=y):
            fp8q.fp8_blockscaled_gemm(aq, as_, l["bq"], l["bs"], out=y)
        g()
        t = time_loop(g, reps, torch, label=f"small_m/{l['name']}")
        rows, panels = fp8q.fp8_blockscaled_gemm_tile_plan(M, l["N"])  # the library's own choice
        out[l["name"]] = {"gemm_us": round(t * 1e6, 2), "tflops": round(2.0 * M * l["N"] * l["K"] / t / 1e12, 1),
                          "tile_plan": {"rows_on_256_token_tiles": rows, "panels_on_256_token_tiles": panels,
                                        "panels": -(-l["N"] // 256), "tokens": M}}
        log(f"M={M} {l['name']}: {out[l['name']]}")
    return {"tokens": M, "per_layer": out}


def pow2_gemm(fp8q, layers, torch, M, reps):
    """The same four layers with power-of-two scales (the recipe's pow2 option):
    activations and weights quantized in pow2 mode, product by the GEMM whose
    matrix cores apply the scales (E8M0).  Steps: quantize + GEMM per layer."""
    ops = []
    for l in layers:
        bq, bs = fp8q.fp8_quant_weight_128x128(l["w"], "pow2")
        aq, as_ = fp8q.fp8_quant_act_1x128(l["x"], "pow2")
        ops.append((l, aq, as_, bq, bs))
    torch.cuda.synchronize()
    per, g_s, g_f = {}, 0.0, 0.0
    for l, aq, as_, bq, bs in ops:
        fp8q.fp8_blockscaled_gemm_pow2(aq, as_, bq, bs, out=l["y"])
        t = time_loop(lambda: fp8q.fp8_blockscaled_gemm_pow2(aq, as_, bq, bs, out=l["y"]), reps, torch,
                      label=f"pow2_gemm/{l['name']}")
        f = 2.0 * M * l["N"] * l["K"]
        g_s += t
        g_f += f
        per[l["name"]] = {"gemm_us": round(t * 1e6, 2), "gemm_tflops": round(f / t / 1e12, 1)}

    def step():
        for l, aq, as_, bq, bs in ops:
            fp8q.fp8_quant_act_1x128(l["x"], "pow2", out=(aq, as_))
            fp8q.fp8_blockscaled_gemm_pow2(aq, as_, bq, bs, out=l["y"])
    step()
    t_step = time_loop(step, reps, torch, label="pow2_step")
    tf = g_f / g_s / 1e12
    log(f"pow2 gemm {tf:.1f} TFLOP/s; pow2 step {g_f / t_step / 1e12:.1f} TFLOP/s")
    del ops
    return {"gemm_tflops": round(tf, 1), "gemm_frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4),
            "step_tflops": round(g_f / t_step / 1e12, 1), "per_layer": per}


def fused_output_quant(fp8q, layers, torch, M, reps):
    """Each layer's GEMM with its output quantized for the next FP8 layer (E4M3,
    1x128 blocks): the GEMM followed by a separate activation-quantization pass
    over its bf16 output, against the GEMM whose epilogue quantizes (one
    kernel; the bf16 output never goes to memory).  Same bytes either way."""
    per, t_sep, t_fus, flops = {}, 0.0, 0.0, 0.0
    for l in layers:
        aq, as_, bq, bs, y = l["aq"], l["as_"], l["bq"], l["bs"], l["y"]
        yq = torch.empty((M, l["N"]), dtype=torch.uint8, device=y.device)
        ys = torch.empty((M, l["N"] // 128), dtype=torch.float32, device=y.device)

        def separate():
            fp8q.fp8_blockscaled_gemm(aq, as_, bq, bs, out=y)
            fp8q.fp8_quant_act_1x128(y, "amax", out=(yq, ys))

        def fused():
            fp8q.fp8_blockscaled_gemm_quant(aq, as_, bq, bs, "amax", out=(yq, ys))
        separate()
        fused()
        ts = time_loop(separate, reps, torch, label=f"fused_output_quant/{l['name']}/separate")
        tf = time_loop(fused, reps, torch, label=f"fused_output_quant/{l['name']}/fused")
        f = 2.0 * M * l["N"] * l["K"]
        t_sep += ts
        t_fus += tf
        flops += f
        per[l["name"]] = {"separate_us": round(ts * 1e6, 2), "fused_us": round(tf * 1e6, 2),
                          "fused_tflops": round(f / tf / 1e12, 1), "speedup": round(ts / tf, 3)}
        del yq, ys
    log(f"fused output quant: {flops / t_fus / 1e12:.1f} TFLOP/s vs {flops / t_sep / 1e12:.1f} separate")
    return {"fused_tflops": round(flops / t_fus / 1e12, 1), "separate_tflops": round(flops / t_sep / 1e12, 1),
            "speedup": round(t_sep / t_fus, 3), "per_layer": per,
            "swiglu": fused_swiglu(fp8q, layers, torch, M, reps)}


def fused_swiglu(fp8q, layers, torch, M, reps):
    """The gate+up layer (weight rows in alternating 128-row gate/up blocks)
    with SwiGLU and the down projection's activation quantization in its
    epilogue, against the unfused sequence: bf16 GEMM, silu(gate) * up as
    torch elementwise ops on the bf16 halves, then the 1x128 quantizer.  The
    plain bf16 GEMM alone is timed too: the epilogue's cost over it."""
    l = next(l for l in layers if l["name"] == "gate_up")
    aq, as_, bq, bs, y = l["aq"], l["as_"], l["bq"], l["bs"], l["y"]
    F = l["N"] // 2
    hq = torch.empty((M, F), dtype=torch.uint8, device=y.device)
    hs = torch.empty((M, F // 128), dtype=torch.float32, device=y.device)
    yv = y.view(M, F // 128, 2, 128)
    h = torch.empty((M, F), dtype=torch.bfloat16, device=y.device)
    hv = h.view(M, F // 128, 128)

    def gemm():
        fp8q.fp8_blockscaled_gemm(aq, as_, bq, bs, out=y)

    def separate():
        gemm()
        torch.mul(torch.nn.functional.silu(yv[:, :, 0]), yv[:, :, 1], out=hv)
        fp8q.fp8_quant_act_1x128(h, "amax", out=(hq, hs))

    def fused():
        fp8q.fp8_blockscaled_gemm_swiglu_quant(aq, as_, bq, bs, "amax", out=(hq, hs))
    separate()
    fused()
    tg = time_loop(gemm, reps, torch, label="swiglu/gemm_alone")
    ts = time_loop(separate, reps, torch, label="swiglu/separate")
    tf = time_loop(fused, reps, torch, label="swiglu/fused")
    f = 2.0 * M * l["N"] * l["K"]
    log(f"fused swiglu: {tf * 1e6:.1f} us ({f / tf / 1e12:.1f} TFLOP/s) vs {ts * 1e6:.1f} us separate, "
        f"{tg * 1e6:.1f} us bf16 GEMM alone")
    del hq, hs, h
    return {"layer": "gate_up", "M": M, "F": F, "K": l["K"], "fused_us": round(tf * 1e6, 2),
            "separate_us": round(ts * 1e6, 2), "gemm_alone_us": round(tg * 1e6, 2),
            "fused_tflops": round(f / tf / 1e12, 1), "speedup": round(ts / tf, 3),
            "epilogue_overhead": round(tf / tg - 1.0, 4)}


def rmsnorm_quant(fp8q, torch, dev, M, reps, copy_gbs):
    """RMS normalization fused with the 1x128 quantization of its output, on
    the Llama-3.1-8B hidden state (4096 tokens x 4096), rotating through
    >= 1.2 GB of distinct inputs: against torch's bf16 rms_norm followed by
    fp8_quant_act_1x128, and against fp8_quant_act_1x128 alone (the same
    bytes moved without the norm).  Algorithmic bytes: 2 per input value, 1
    per code, 4 per scale (gamma, 8 KB, not counted)."""
    K = 4096
    nrot = max(1, math.ceil(1.2e9 / (M * K * 3)))
    xs = [torch.randn((M, K), device=dev, dtype=torch.float32).to(torch.bfloat16) for _ in range(nrot)]
    g = (1.0 + 0.1 * torch.randn(K, device=dev)).to(torch.bfloat16)
    q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    s = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    ctr = [0]

    def fused():
        fp8q.fp8_rmsnorm_quant_1x128(xs[ctr[0] % nrot], g, 1e-5, "amax", out=(q, s))
        ctr[0] += 1

    def separate():
        h = torch.nn.functional.rms_norm(xs[ctr[0] % nrot], (K,), weight=g, eps=1e-5)
        fp8q.fp8_quant_act_1x128(h, "amax", out=(q, s))
        ctr[0] += 1

    def quant_only():
        fp8q.fp8_quant_act_1x128(xs[ctr[0] % nrot], "amax", out=(q, s))
        ctr[0] += 1
    fused()
    separate()
    tf = time_loop(fused, reps * nrot, torch, label="rmsnorm_quant/fused")
    ts = time_loop(separate, reps * nrot, torch, label="rmsnorm_quant/separate")
    tq = time_loop(quant_only, reps * nrot, torch, label="rmsnorm_quant/quant_alone")
    b = act_quant_bytes(M, K)
    log(f"rmsnorm+quant {b / tf / 1e9:.1f} GB/s ({tf * 1e6:.1f} us) vs {ts * 1e6:.1f} us separate, "
        f"{tq * 1e6:.1f} us quantizer alone")
    del xs
    return {"M": M, "K": K, "fused_us": round(tf * 1e6, 2), "fused_gbs": round(b / tf / 1e9, 1),
            "fused_frac_hbm": round(b / tf / 1e9 / HBM_PEAK_GBS, 4),
            "fused_frac_copy": round(b / tf / 1e9 / copy_gbs, 4) if copy_gbs else None,
            "separate_us": round(ts * 1e6, 2), "speedup": round(ts / tf, 3),
            "quant_alone_us": round(tq * 1e6, 2)}


def recalibration(fp8q, synth, torch, dev, copy_gbs=None):
    """Requantize all 128 linear weights of the 32-layer Llama-3.1-8B shape."""
    log("recalibration pass: generating 32 x 4 weights")
    ws, outs, total = [], [], 0
    for layer in range(synth.LLAMA_NUM_LAYERS):
        for kind in range(4):
            w = synth.llama_weight(layer, kind, device=dev)
            N, K = w.shape
            ws.append(w)
            outs.append((torch.empty((N, K), dtype=torch.uint8, device=dev),
                         torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)))
            total += weight_quant_bytes(N, K)
    torch.cuda.synchronize()
    res = {"matrices": len(ws), "params": int(sum(w.numel() for w in ws)), "bytes_per_pass": total}
    # one launch for all 128 matrices (the job table is built once per weight set)
    batch = fp8q.WeightBatch(ws, outs)
    for mode in ("amax", "pow2"):
        def one_pass(mode=mode):
            for w, o in zip(ws, outs):
                fp8q.fp8_quant_weight_128x128(w, mode, out=o)

        def batched(mode=mode):
            fp8q.fp8_quant_weight_128x128_batched(batch, mode)
        for name, fn in (("per_matrix", one_pass), ("batched", batched)):
            fn()
            t = time_loop(fn, 3, torch, label=f"recalibration/{mode}/{name}")
            gbs = total / t / 1e9
            r = {"ms_per_pass": round(t * 1e3, 3), "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
            if copy_gbs:
                r["frac_copy"] = round(gbs / copy_gbs, 4)
            res.setdefault(mode, {})[name] = r
            log(f"recalibration {mode} {name}: {t * 1e3:.3f} ms/pass, {gbs:.1f} GB/s")
    del ws, outs, batch
    torch.cuda.empty_cache()
    return res


def moe_dispatch_order(fp8q, synth, torch, dev, shape):
    """The routing table of a synthetic MoE workload on the device and its
    dispatch order from the library (offsets, row index)."""
    ids = torch.from_numpy(synth.moe_routing(shape)).to(dev)
    off, rows, _ = fp8q.fp8_moe_permute(ids, shape.routed_experts, shape.shared_experts)
    return ids, off, rows


def moe(fp8q, synth, torch, dev, reps):
    """Grouped GEMM on the Qwen3-30B-A3B and Moonlight-16B expert shapes, rows
    in the library's dispatch order; beside it a dense bf16 torch.matmul with
    the same M_total x N x K (one weight for all rows) as a labelled proxy for
    a bf16 grouped GEMM (the FP8/BF16 ratio of the pages' linear layers)."""
    out = {}
    for shape in (synth.QWEN3, synth.MOONLIGHT):
        _, offd, rows = moe_dispatch_order(fp8q, synth, torch, dev, shape)
        for layer in ("gate_up", "down"):
            w = synth.moe_weights(shape, layer, device=dev)
            if layer == "gate_up":
                xt = synth.moe_token_matrix(shape, device=dev)
                x = torch.index_select(xt, 0, rows.long())
                del xt
            else:
                x = synth.moe_down_input(shape, device=dev)
            G, N, K = w.shape
            Mt = x.shape[0]
            bq = torch.empty((G, N, K), dtype=torch.uint8, device=dev)
            bs = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device=dev)
            for g in range(G):
                fp8q.fp8_quant_weight_128x128(w[g], out=(bq[g], bs[g]))
            aq, as_ = fp8q.fp8_quant_act_1x128(x)
            y = torch.empty((Mt, N), dtype=torch.bfloat16, device=dev)
            label = f"moe/{shape.name}/{layer}"
            t = time_loop(lambda: fp8q.fp8_grouped_gemm(aq, as_, bq, bs, offd, out=y), reps, torch, label=label)
            flops = 2.0 * Mt * N * K
            tf = flops / t / 1e12
            hbm_bytes = Mt * K + G * N * K + 2 * Mt * N + Mt * (K // 128) * 4 + G * (N // 128) * (K // 128) * 4
            roof = min(FP8_PEAK_TFLOPS, flops / (hbm_bytes / (HBM_PEAK_GBS * 1e9)) / 1e12)
            w0 = w[0]
            for _ in range(3):
                torch.matmul(x, w0.t(), out=y)
            tb = time_loop(lambda: torch.matmul(x, w0.t(), out=y), reps, torch, label=label + "/bf16_dense_proxy")
            out[f"{shape.name}/{layer}"] = {
                "rows": Mt, "groups": G, "N": N, "K": K, "us": round(t * 1e6, 2),
                "tflops": round(tf, 1), "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4),
                "roof_tflops": round(roof, 1), "frac_roof": round(tf / roof, 4),
                "bf16_dense_proxy_tflops": round(flops / tb / 1e12, 1),
                "fp8_over_bf16_dense_proxy": round(tb / t, 3)}
            log(f"moe {shape.name} {layer}: {tf:.1f} TFLOP/s ({t * 1e6:.1f} us), roof {roof:.0f}; "
                f"bf16 dense proxy {flops / tb / 1e12:.1f}")
            if layer == "gate_up":
                out[f"{shape.name}/gate_up_swiglu_quant"] = moe_swiglu(fp8q, torch, aq, as_, bq, bs, offd, y,
                                                                       reps, shape.name, t)
            del x, w, w0, bq, bs, aq, as_, y
            torch.cuda.empty_cache()
    out["bf16_dense_proxy"] = ("torch.matmul in bf16 of all M_total rows against one expert's weight: the same "
                               "flops as the grouped GEMM in one dense call, standing in for a bf16 grouped GEMM")
    return out


def moe_swiglu(fp8q, torch, aq, as_, bq, bs, offd, y, reps, name, t_gemm):
    """The experts' gate+up GEMM with SwiGLU and the down projection's 1x128
    quantization in its epilogue (weight rows read as alternating 128-row
    gate/up blocks per expert), against the unfused sequence: the bf16 grouped
    GEMM, silu(gate) * up as torch elementwise ops on the bf16 halves, then
    the 1x128 quantizer.  t_gemm: the bf16 grouped GEMM alone (timed above)."""
    Mt, N = y.shape
    F = N // 2
    hq = torch.empty((Mt, F), dtype=torch.uint8, device=y.device)
    hs = torch.empty((Mt, F // 128), dtype=torch.float32, device=y.device)
    h = torch.empty((Mt, F), dtype=torch.bfloat16, device=y.device)
    yv, hv = y.view(Mt, F // 128, 2, 128), h.view(Mt, F // 128, 128)

    def separate():
        fp8q.fp8_grouped_gemm(aq, as_, bq, bs, offd, out=y)
        torch.mul(torch.nn.functional.silu(yv[:, :, 0]), yv[:, :, 1], out=hv)
        fp8q.fp8_quant_act_1x128(h, "amax", out=(hq, hs))

    def fused():
        fp8q.fp8_grouped_gemm_swiglu_quant(aq, as_, bq, bs, offd, out=(hq, hs))
    separate()
    fused()
    ts = time_loop(separate, reps, torch, label=f"moe/{name}/swiglu/separate")
    tf = time_loop(fused, reps, torch, label=f"moe/{name}/swiglu/fused")
    f = 2.0 * Mt * N * bq.shape[2]
    log(f"moe {name} gate_up + swiglu + quant fused: {tf * 1e6:.1f} us ({f / tf / 1e12:.1f} TFLOP/s) vs "
        f"{ts * 1e6:.1f} us separate, {t_gemm * 1e6:.1f} us bf16 grouped GEMM alone")
    del hq, hs, h
    return {"F": F, "fused_us": round(tf * 1e6, 2), "fused_tflops": round(f / tf / 1e12, 1),
            "separate_us": round(ts * 1e6, 2), "gemm_alone_us": round(t_gemm * 1e6, 2),
            "speedup": round(ts / tf, 3), "over_gemm_alone": round(t_gemm / tf, 3)}


def backward(fp8q, synth, layers, torch, dev, M, reps):
    import numpy as np
    """Backward pass of the four Llama-shaped layers at 4096 tokens (training
    end to end in FP8): per layer, dY [M, N] ~ N(0, 1e-3) quantized in both
    layouts in one pass, X in 128-token column blocks (its row blocks are the
    forward pass's), W's tiles in both layouts, then the data gradient
    dX = dY W (dense GEMM on W's transposed tiles) and the weight gradient
    dW = dY^T X (1x128 blocks on both operands)."""
    out, tot = {}, {"dgrad_s": 0.0, "wgrad_s": 0.0, "quant_s": 0.0, "flops": 0.0}
    for i, l in enumerate(layers):
        N, K = l["N"], l["K"]
        Mp = (M + 127) // 128 * 128
        g = synth.normal_bf16((M, N), 1e-3, synth.seed_of(16, i, 2), device=dev)
        gq = torch.empty((M, N), dtype=torch.uint8, device=dev)
        gs = torch.empty((M, N // 128), dtype=torch.float32, device=dev)
        gtq = torch.empty((N, Mp), dtype=torch.uint8, device=dev)
        gts = torch.empty((N, Mp // 128), dtype=torch.float32, device=dev)
        xtq = torch.empty((K, Mp), dtype=torch.uint8, device=dev)
        xts = torch.empty((K, Mp // 128), dtype=torch.float32, device=dev)
        wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
        ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
        wtq = torch.empty((K, N), dtype=torch.uint8, device=dev)
        wts = torch.empty((K // 128, N // 128), dtype=torch.float32, device=dev)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        qg = lambda: fp8q.fp8_quant_act_dual(g, out=(gq, gs, gtq, gts))
        qx = lambda: fp8q.fp8_quant_act_dual(l["x"], out=(None, None, xtq, xts))
        qw = lambda: fp8q.fp8_quant_weight_128x128_dual(l["w"], out=(wq, ws, wtq, wts))
        dg = lambda: fp8q.fp8_blockscaled_gemm(gq, gs, wtq, wts, out=dx)
        wg = lambda: fp8q.fp8_blockscaled_gemm_wgrad(gtq, gts, xtq, xts, out=dw)
        for f in (qg, qx, qw, dg, wg):
            f()
        # power-of-two scales: the same operands quantized in pow2 mode, the
        # weight gradient with both per-row scales on the matrix cores
        gtq2, gts2, xtq2, xts2 = (torch.empty_like(t) for t in (gtq, gts, xtq, xts))
        fp8q.fp8_quant_act_dual(g, mode="pow2", rowwise=False, out=(None, None, gtq2, gts2))
        fp8q.fp8_quant_act_dual(l["x"], mode="pow2", rowwise=False, out=(None, None, xtq2, xts2))
        wg2 = lambda: fp8q.fp8_blockscaled_gemm_wgrad_pow2(gtq2, gts2, xtq2, xts2, out=dw)
        wg2()
        t_wg2 = time_loop(wg2, reps, torch, label=f"backward/{l['name']}/wgrad_pow2")
        del gtq2, gts2, xtq2, xts2
        t_qg, t_qx, t_qw = (time_loop(f, reps, torch, label=f"backward/{l['name']}/{n}")
                            for f, n in ((qg, "quant_dy_dual"), (qx, "quant_x_colwise"), (qw, "quant_w_dual")))
        t_dg = time_loop(dg, reps, torch, label=f"backward/{l['name']}/dgrad")
        t_wg = time_loop(wg, reps, torch, label=f"backward/{l['name']}/wgrad")
        f_dg, f_wg = 2.0 * M * N * K, 2.0 * N * K * Mp
        b_qg = M * N * 4 + 2 * M * (N // 128) * 4         # bf16 in, two code layouts, two scale sets
        b_qx = M * K * 3 + K * (Mp // 128) * 4
        b_qw = N * K * 4 + 2 * (N // 128) * (K // 128) * 4
        out[l["name"]] = {
            "dgrad_tflops": round(f_dg / t_dg / 1e12, 1), "wgrad_tflops": round(f_wg / t_wg / 1e12, 1),
            "dgrad_us": round(t_dg * 1e6, 2), "wgrad_us": round(t_wg * 1e6, 2),
            "wgrad_pow2_tflops": round(f_wg / t_wg2 / 1e12, 1),
            "quant_dy_dual_gbs": round(b_qg / t_qg / 1e9, 1), "quant_x_colwise_gbs": round(b_qx / t_qx / 1e9, 1),
            "quant_w_dual_gbs": round(b_qw / t_qw / 1e9, 1),
            "quant_dy_us": round(t_qg * 1e6, 2), "quant_x_us": round(t_qx * 1e6, 2),
            "quant_w_us": round(t_qw * 1e6, 2)}
        log(f"backward {l['name']}: dgrad {f_dg / t_dg / 1e12:.1f} TFLOP/s, wgrad {f_wg / t_wg / 1e12:.1f} "
            f"TFLOP/s (pow2 {f_wg / t_wg2 / 1e12:.1f}), dY dual {b_qg / t_qg / 1e9:.0f} GB/s, X colwise {b_qx / t_qx / 1e9:.0f} GB/s, "
            f"W dual {b_qw / t_qw / 1e9:.0f} GB/s")
        tot["dgrad_s"] += t_dg
        tot["wgrad_s"] += t_wg
        tot["quant_s"] += t_qg + t_qx
        tot["flops"] += f_dg + f_wg
        del g, gq, gs, gtq, gts, xtq, xts, wq, ws, wtq, wts, dx, dw
        torch.cuda.empty_cache()
    # The two-layout activation quantizer on >= 1.2 GB of rotating inputs per
    # shape (the 256 MB last-level cache cannot hold them), as the 1x128
    # quantizer is timed: its HBM rate, comparable with the copy kernel's.
    q_s, q_b = 0.0, 0.0
    Mp = (M + 127) // 128 * 128
    for l in layers:
        K = l["K"]
        nrot = max(1, int(np.ceil(1.2e9 / (M * K * 4))))
        xs = [l["x"]] + [torch.randn((M, K), device=dev, dtype=torch.float32).to(torch.bfloat16)
                         for _ in range(nrot - 1)]
        bufs = (torch.empty((M, K), dtype=torch.uint8, device=dev),
                torch.empty((M, K // 128), dtype=torch.float32, device=dev),
                torch.empty((K, Mp), dtype=torch.uint8, device=dev),
                torch.empty((K, Mp // 128), dtype=torch.float32, device=dev))
        ctr = [0]

        def qd(xs=xs, bufs=bufs, ctr=ctr):
            fp8q.fp8_quant_act_dual(xs[ctr[0] % len(xs)], out=bufs)
            ctr[0] += 1
        qd()
        t = time_loop(qd, reps * len(xs), torch, label=f"backward/{l['name']}/act_dual_rotating")
        b = M * K * 4 + M * (K // 128) * 4 + K * (Mp // 128) * 4
        q_s += t
        q_b += b
        out[l["name"]]["quant_x_dual_rotating_gbs"] = round(b / t / 1e9, 1)
        del xs, bufs
        torch.cuda.empty_cache()
    out["act_dual_rotating"] = {"gbs": round(q_b / q_s / 1e9, 1), "frac_hbm": round(q_b / q_s / 1e9 / HBM_PEAK_GBS, 4),
                                "bytes_per_element": "2 read + 1 + 1 written, + 2 scale sets"}
    log(f"act dual quant (rotating inputs) {q_b / q_s / 1e9:.1f} GB/s")

    step_s = tot["dgrad_s"] + tot["wgrad_s"] + tot["quant_s"]
    out["total"] = {
        "backward_step_ms": round(step_s * 1e3, 3),
        "backward_step_tflops": round(tot["flops"] / step_s / 1e12, 1),
        "dgrad_wgrad_tflops": round(tot["flops"] / (tot["dgrad_s"] + tot["wgrad_s"]) / 1e12, 1),
        "note": "step = quantize dY (both layouts) + X (column blocks) + dgrad + wgrad per layer; "
                "W's transposed tiles are made once per weight update (quant_w_dual)"}
    log(f"backward step {step_s * 1e3:.3f} ms, {tot['flops'] / step_s / 1e12:.1f} TFLOP/s")
    return out


def attention(fp8q, synth, torch, dev, reps):
    """FP8 decode attention over an FP8 KV cache, Llama-3.1-8B shape: 64
    sequences, 32 query and 8 key/value heads of 128, an 8192-token cache,
    lengths drawn uniformly in [2048, 6144] (mean about 4096); random E4M3
    cache rows with scales in [1e-3, 1.1e-2].  HBM-bound: the figure is the
    bytes the kernel must read (the live cache rows and their scales, the
    queries) and write (the output) per launch over its duration."""
    import numpy as np
    B, Hq, Hkv, S, D = 64, 32, 8, 8192, 128
    g = torch.Generator(device=dev).manual_seed(synth.seed_of(18, 0, 0))
    kq = (torch.randn((B, Hkv, S, D), device=dev, generator=g) * 32).clamp(-448, 448).to(torch.float8_e4m3fn)
    vq = (torch.randn((B, Hkv, S, D), device=dev, generator=g) * 32).clamp(-448, 448).to(torch.float8_e4m3fn)
    ks = torch.rand((B, Hkv, S), device=dev, generator=g) * 0.01 + 0.001
    vs = torch.rand((B, Hkv, S), device=dev, generator=g) * 0.01 + 0.001
    cache = (kq.view(torch.uint8), ks, vq.view(torch.uint8), vs)
    lens = np.random.default_rng(np.random.SeedSequence([18, 0, 1])).integers(2048, 6145, B).astype(np.int32)
    dlen = torch.from_numpy(lens).to(dev)
    q = torch.randn((B * Hq, D), device=dev, generator=g).to(torch.bfloat16)
    q_q, q_s = fp8q.fp8_quant_act_1x128(q)
    q_q, q_s = q_q.view(B, Hq, D), q_s.view(B, Hq)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    run = lambda: fp8q.fp8_attention_decode(q_q, q_s, cache, dlen, out=out)
    run()
    t = time_loop(run, reps * 5, torch, label="attention_decode/b64")
    # the same without a workspace: one workgroup per (sequence, head), unsplit
    run1 = lambda: fp8q.fp8_attention_decode(q_q, q_s, cache, dlen, out=out, workspace=None)
    run1()
    t1 = time_loop(run1, reps * 5, torch, label="attention_decode/b64_unsplit")
    kv = int(lens.sum()) * Hkv * 2 * (D + 4)
    nbytes = kv + B * Hq * (D + 4) + B * Hq * D * 2
    # a small batch (the last sequences of a rollout): 8 sequences give 64
    # (sequence, head) pairs, too few to fill the GPU; split vs unsplit
    b8 = 8
    cache8 = tuple(c[:b8] for c in cache)
    q8, s8, d8 = q_q[:b8], q_s[:b8], dlen[:b8]
    out8 = torch.empty((b8, Hq, D), dtype=torch.bfloat16, device=dev)
    r8 = lambda: fp8q.fp8_attention_decode(q8, s8, cache8, d8, out=out8)
    r8u = lambda: fp8q.fp8_attention_decode(q8, s8, cache8, d8, out=out8, workspace=None)
    r8()
    r8u()
    t8 = time_loop(r8, reps * 5, torch, label="attention_decode/b8_split")
    t8u = time_loop(r8u, reps * 5, torch, label="attention_decode/b8_unsplit")
    nb8 = int(lens[:b8].sum()) * Hkv * 2 * (D + 4) + b8 * Hq * (D + 4) + b8 * Hq * D * 2
    # the cache append of one decode step (one key and value row per sequence and head)
    kn = torch.randn((B, Hkv, D), device=dev, generator=g).to(torch.bfloat16)
    vn = torch.randn((B, Hkv, D), device=dev, generator=g).to(torch.bfloat16)
    pos = torch.from_numpy(np.minimum(lens, S - 1)).to(dev)
    app = lambda: fp8q.fp8_kv_cache_append(kn, vn, pos, cache)
    app()
    t_app = time_loop(app, reps * 5, torch, label="attention_decode/append")
    res = {"batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "cache_tokens": S,
           "mean_len": float(lens.mean()), "us": round(t * 1e6, 2), "gbs": round(nbytes / t / 1e9, 1),
           "frac_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4), "bytes": nbytes,
           "kv_bytes_fp8": kv, "kv_bytes_bf16_equivalent": int(lens.sum()) * Hkv * 2 * D * 2,
           "append_us": round(t_app * 1e6, 2),
           "unsplit_us": round(t1 * 1e6, 2), "unsplit_gbs": round(nbytes / t1 / 1e9, 1),
           "batch8": {"split_us": round(t8 * 1e6, 2), "split_gbs": round(nb8 / t8 / 1e9, 1),
                      "unsplit_us": round(t8u * 1e6, 2), "unsplit_gbs": round(nb8 / t8u / 1e9, 1)}}
    log(f"attention decode {t * 1e6:.1f} us, {nbytes / t / 1e9:.0f} GB/s (unsplit {t1 * 1e6:.1f} us); "
        f"8 sequences: split {t8 * 1e6:.1f} us ({nb8 / t8 / 1e9:.0f} GB/s), unsplit {t8u * 1e6:.1f} us; "
        f"cache append {t_app * 1e6:.1f} us")
    res["prefill"] = prefill(fp8q, torch, dev, g, cache, reps)
    del kq, vq, ks, vs, cache
    torch.cuda.empty_cache()
    return res


def prefill(fp8q, torch, dev, g, cache, reps):
    """FP8 attention for many query tokens, Llama-3.1-8B attention shape: one
    4096-token sequence prefilled from position 0 (causal: token t sees cache
    rows 0..t) over the first sequence of the decode cache, 32 query and 8
    key/value heads.  Matrix-core bound: flops 2*128 for q.k plus 2*128 for
    p.v per (query, visible key) pair and query head, T(T+1)/2 pairs per
    head.  Beside it the multi-token append of the 4096 tokens' K and V."""
    import numpy as np
    T, Hq, Hkv, D = 4096, 32, 8, 128
    c1 = tuple(c[:1] for c in cache)
    q = torch.randn((T * Hq, D), device=dev, generator=g).to(torch.bfloat16)
    q_q, q_s = fp8q.fp8_quant_act_1x128(q)
    q_q, q_s = q_q.view(1, T, Hq, D), q_s.view(1, T, Hq)
    start = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty((1, T, Hq, D), dtype=torch.bfloat16, device=dev)
    run = lambda: fp8q.fp8_attention_prefill(q_q, q_s, c1, start, out=out)
    run()
    t = time_loop(run, reps, torch, label="attention_prefill/llama4096")
    flops = 4.0 * D * Hq * T * (T + 1) / 2
    kn = torch.randn((1, T, Hkv, D), device=dev, generator=g).to(torch.bfloat16)
    vn = torch.randn((1, T, Hkv, D), device=dev, generator=g).to(torch.bfloat16)
    app = lambda: fp8q.fp8_kv_cache_append_tokens(kn, vn, start, c1)
    app()
    t_app = time_loop(app, reps, torch, label="attention_prefill/append_tokens")
    app_bytes = 2 * T * Hkv * (2 * D + D + 4)
    log(f"attention prefill 4096 tokens: {t * 1e6:.1f} us, {flops / t / 1e12:.1f} TFLOP/s; "
        f"append of 4096 tokens {t_app * 1e6:.1f} us ({app_bytes / t_app / 1e9:.0f} GB/s)")
    return {"tokens": T, "q_heads": Hq, "kv_heads": Hkv, "causal": True, "us": round(t * 1e6, 2),
            "tflops": round(flops / t / 1e12, 1), "frac_fp8_peak": round(flops / t / 1e12 / FP8_PEAK_TFLOPS, 4),
            "flops": flops, "append_tokens_us": round(t_app * 1e6, 2),
            "append_tokens_gbs": round(app_bytes / t_app / 1e9, 1)}


def dispatch(fp8q, synth, torch, dev, reps):
    """MoE gate_up layer from the routing table to the expert outputs.  Route:
    the library's dispatch order (fp8_moe_permute: group offsets and row ->
    token map on the device).  Quantize before dispatch: quantize the T token
    rows once, then the grouped GEMM gathers each routed row's FP8 bytes by
    index.  Against quantize after dispatch: gather the bf16 rows (torch's
    index copy, standing in for the dispatch of bf16 rows on one GPU),
    quantize all M_total routed rows, grouped GEMM."""
    out = {}
    for shape in (synth.QWEN3, synth.MOONLIGHT):
        ids, offd, idx = moe_dispatch_order(fp8q, synth, torch, dev, shape)
        xt = synth.moe_token_matrix(shape, device=dev)
        w = synth.moe_weights(shape, "gate_up", device=dev)
        G, N, K = w.shape
        T, Mt = xt.shape[0], idx.numel()
        E, ns = shape.routed_experts, shape.shared_experts
        bq = torch.empty((G, N, K), dtype=torch.uint8, device=dev)
        bs = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device=dev)
        for g in range(G):
            fp8q.fp8_quant_weight_128x128(w[g], out=(bq[g], bs[g]))
        del w
        ws = torch.empty(fp8q.fp8_moe_permute_workspace_size(T, shape.top_k, E), dtype=torch.uint8, device=dev)
        entry = torch.empty(T * shape.top_k, dtype=torch.int32, device=dev)
        idx64 = idx.long()
        xr = torch.empty((Mt, K), dtype=torch.bfloat16, device=dev)
        aq_r = torch.empty((Mt, K), dtype=torch.uint8, device=dev)
        as_r = torch.empty((Mt, K // 128), dtype=torch.float32, device=dev)
        aq_t = torch.empty((T, K), dtype=torch.uint8, device=dev)
        as_t = torch.empty((T, K // 128), dtype=torch.float32, device=dev)
        y = torch.empty((Mt, N), dtype=torch.bfloat16, device=dev)

        def route():
            fp8q.fp8_moe_permute(ids, E, ns, out=(offd, idx, entry), workspace=ws)

        def after():
            route()
            torch.index_select(xt, 0, idx64, out=xr)
            fp8q.fp8_quant_act_1x128(xr, out=(aq_r, as_r))
            fp8q.fp8_grouped_gemm(aq_r, as_r, bq, bs, offd, out=y)

        def before():
            route()
            fp8q.fp8_quant_act_1x128(xt, out=(aq_t, as_t))
            fp8q.fp8_grouped_gemm_gather(aq_t, as_t, bq, bs, offd, idx, out=y)

        after()
        before()
        lb = f"dispatch/{shape.name}"
        t_after = time_loop(after, reps, torch, label=lb + "/after")
        t_before = time_loop(before, reps, torch, label=lb + "/before")
        t_route = time_loop(route, reps, torch, label=lb + "/route")
        t_copy = time_loop(lambda: torch.index_select(xt, 0, idx64, out=xr), reps, torch, label=lb + "/bf16_gather")
        t_qr = time_loop(lambda: fp8q.fp8_quant_act_1x128(xr, out=(aq_r, as_r)), reps, torch,
                         label=lb + "/quant_routed_rows")
        t_qt = time_loop(lambda: fp8q.fp8_quant_act_1x128(xt, out=(aq_t, as_t)), reps, torch,
                         label=lb + "/quant_tokens")
        t_gr = time_loop(lambda: fp8q.fp8_grouped_gemm(aq_r, as_r, bq, bs, offd, out=y), reps, torch,
                         label=lb + "/grouped_gemm")
        t_gg = time_loop(lambda: fp8q.fp8_grouped_gemm_gather(aq_t, as_t, bq, bs, offd, idx, out=y), reps, torch,
                         label=lb + "/gather_gemm")
        us = lambda t: round(t * 1e6, 2)
        out[shape.name] = {
            "tokens": T, "rows": Mt, "groups": G, "N": N, "K": K,
            "after_us": us(t_after), "before_us": us(t_before),
            "before_speedup": round(t_after / t_before, 3),
            "route_us": us(t_route), "bf16_gather_copy_us": us(t_copy), "quant_routed_rows_us": us(t_qr),
            "quant_tokens_us": us(t_qt), "grouped_gemm_us": us(t_gr), "gather_gemm_us": us(t_gg),
            "gather_gemm_over_grouped": round(t_gg / t_gr, 3),
            "dispatched_bytes_bf16": Mt * K * 2, "dispatched_bytes_fp8": Mt * K + Mt * (K // 128) * 4,
            "chain": "route (fp8_moe_permute) + quantize + GEMM, from the routing table to the expert outputs",
        }
        log(f"dispatch {shape.name}: route {t_route * 1e6:.1f} us; after {t_after * 1e6:.1f} us, "
            f"before {t_before * 1e6:.1f} us (gather GEMM {t_gg * 1e6:.1f} vs grouped {t_gr * 1e6:.1f} us)")

        # The experts' whole FFN (gate+up, SwiGLU, down) from the routing table,
        # the expert outputs in dispatch order (the top-k weighted combine back
        # to tokens is outside the FP8 path).  FP8 end to end: tokens quantized
        # once, the gathering gate+up GEMM with SwiGLU and the down
        # projection's quantization in its epilogue, the grouped down GEMM on
        # its codes.  Against: bf16 gather, quantize the routed rows, bf16
        # gate+up, torch SwiGLU, quantize h, grouped down GEMM.
        wd = synth.moe_weights(shape, "down", device=dev)
        Hd, F = wd.shape[1], wd.shape[2]
        dq = torch.empty((G, Hd, F), dtype=torch.uint8, device=dev)
        dsc = torch.empty((G, Hd // 128, F // 128), dtype=torch.float32, device=dev)
        for g in range(G):
            fp8q.fp8_quant_weight_128x128(wd[g], out=(dq[g], dsc[g]))
        del wd
        hq = torch.empty((Mt, F), dtype=torch.uint8, device=dev)
        hs = torch.empty((Mt, F // 128), dtype=torch.float32, device=dev)
        h = torch.empty((Mt, F), dtype=torch.bfloat16, device=dev)
        yd = torch.empty((Mt, Hd), dtype=torch.bfloat16, device=dev)
        yv, hv = y.view(Mt, F // 128, 2, 128), h.view(Mt, F // 128, 128)

        def ffn_fp8():
            route()
            fp8q.fp8_quant_act_1x128(xt, out=(aq_t, as_t))
            fp8q.fp8_grouped_gemm_swiglu_quant(aq_t, as_t, bq, bs, offd, row_index=idx, out=(hq, hs))
            fp8q.fp8_grouped_gemm(hq, hs, dq, dsc, offd, out=yd)

        def ffn_unfused():
            after()
            torch.mul(torch.nn.functional.silu(yv[:, :, 0]), yv[:, :, 1], out=hv)
            fp8q.fp8_quant_act_1x128(h, out=(hq, hs))
            fp8q.fp8_grouped_gemm(hq, hs, dq, dsc, offd, out=yd)

        ffn_fp8()
        ffn_unfused()
        t_ffn = time_loop(ffn_fp8, reps, torch, label=lb + "/ffn_fp8")
        t_ffn_u = time_loop(ffn_unfused, reps, torch, label=lb + "/ffn_unfused")
        flops = 2.0 * Mt * K * N + 2.0 * Mt * F * Hd
        out[shape.name]["expert_ffn"] = {
            "fp8_us": us(t_ffn), "unfused_us": us(t_ffn_u), "speedup": round(t_ffn_u / t_ffn, 3),
            "fp8_tflops": round(flops / t_ffn / 1e12, 1), "F": F, "hidden": Hd,
            "chain": ("route, quantize T tokens, gathering gate+up GEMM with SwiGLU + quantization epilogue, "
                      "grouped down GEMM; against route, bf16 gather, quantize routed rows, bf16 gate+up, "
                      "torch SwiGLU, quantize h, grouped down GEMM")}
        log(f"dispatch {shape.name} expert FFN: FP8 end to end {t_ffn * 1e6:.1f} us "
            f"({flops / t_ffn / 1e12:.1f} TFLOP/s) vs {t_ffn_u * 1e6:.1f} us unfused")
        del xt, bq, bs, xr, aq_r, as_r, aq_t, as_t, y, ws, entry, dq, dsc, hq, hs, h, yd
        torch.cuda.empty_cache()
    return out


def bf16_compare(layers, torch, M, reps, fp8_gemm_tflops):
    """torch.matmul in bf16 (hipBLASLt) on the same shapes, for the FP8/BF16 ratio."""
    tot_s, tot_f, per = 0.0, 0.0, {}
    for l in layers:
        x, w = l["x"], l["w"]
        for _ in range(3):  # library heuristics / first-call setup stay out of the timing
            torch.matmul(x, w.t())
        t = time_loop(lambda: torch.matmul(x, w.t()), reps, torch, label=f"bf16_matmul/{l['name']}")
        f = 2.0 * M * l["N"] * l["K"]
        tot_s += t
        tot_f += f
        per[l["name"]] = round(f / t / 1e12, 1)
    tf = tot_f / tot_s / 1e12
    log(f"bf16 torch.matmul {tf:.1f} TFLOP/s")
    out = {"tflops": round(tf, 1), "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
           "per_layer_tflops": per, "fp8_over_bf16": round(fp8_gemm_tflops / tf, 3)}
    out["vendor_fp8_tensorwise"] = vendor_fp8_tensorwise(layers, torch, M, reps, fp8_gemm_tflops)
    return out


def vendor_fp8_tensorwise(layers, torch, M, reps, fp8_gemm_tflops):
    """torch._scaled_mm (hipBLASLt) in E4M3 with ONE scale per tensor on the
    same shapes: the vendor's FP8 GEMM without block scales (the library has
    no 1x128/128x128 block-scaled mode on this platform), for context."""
    try:
        one = torch.ones((), device="cuda")
        tot_s, tot_f, per = 0.0, 0.0, {}
        for l in layers:
            xq = l["x"].to(torch.float8_e4m3fn)
            wq = l["w"].to(torch.float8_e4m3fn)
            run = lambda: torch._scaled_mm(xq, wq.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
            for _ in range(3):
                run()
            t = time_loop(run, reps, torch, label=f"vendor_fp8_tensorwise/{l['name']}")
            f = 2.0 * M * l["N"] * l["K"]
            tot_s += t
            tot_f += f
            per[l["name"]] = round(f / t / 1e12, 1)
            del xq, wq
    except (RuntimeError, AttributeError) as e:
        return {"error": str(e).splitlines()[0][:200]}
    tf = tot_f / tot_s / 1e12
    log(f"vendor fp8 tensorwise {tf:.1f} TFLOP/s")
    return {"tflops": round(tf, 1), "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4), "per_layer_tflops": per,
            "blockscaled_over_tensorwise": round(fp8_gemm_tflops / tf, 3)}


def _cpu_model():
    try:
        import subprocess
        txt = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in txt.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, ValueError):
        pass
    return None


def power_under_load(fp8q, layers, torch, step_flops, seconds=2.0, period=0.02):
    """GPU socket power while the step runs back to back for about two
    seconds, sampled every 20 ms through amdsmi (read-only queries) on the
    device the step runs on (matched by PCI bus), beside the idle power just
    before.  Reported unavailable, with the reason, when amdsmi cannot read
    it.  The step rate of this loop (50 steps between synchronizations, after
    20 more warm-up steps) is reported with it; it is not the headline
    figure."""
    import threading
    try:
        import amdsmi
    except ImportError as e:
        return {"available": False, "reason": f"amdsmi not importable: {e}"}
    try:
        amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
    except Exception as e:  # noqa: BLE001 - any failure means no reading
        return {"available": False, "reason": f"amdsmi_init: {e}"}
    try:
        handles = amdsmi.amdsmi_get_processor_handles()
        props = torch.cuda.get_device_properties(torch.cuda.current_device())
        want = (getattr(props, "pci_domain_id", None), getattr(props, "pci_bus_id", None))
        handle = None
        for h in handles:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
            dom, bus = int(bdf.split(":")[0], 16), int(bdf.split(":")[1], 16)
            if (dom, bus) == want:
                handle = h
        if handle is None and len(handles) == 1:
            handle = handles[0]
        if handle is None:
            return {"available": False, "reason": f"no amdsmi device matches PCI {want} among {len(handles)}"}

        def read():
            info = amdsmi.amdsmi_get_power_info(handle)
            for key in ("current_socket_power", "average_socket_power", "socket_power"):
                v = info.get(key)
                if isinstance(v, (int, float)) and v > 0:
                    return float(v), key
            return None, None

        first, key = read()
        if first is None:
            return {"available": False, "reason": "amdsmi reports no socket power for this device"}
        idle = []
        t_end = time.perf_counter() + 0.5
        while time.perf_counter() < t_end:
            idle.append(read()[0])
            time.sleep(period)
        samples, stop = [], threading.Event()

        def poll():
            while not stop.is_set():
                samples.append(read()[0])
                time.sleep(period)

        def step():
            for l in layers:
                fp8q.fp8_quant_act_1x128(l["x"], out=(l["aq"], l["as_"]))
                fp8q.fp8_blockscaled_gemm(l["aq"], l["as_"], l["bq"], l["bs"], out=l["y"])
        for _ in range(20):  # reach the loaded clock and power state first
            step()
        torch.cuda.synchronize()
        th = threading.Thread(target=poll, daemon=True)
        Ev = torch.cuda.Event
        start, end = Ev(enable_timing=True), Ev(enable_timing=True)
        n, t0 = 0, time.perf_counter()
        th.start()
        start.record()
        while time.perf_counter() - t0 < seconds:
            for _ in range(50):
                step()
            n += 50
            torch.cuda.synchronize()
        end.record()
        torch.cuda.synchronize()
        stop.set()
        th.join()
        samples = [v for v in samples if v is not None]
        idle = [v for v in idle if v is not None]
        t_step = start.elapsed_time(end) / 1e3 / n
        avg = sum(samples) / len(samples) if samples else None
        tflops = step_flops / t_step / 1e12
        res = {"available": True, "quantity": key, "unit": "W",
               "workload": "the step (act quant + GEMM, 4 Llama layers) back to back, 50 steps per sync",
               "seconds": round(time.perf_counter() - t0, 2), "steps": n, "samples": len(samples),
               "avg_w": round(avg, 1) if avg else None, "max_w": round(max(samples), 1) if samples else None,
               "idle_w": round(sum(idle) / len(idle), 1) if idle else None,
               "loop_tflops": round(tflops, 1), "tflops_per_w": round(tflops / avg, 3) if avg else None}
        log(f"power under load: {res['avg_w']} W average ({res['max_w']} max, {res['idle_w']} idle), "
            f"{tflops:.1f} TFLOP/s in this loop, {res['tflops_per_w']} TFLOP/s per W")
        return res
    except Exception as e:  # noqa: BLE001 - a failed reading must not stop the benchmark
        return {"available": False, "reason": f"{type(e).__name__}: {e}"}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:  # noqa: BLE001
            pass


def cpu_baseline(layers, synth, M, one_thread_rows):
    """The CPU oracle, as it stands, on the step's workload: the full step
    (1x128 quantization of each layer's 4096 activation rows + the fp64
    block-scaled GEMM) on all host threads.  The weights are quantized by the
    oracle itself, outside the timing (as they are once per policy update).
    Also: a labelled single-thread run on the first rows of each layer, and
    the oracle's quantizers in GB/s (one Llama activation, one recalibration
    matrix)."""
    import oracle
    import numpy as np
    log(f"cpu baseline: oracle on the full step ({M} tokens x 4 layers)")
    inputs = []
    for l in layers:
        xs = synth.bf16_bits(l["x"])
        bq, bs = oracle.quant_weight_128x128(synth.bf16_bits(l["w"]))
        inputs.append((xs, bq, bs, l["N"], l["K"]))
    threads = oracle.num_threads()

    def run(rows):
        flops, t0 = 0.0, time.perf_counter()
        for xs, bq, bs, N, K in inputs:
            aq, as_ = oracle.quant_act_1x128(np.ascontiguousarray(xs[:rows]))
            oracle.gemm_f64(aq, as_, bq, bs)
            flops += 2.0 * rows * N * K
        return flops, time.perf_counter() - t0
    flops, dt = run(M)
    v = flops / dt / 1e12
    log(f"cpu baseline {v * 1e3:.2f} GFLOP/s in {dt:.1f} s on {threads} threads")
    oracle.set_num_threads(1)
    try:
        f1, d1 = run(one_thread_rows)
    finally:
        oracle.set_num_threads(0)
    log(f"cpu baseline, 1 thread: {f1 / d1 / 1e9:.2f} GFLOP/s in {d1:.1f} s")
    # quantizers: a 4096 x 4096 activation and the largest recalibration matrix
    xq = inputs[1][0]
    t0 = time.perf_counter()
    oracle.quant_act_1x128(xq)
    ta = time.perf_counter() - t0
    wq = synth.bf16_bits(layers[2]["w"])
    t0 = time.perf_counter()
    oracle.quant_weight_128x128(wq)
    tw = time.perf_counter() - t0
    ga = act_quant_bytes(*xq.shape) / ta / 1e9
    gw = weight_quant_bytes(*wq.shape) / tw / 1e9
    log(f"cpu oracle quantizers: activation {ga:.2f} GB/s, weight {gw:.2f} GB/s")
    return {"value": round(v, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2), "cpu_model": _cpu_model(),
            "sample": f"the full step: all {M} tokens of each of the 4 Llama layers, 1x128 activation "
                      "quantization + fp64 block-scaled GEMM (weights quantized by the oracle, untimed)",
            "one_thread": {"value": round(f1 / d1 / 1e12, 6), "unit": "TFLOP/s", "seconds": round(d1, 2),
                           "sample": f"first {one_thread_rows} tokens of each of the 4 layers"},
            "quantizers": {"act_gbs": round(ga, 3), "act_shape": list(xq.shape),
                           "weight_gbs": round(gw, 3), "weight_shape": list(wq.shape),
                           "bytes": "algorithmic: 2 read + 1 written per element + 4 per scale"}}


if __name__ == "__main__":
    main()
