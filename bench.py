"""Benchmark of the MoE layer step (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload balanced] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic input: router top-k and
metadata, permute, the two forward grouped GEMMs, combine, then combine backward, the four
backward grouped GEMMs, route backward and permute backward.  Inputs are resident in HBM before
the timed region.  The default workload is the balanced-routing layer (8192 tokens, d 2048,
64 experts, top-4, SwiGLU d_ff 1024, bf16, round-robin logits), fwd+bwd.

Prints one JSON line with the throughput (tokens/s), the roofline of the dominant kernel (the
gate/up grouped GEMM, timed with HIP events on the stream it runs on, during the timed steps)
and the oracle's throughput on the host cores over a bounded token sample (a baseline only).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd+bwd tokens/s/GPU; grouped-GEMM TFLOP/s as % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_MXFP8_TFLOPS = 5000.0
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="balanced", choices=["tiny", "balanced", "sweep", "skewed", "mxfp8"])
    ap.add_argument("--experts", type=int, default=None, help="expert count for the sweep workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    return ap.parse_args()


def workload_config(args):
    import synth
    cfg = synth.CONFIGS[args.workload]
    if args.experts is not None:
        cfg = cfg.with_(E=args.experts)
    return cfg


def describe(cfg):
    kind = {"roundrobin": "balanced (round-robin) routing", "normal": "random N(0,1) logits",
            "zipf": "Zipf-skewed routing", "router": "router-projected logits"}[cfg.logits]
    prec = "MXFP8 expert GEMMs" if cfg.mxfp8 else "bf16"
    return (f"MoE layer fwd+bwd, {kind}: T={cfg.T}, d_model={cfg.d}, E={cfg.E}, top-{cfg.k}, "
            f"SwiGLU d_ff={cfg.f}, {prec}, fp32 accumulate, seed {cfg.seed}")


def run_gpu(cfg, steps, warmup):
    import torch

    import synth
    from expert_ffn_layer_top_amd import layer

    dev = torch.device("cuda:0")
    inputs = synth.to_torch(synth.make_inputs(cfg), dev)
    w = layer.Weights(inputs["w_gate"], inputs["w_up"], inputs["w_down"], w_r=inputs.get("w_r"))
    if cfg.mxfp8:
        w.quantize_mx()
    x, dy, logits = inputs["x"], inputs["dy"], inputs.get("logits")

    def step(events=None):
        if cfg.mxfp8:
            w.quantize_mx()                  # weights are re-quantised every step (both directions)
        ctx = layer.forward(x, w, cfg.k, logits=logits, mxfp8=cfg.mxfp8, gate_up_events=events)
        if not cfg.forward_only:
            layer.backward(ctx, w, dy)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gate_up_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    return elapsed, gate_up_ms


def cpu_baseline(cfg, sample_tokens):
    """The oracle as it stands, on the first `sample_tokens` tokens of the same workload (same
    weights, same routing construction), forward + backward, timed on the host cores."""
    import numpy as np
    import threadpoolctl

    import synth
    from oracle import moe

    s = min(sample_tokens, cfg.T)
    inputs = synth.make_inputs(cfg)
    x, dy = inputs["x"][:s], inputs["dy"][:s]
    t0 = time.perf_counter()
    logits = inputs["logits"][:s] if "logits" in inputs else moe.router_project(x, inputs["w_r"])
    fwd = moe.layer_forward(x, logits, cfg.k, inputs["w_gate"], inputs["w_up"], inputs["w_down"])
    if not cfg.forward_only:
        bwd = moe.layer_backward(fwd, dy, inputs["w_gate"], inputs["w_up"], inputs["w_down"])
        if "w_r" in inputs:
            moe.router_project_bwd(x, inputs["w_r"], bwd["d_logits"])
    secs = time.perf_counter() - t0
    blas = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    threads = max((p.get("num_threads", 1) for p in blas), default=1)
    assert np.isfinite(fwd["y"]).all()
    return dict(value=s / secs, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"first {s} of {cfg.T} tokens, full expert weights, fwd+bwd, float64 numpy "
                       f"({secs:.1f} s; BLAS threads {threads}, affinity {len(os.sched_getaffinity(0))} cores)")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (no collectives or sharding); use --gpus 1",
              file=sys.stderr)
        return 2
    cfg = workload_config(args)
    elapsed, gate_up_ms = run_gpu(cfg, args.steps, args.warmup)
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = cfg.T * args.steps / elapsed
    flops = 4.0 * cfg.n * cfg.d * cfg.f                      # gate + up products of every routed row
    achieved = flops / (gate_up_ms * 1e-3) / 1e12
    peak = PEAK_MXFP8_TFLOPS if cfg.mxfp8 else PEAK_BF16_TFLOPS
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if cfg.mxfp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": describe(cfg), "T": cfg.T, "d_model": cfg.d, "experts": cfg.E,
                   "top_k": cfg.k, "d_ff": cfg.f, "fwd_bwd": not cfg.forward_only},
        "roofline": {"bound": "mfma", "kernel": "grouped GEMM gate/up + SwiGLU epilogue",
                     "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": None,
                     "avg_ms": round(gate_up_ms, 4), "flop_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
