"""Benchmark of the MoE layer step (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload balanced] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic input: router top-k and
metadata, permute, the two forward grouped GEMMs, combine, then combine backward, the four
backward grouped GEMMs, route backward and permute backward.  Inputs are resident in HBM before
the timed region.  The default workload is the balanced-routing layer (8192 tokens, d 2048,
64 experts, top-4, SwiGLU d_ff 1024, bf16, round-robin logits), fwd+bwd.

Prints one JSON line with the throughput (tokens/s), the roofline of the dominant kernel and the
oracle's throughput on the host cores over a bounded token sample (a baseline only).

After the W warm-up steps, untimed steps continue until --settle seconds (default 1) after the
first one: a fresh process on a fresh box stalls for milliseconds around its first steps and its
clocks ramp over the next tens of steps.  Then an instrumented pass of K steps brackets every
call of the step with HIP
events on the stream it runs on (each grouped-GEMM call is one kernel): its averages give
`gemm_ms` / `gemm_tflops` and, for the routing and row-movement calls, achieved HBM GB/s on their
algorithmic bytes (`rows_hbm_gbs`, against the 8000 GB/s peak; `aux_hbm_gbs` likewise for the
router products and the MXFP8 quantisers where the workload has them), and they pick the dominant
kernel, the GEMM with the largest average duration (under MXFP8 the forward down call, which
also quantises A, is not a candidate).  Then the timed region runs K more steps with only the
dominant kernel bracketed: `value` and `ms_per_step` come from it, and so does the roofline's
average duration (an event pair around every call costs the step 2-5%).  The dominant GEMM's
`traffic` (HBM bytes per launch) comes from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary kept
in profiles/, and is null when that summary is missing or was taken on other kernel sources.

--copy-probe N runs torch's elementwise negation over an fp32 buffer of N bytes three times
before the warm-up: the plain copy kernel that calibrates the HBM byte counters.
"""

import argparse
import gc
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
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES")
    ap.add_argument("--settle", type=float, default=1.0, metavar="SECONDS",
                    help="after the warm-up, keep stepping (untimed) until this long after the first step")
    ap.add_argument("--flush", action="store_true",
                    help="instrumented pass: write 1 GiB of scratch between steps (cold L2 and last-level cache)")
    ap.add_argument("--recompute", action="store_true",
                    help="per-layer activation recompute: the backward re-runs the gate/up product")
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
    return (f"MoE layer {'forward' if cfg.forward_only else 'fwd+bwd'}, {kind}: T={cfg.T}, d_model={cfg.d}, E={cfg.E}, top-{cfg.k}, "
            f"SwiGLU d_ff={cfg.f}, {prec}, fp32 accumulate, seed {cfg.seed}")


def gemm_flops(cfg):
    """Algorithmic flop of each grouped-GEMM call over the routed rows (n = T k)."""
    ndf = float(cfg.n) * cfg.d * cfg.f
    return {"gate_up": 4 * ndf, "down": 2 * ndf, "dgrad_down": 2 * ndf, "wgrad_down": 2 * ndf,
            "dgrad_gate_up": 4 * ndf, "wgrad_gate_up": 4 * ndf, "recompute": 4 * ndf}


def copy_probe(nbytes):
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def run_gpu(cfg, steps, warmup, probe_bytes=0, recompute=False, flush=False, settle=1.0):
    import torch

    import synth
    from expert_ffn_layer_top_amd import layer

    dev = torch.device("cuda:0")
    if probe_bytes:
        copy_probe(probe_bytes)
    inputs = synth.to_torch(synth.make_inputs(cfg), dev)
    w = layer.Weights(inputs["w_gate"], inputs["w_up"], inputs["w_down"], w_r=inputs.get("w_r"))
    if cfg.mxfp8:
        w.quantize_mx()
    x, dy, logits = inputs["x"], inputs["dy"], inputs.get("logits")
    calls = layer.GEMM_CALLS if not cfg.forward_only else ("gate_up", "down")
    if recompute and not cfg.forward_only:
        calls = calls + (layer.RECOMPUTE_CALL,)
    rows = layer.ROW_CALLS if not cfg.forward_only else ("route", "permute", "combine")
    # router products and MXFP8 quantisers, where the workload has them
    aux = ()
    if cfg.logits == "router":
        aux += layer.ROUTER_CALLS if not cfg.forward_only else ("router",)
    if cfg.mxfp8:
        aux += ("quant_w",) + (layer.QUANT_CALLS if not cfg.forward_only else ("quant_x",))

    def step(events=None):
        if cfg.mxfp8:
            qw = events.get("quant_w") if events else None
            if qw:
                qw[0].record()
            w.quantize_mx()                  # weights are re-quantised every step (both directions)
            if qw:
                qw[1].record()
        ctx = layer.forward(x, w, cfg.k, logits=logits, mxfp8=cfg.mxfp8, events=events, recompute=recompute)
        if not cfg.forward_only:
            layer.backward(ctx, w, dy, events=events)

    def pairs(names):
        return [{c: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for c in names}
                for _ in range(steps)]

    def mean_ms(evs, c):
        return sum(e[c][0].elapsed_time(e[c][1]) for e in evs) / len(evs)

    t_first = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # settle: a fresh process stalls for milliseconds around its first steps and the clocks ramp
    # over the next tens of steps, which per-kernel events do not see but a short wall-clock
    # region does; untimed steps until `settle` seconds after the first one
    settled = 0
    while time.perf_counter() - t_first < settle:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
        settled += 4
    # no collector pauses in the measured passes (a full collection can stall the host for tens of
    # milliseconds while the GPU drains its queue): collect now, re-enable at the end
    gc.collect()
    gc.disable()
    # instrumented pass: every call bracketed
    evs = pairs(calls + rows + aux)
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev) if flush else None
    for i in range(steps):
        if scratch is not None:
            scratch.fill_(float(i))          # 1 GiB written: evicts the step's data from L2 and MALL
        step(evs[i])
    torch.cuda.synchronize()
    gemm_ms = {c: mean_ms(evs, c) for c in calls}
    row_ms = {c: mean_ms(evs, c) for c in rows}
    aux_ms = {c: mean_ms(evs, c) for c in aux}
    cand = [c for c in calls if not (cfg.mxfp8 and c == "down") and c != layer.RECOMPUTE_CALL]
    dom = max(cand, key=lambda c: gemm_ms[c])
    # timed region: the dominant kernel alone bracketed
    evd = pairs((dom,))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evd[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gc.enable()
    return elapsed, gemm_ms, row_ms, aux_ms, dom, mean_ms(evd, dom), settled


def traffic_of(cfg, call):
    """HBM bytes per launch of `call` from its counter summary, if it matches the current sources."""
    from expert_ffn_layer_top_amd import profsum
    dtype = "mxfp8" if cfg.mxfp8 else "bf16"
    tag = cfg.name if cfg.name != "sweep" else f"sweep_E{cfg.E}"
    path = os.path.join(ROOT, "profiles", f"{call}_{dtype}_{tag}_traffic.txt")
    t = profsum.read_traffic(path)
    if (t is None or t.get("source_sha256") != profsum.source_sha256(dtype)
            or t.get("kernel") != profsum.kernel_name(call, dtype, cfg.d, cfg.f)):
        return None
    return float(t["traffic_bytes"])


def row_bytes(cfg, call):
    """Algorithmic HBM bytes of the routing and row-movement calls (each element read or written
    once; bf16 rows, E4M3 rows + E8M0 scales for the MXFP8 permute, fp32 gates and logits)."""
    T, d, E, k = float(cfg.T), cfg.d, cfg.E, cfg.k
    eb = 1 + 1 / 32 if cfg.mxfp8 else 2
    return {"route": T * (4 * E + 12 * k),
            "permute": (1 + k) * T * d * eb + 4 * T * k,
            "combine": (k + 1) * T * d * 2 + 8 * T * k,
            "combine_bwd": (2 * k + 1) * T * d * 2 + 12 * T * k,
            "permute_bwd": (k + 1) * T * d * 2 + 4 * T * k,
            "route_bwd": T * (4 * E + 12 * k)}[call]


def aux_bytes(cfg, call):
    """Algorithmic HBM bytes of the router products and the MXFP8 quantiser calls: each element
    read or written once (quantisers: 2 B read, 1 + 1/32 B written per element and layout; the
    grouped token blocks counted over the n routed rows, padding excluded)."""
    T, d, E, n, f = float(cfg.T), cfg.d, cfg.E, float(cfg.n), cfg.f
    q = 2 + 1 + 1 / 32
    return {"router": T * d * 2 + d * E * 4 + T * E * 4,
            "router_bwd": T * E * 4 * 2 + d * E * 4 * 2 + T * d * 4 + T * d * 2,
            "quant_w": 3 * E * d * f * (2 + 2 * (1 + 1 / 32)),
            "quant_x": T * d * q, "quant_dg": n * f * q, "quant_du": n * f * q, "quant_dyT": n * d * q,
            "quant_aT": n * f * q, "quant_dgT": n * f * q, "quant_duT": n * f * q, "quant_xT": n * d * q}[call]


def gemm_bytes(cfg, call):
    """Algorithmic HBM bytes of one grouped-GEMM call: each operand read once, each output written
    once (bf16 2 B; MXFP8 operands 1 B + 1/32 B of scale)."""
    n, d, f, E = float(cfg.n), cfg.d, cfg.f, cfg.E
    ob = 1 + 1 / 32 if cfg.mxfp8 else 2
    if call == "recompute":
        call = "gate_up"
    return {"gate_up": ob * (n * d + 2 * E * f * d) + 2 * 3 * n * f,
            "down": ob * (n * f + E * d * f) + 2 * n * d,
            "dgrad_down": ob * (n * d + E * d * f) + 2 * 2 * n * f + 2 * 2 * n * f,
            "wgrad_down": ob * (n * d + n * f) + 2 * E * d * f,
            "dgrad_gate_up": ob * (2 * n * f + 2 * E * f * d) + 2 * n * d,
            "wgrad_gate_up": ob * (2 * n * f + n * d) + 2 * 2 * E * f * d}[call]


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
    elapsed, gemm_ms, row_ms, aux_ms, dom, dom_ms, settled = run_gpu(cfg, args.steps, args.warmup, args.copy_probe,
                                                                     args.recompute, args.flush, args.settle)
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = cfg.T * args.steps / elapsed
    flops = gemm_flops(cfg)
    achieved = flops[dom] / (dom_ms * 1e-3) / 1e12
    peak = PEAK_MXFP8_TFLOPS if cfg.mxfp8 else PEAK_BF16_TFLOPS
    from expert_ffn_layer_top_amd import profsum
    dtype = "mxfp8" if cfg.mxfp8 else "bf16"
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settled,          # untimed steps after the warm-up (--settle seconds)
        "instrumented_steps": args.steps,  # untimed pass with every call bracketed
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": describe(cfg), "T": cfg.T, "d_model": cfg.d, "experts": cfg.E,
                   "top_k": cfg.k, "d_ff": cfg.f, "fwd_bwd": not cfg.forward_only,
                   "activation_recompute": bool(args.recompute), "instrumented_pass_flushed": bool(args.flush)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic_of(cfg, dom),
                     "kernel": f"{profsum.kernel_name(dom, dtype, cfg.d, cfg.f)} ({dom})",
                     "avg_ms": round(dom_ms, 4), "flop_per_launch": flops[dom],
                     "algorithmic_bytes": round(gemm_bytes(cfg, dom))},
        "gemm_ms": {c: round(v, 4) for c, v in gemm_ms.items()},
        "gemm_tflops": {c: round(flops[c] / (v * 1e-3) / 1e12, 1) for c, v in gemm_ms.items()},
        "rows_us": {c: round(v * 1e3, 1) for c, v in row_ms.items()},
        "rows_hbm_gbs": {c: round(row_bytes(cfg, c) / (v * 1e-3) / 1e9, 1) for c, v in row_ms.items()},
        "hbm_peak_gbs": HBM_PEAK_GBS,
    }
    if aux_ms:
        out["aux_us"] = {c: round(v * 1e3, 1) for c, v in aux_ms.items()}
        out["aux_hbm_gbs"] = {c: round(aux_bytes(cfg, c) / (v * 1e-3) / 1e9, 1) for c, v in aux_ms.items()}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
