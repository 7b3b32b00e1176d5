"""Benchmark of the MoE layer step (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mxfp8] [--experts E]
                    [--no-flush] [--no-cpu-baseline] [--recompute] [--copy-probe BYTES]

A step is one pass of the whole hot path over one batch of synthetic input.  The default
workload is the largest one, the MXFP8 layer: 32768 tokens, d_model 7168, 64 experts, top-4,
SwiGLU d_ff 2048, every expert product on E4M3 operands with one E8M0 scale per 32 elements
along its contraction dimension.  Its step is: the expert weights quantised in both contraction
directions, the router projection, router top-k and metadata, x quantised and permuted, the two
forward grouped GEMMs (A quantised between them), combine; then the fused combine backward
(dYexp leaves as MXFP8 row blocks), route and router backward, the four backward grouped GEMMs
with their operands quantised (row blocks for the dgrads, grouped token blocks for the wgrads)
and the permute backward.  Inputs are resident in HBM before any timed region.

Protocol (events are created before the first warm-up step):
  1. W warm-up steps.
  2. Instrumented pass, K steps.  Before each, 1 GiB of scratch is read (cold L2 and last-level
     cache, with no dirty lines left whose write-back would land on the step's first calls, as a
     flush by writing leaves; --no-flush skips it).  Every call of the step is bracketed with HIP events
     on the stream it runs on, and so is the whole step.  Gives per-call medians: TFLOP/s of each
     grouped GEMM (`gemm_ms`, `gemm_tflops`), achieved HBM GB/s of the routing and row calls
     (`rows_*`) and of the router products and MXFP8 quantisers (`aux_*`) on their algorithmic
     bytes, and the cold step time (`step_ms_flushed`: median, p10, p90).  It also picks the
     dominant kernel: the grouped GEMM with the largest median.
  3. Timed region, K steps back to back (warm: in training the layer's input was just written by
     the layer before it): an event at every step boundary and a pair around the dominant GEMM.
     `value` = T K / wall-clock seconds, `ms_per_step` = wall-clock / K, `step_ms` = median, p10,
     p90 of the per-step event durations; the roofline's duration is the dominant GEMM's mean.
  4. MXFP8: K more steps without re-quantising the weights (training quantises them once per
     optimizer step): `ms_per_step_excl_weight_quant` (wall-clock / K).

`roofline.traffic` and the counter columns (`*_traffic_bytes`, `*_counter_gbs`) come from the
rocprofv3 FETCH_SIZE / WRITE_SIZE summary of the workload under profiles/ (hbm_traffic_<workload>.txt,
written by `python -m expert_ffn_layer_top_amd.profsum step-traffic` from two runs of this script
with --copy-probe), per call, and are null for a call whose kernel sources changed since.

`cpu_baseline` times the oracle as it stands on the host cores over a bounded sample of the
same workload (see cpu_baseline_*), as a baseline only.
"""

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd+bwd tokens/s/GPU; grouped-GEMM TFLOP/s as % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_MXFP8_TFLOPS = 5000.0
HBM_PEAK_GBS = 8000.0
FLUSH_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mxfp8", choices=["tiny", "balanced", "sweep", "skewed", "mxfp8"])
    ap.add_argument("--experts", type=int, default=None, help="expert count for the sweep workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="first run torch's negation over an fp32 buffer of BYTES three times (the "
                         "plain copy kernel that calibrates the HBM byte counters)")
    ap.add_argument("--no-flush", action="store_true", help="instrumented pass without the 1 GiB flush")
    ap.add_argument("--recompute", action="store_true",
                    help="per-layer activation recompute: the backward re-runs the gate/up product")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured-ceiling probes")
    return ap.parse_args()


def workload_config(args):
    import synth
    cfg = synth.CONFIGS[args.workload]
    if args.experts is not None:
        cfg = cfg.with_(E=args.experts)
    return cfg


def workload_tag(cfg):
    return cfg.name if cfg.name != "sweep" else f"sweep_E{cfg.E}"


def describe(cfg):
    kind = {"roundrobin": "balanced (round-robin) routing", "normal": "random N(0,1) logits",
            "zipf": "Zipf-skewed routing", "router": "router-projected logits"}[cfg.logits]
    prec = ("MXFP8 expert GEMMs (E4M3 + E8M0 per 32 along K), weights re-quantised every step"
            if cfg.mxfp8 else "bf16")
    return (f"MoE layer {'forward' if cfg.forward_only else 'fwd+bwd'}, {kind}: T={cfg.T}, d_model={cfg.d}, "
            f"E={cfg.E}, top-{cfg.k}, SwiGLU d_ff={cfg.f}, {prec}, fp32 accumulate, seed {cfg.seed}")


# ------------------------------------------------------------------ algorithmic work

def gemm_flops(cfg):
    """Algorithmic flop of each grouped-GEMM call over the routed rows (n = T k)."""
    ndf = float(cfg.n) * cfg.d * cfg.f
    return {"gate_up": 4 * ndf, "down": 2 * ndf, "dgrad_down": 2 * ndf, "wgrad_down": 2 * ndf,
            "dgrad_gate_up": 4 * ndf, "wgrad_gate_up": 4 * ndf, "recompute": 4 * ndf}


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


def row_bytes(cfg, call):
    """Algorithmic HBM bytes of the routing and row-movement calls: every element they must read
    or write, once (bf16 rows 2 B; MXFP8 rows 1 B + 1/32 B of scale; fp32 gates and logits; int32
    indices)."""
    T, d, E, k = float(cfg.T), cfg.d, cfg.E, cfg.k
    n = T * k
    mx = 1 + 1 / 32
    router = cfg.logits == "router"
    if call == "route":          # logits in; topk_idx, gates, dest, row_token out
        return T * 4 * E + n * 16
    if call == "permute":        # x rows in, k copies out (MXFP8: quantised on the way), dest in
        return T * d * 2 + n * d * (mx if cfg.mxfp8 else 2) + 4 * n
    if call == "combine":        # yexp rows, gates, dest in; y out
        return (n + T) * d * 2 + 8 * n
    if call == "combine_bwd":    # dy, yexp rows, gates, dest in; dyexp (bf16, or MX row blocks + row gates), d_gate out
        out = n * d * mx + 4 * n if cfg.mxfp8 else n * d * 2
        return T * d * 2 + n * d * 2 + 8 * n + out + 4 * n
    if call == "permute_bwd":    # dxp rows, dest (and d_logits, w_r for the router's dx term) in; dx out
        return (n + T) * d * 2 + 4 * n + ((T + d) * E * 4 if router else 0)
    if call == "route_bwd":      # gates, idx, d_gate in; d_logits out
        return T * 4 * E + 12 * n
    raise KeyError(call)


def aux_bytes(cfg, call):
    """Algorithmic HBM bytes of the router products and the MXFP8 quantiser calls, each element
    read or written once (quantisers: 2 B read, 1 + 1/32 B written per element; the grouped token
    blocks write their padded token axis, and a gather through row_token reads each source row
    once)."""
    T, d, E, n, f = float(cfg.T), cfg.d, cfg.E, float(cfg.n), cfg.f
    mx = 1 + 1 / 32
    P = float(((cfg.n + 128 * cfg.E + 127) // 128) * 128)   # padded token axis of the grouped blocks
    if call == "router":         # x, w_r in; logits out
        return T * d * 2 + d * E * 4 + T * E * 4
    if call == "router_bwd":     # d_logits, x in; dw_r out (the dx term is the permute backward's)
        return T * E * 4 + T * d * 2 + d * E * 4
    if call == "quant_w":        # three weights, both layouts from one read
        return 3 * E * d * f * (2 + 2 * mx)
    if call in ("quant_a", "quant_dg", "quant_du"):   # both layouts from one read
        return n * f * (2 + mx) + P * f * mx
    if call == "quant_dyT":      # dy gathered through row_token with the row gates
        return T * d * 2 + n * 8 + P * d * mx
    if call == "quant_xT":
        return T * d * 2 + n * 4 + P * d * mx
    raise KeyError(call)


# ------------------------------------------------------------------ GPU timing

def copy_probe(nbytes):
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def pct(v, q):
    """Percentile q (0..100) of a list, linear interpolation."""
    s = sorted(v)
    if len(s) == 1:
        return s[0]
    x = (len(s) - 1) * q / 100.0
    i = int(x)
    j = min(i + 1, len(s) - 1)
    return s[i] + (s[j] - s[i]) * (x - i)


def dist(v):
    return {"median": round(statistics.median(v), 4), "p10": round(pct(v, 10), 4), "p90": round(pct(v, 90), 4)}


def run_gpu(cfg, steps, warmup, probe_bytes=0, recompute=False, flush=True):
    import torch

    import synth
    from expert_ffn_layer_top_amd import layer

    dev = torch.device("cuda:0")
    if probe_bytes:
        copy_probe(probe_bytes)
    inputs = synth.to_torch(synth.make_inputs(cfg), dev)
    w = layer.Weights(inputs["w_gate"], inputs["w_up"], inputs["w_down"], w_r=inputs.get("w_r"))
    x, dy, logits = inputs["x"], inputs["dy"], inputs.get("logits")
    calls = layer.GEMM_CALLS if not cfg.forward_only else ("gate_up", "down")
    if recompute and not cfg.forward_only:
        calls = calls + (layer.RECOMPUTE_CALL,)
    rows = layer.ROW_CALLS if not cfg.forward_only else ("route", "permute", "combine")
    aux = ()
    if cfg.logits == "router":
        aux += layer.ROUTER_CALLS if not cfg.forward_only else ("router",)
    if cfg.mxfp8:
        aux += ("quant_w",) + layer.QUANT_CALLS_FWD + (layer.QUANT_CALLS if not cfg.forward_only else ())

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def step(events=None, quant_weights=True):
        if cfg.mxfp8 and quant_weights:
            qw = events.get("quant_w") if events else None
            if qw:
                qw[0].record()
            w.quantize_mx()                  # the weights in both contraction directions
            if qw:
                qw[1].record()
        elif cfg.mxfp8 and not w.mx:
            w.quantize_mx()
        ctx = layer.forward(x, w, cfg.k, logits=logits, mxfp8=cfg.mxfp8, events=events, recompute=recompute)
        if not cfg.forward_only:
            layer.backward(ctx, w, dy, events=events)

    # every event of the run exists before the first step
    names = calls + rows + aux
    inst = [{c: (ev(), ev()) for c in names + ("step",)} for _ in range(steps)]
    bounds = [ev() for _ in range(steps + 1)]
    bounds_nq = [ev() for _ in range(steps + 1)]
    scratch = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev) if flush else None

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # instrumented pass (cold caches unless --no-flush)
    for i in range(steps):
        if scratch is not None:
            scratch.sum()                    # 1 GiB read: evicts the step's data from L2 and MALL
        inst[i]["step"][0].record()
        step(inst[i])
        inst[i]["step"][1].record()
    torch.cuda.synchronize()

    def med(c):
        return statistics.median(e[c][0].elapsed_time(e[c][1]) for e in inst)

    gemm_ms = {c: med(c) for c in calls}
    row_ms = {c: med(c) for c in rows}
    aux_ms = {c: med(c) for c in aux}
    step_flushed = [e["step"][0].elapsed_time(e["step"][1]) for e in inst]
    cand = [c for c in calls if c != layer.RECOMPUTE_CALL]
    dom = max(cand, key=lambda c: gemm_ms[c])
    domev = [{dom: (ev(), ev())} for _ in range(steps)]
    torch.cuda.synchronize()

    # timed region: steps back to back
    t0 = time.perf_counter()
    bounds[0].record()
    for i in range(steps):
        step(domev[i])
        bounds[i + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = [bounds[i].elapsed_time(bounds[i + 1]) for i in range(steps)]
    dom_ms = statistics.mean(e[dom][0].elapsed_time(e[dom][1]) for e in domev)

    res = dict(elapsed=elapsed, gemm_ms=gemm_ms, row_ms=row_ms, aux_ms=aux_ms, dom=dom, dom_ms=dom_ms,
               step_ms=step_ms, step_flushed=step_flushed)
    if cfg.mxfp8:
        # the same steps with the weights quantised once, outside the region
        t0 = time.perf_counter()
        bounds_nq[0].record()
        for i in range(steps):
            step(quant_weights=False)
            bounds_nq[i + 1].record()
        torch.cuda.synchronize()
        res["elapsed_nq"] = time.perf_counter() - t0
        res["step_ms_nq"] = [bounds_nq[i].elapsed_time(bounds_nq[i + 1]) for i in range(steps)]
    return res


# ------------------------------------------------------------------ measured ceilings

def measured_ceilings():
    """What this GPU sustains on its two bounding resources, from the self-written probes in
    libmoe_probe.so (expert_ffn_layer_top_amd/probe/ceiling.hip), timed with HIP events on the
    current stream: MFMA-only loops (bf16 16x16x32 and block-scaled fp8 16x16x128, one and four
    waves per SIMD), a 1 GiB streaming copy and read, and the grouped GEMMs' LDS-DMA operand stream
    without the MFMAs (L2-resident panels; panels from HBM in the products' tile cells), with the
    GEMM rate that stream alone allows.  Each is run twice; the second run counts."""
    import ctypes

    import torch
    from expert_ffn_layer_top_amd import build as _b
    if not os.path.exists(_b.PROBE_LIB):
        raise RuntimeError(f"{_b.PROBE_LIB} is missing: build it with `python -m expert_ffn_layer_top_amd.build`")
    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.probe_mfma_flop.restype = ctypes.c_double
    lib.probe_mfma_flop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p]
    lib.probe_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def timed(fn):
        ms = None
        for _ in range(2):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            st = fn()
            b.record()
            torch.cuda.synchronize()
            if st != 0:
                raise RuntimeError(f"probe launch failed ({st})")
            ms = a.elapsed_time(b)
        return ms

    out = {}
    for name, fp8, iters in (("mfma_bf16", 0, 20000), ("mfma_fp8", 1, 10000)):
        for waves in (1, 4):
            blocks = cus * waves                      # 4 waves per block: `waves` per SIMD
            buf = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
            ms = timed(lambda: lib.probe_mfma(fp8, blocks, iters, ctypes.c_void_p(buf.data_ptr()),
                                              ctypes.c_void_p(stream)))
            out[f"{name}_tflops_{waves}w"] = round(lib.probe_mfma_flop(fp8, blocks, iters) / (ms * 1e-3) / 1e12, 1)
            del buf
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    red = torch.empty(cus * 8, dtype=torch.int32, device=dev)
    ms = timed(lambda: lib.probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                                      cus * 8, ctypes.c_void_p(stream)))
    out["hbm_copy_gbs"] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
    ms = timed(lambda: lib.probe_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(red.data_ptr()),
                                      cus * 8, ctypes.c_void_p(stream)))
    out["hbm_read_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del src, dst, red
    # the grouped GEMMs' operand stream alone (LDS-DMA, 256-row panels, 128-byte K steps), on
    # L2-resident panels and on panels arriving from HBM in the products' 8 x 4 cells; a 256 x 256
    # tile does 256 * 256 * 2 * K flops per 512 * K-step bytes: 256 flop per streamed byte in fp8
    # (K = 128 per step), 128 in bf16 (K = 64)
    lib.probe_dma_bytes.restype = ctypes.c_double
    lib.probe_dma_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.probe_dma_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    kbytes, rounds, pbytes = 7168, 4, 512 << 20
    npanels = pbytes // (256 * kbytes)
    pa = torch.ones(pbytes, dtype=torch.uint8, device=dev)
    pb = torch.ones(pbytes, dtype=torch.uint8, device=dev)
    for name, shared in (("lds_dma_l2_gbs", 1), ("lds_dma_hbm_cells_gbs", 0)):
        ms = timed(lambda: lib.probe_dma_stream(ctypes.c_void_p(pa.data_ptr()), ctypes.c_void_p(pb.data_ptr()), kbytes,
                                                npanels, rounds, shared, cus, ctypes.c_void_p(stream)))
        out[name] = round(lib.probe_dma_bytes(cus, kbytes, rounds) / (ms * 1e-3) / 1e9, 1)
    # the products' K step alone (stream + fragment reads + block-scaled fp8 MFMAs, no scales,
    # no epilogue), and with one part removed at a time
    lib.probe_kstep_flop.restype = ctypes.c_double
    lib.probe_kstep_flop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.probe_kstep.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    kout = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    ks = {}
    for name, v in (("4_waves", 0), ("8_waves", 1), ("4_waves_no_dma", 2), ("4_waves_no_lds_reads", 3)):
        ms = timed(lambda: lib.probe_kstep(v, ctypes.c_void_p(pa.data_ptr()), ctypes.c_void_p(pb.data_ptr()), kbytes,
                                           npanels, 8, cus, ctypes.c_void_p(kout.data_ptr()), ctypes.c_void_p(stream)))
        ks[name] = round(lib.probe_kstep_flop(cus, kbytes, 8) / (ms * 1e-3) / 1e12, 1)
    out["mx_kstep_tflops"] = ks
    del pa, pb, kout
    out["gemm_stream_bound_tflops"] = {"mxfp8": round(out["lds_dma_hbm_cells_gbs"] * 0.256, 1),
                                       "bf16": round(out["lds_dma_hbm_cells_gbs"] * 0.128, 1)}
    out["probe"] = ("expert_ffn_layer_top_amd/probe/ceiling.hip: MFMA-only loops (16 independent "
                    "accumulators per wave, register operands), 1 GiB copy (read + write bytes) and read, "
                    "LDS-DMA operand stream of 256-row panels (shared: L2-resident; cells: 8 x 4 panels per "
                    "XCD per round from 512 MiB buffers); gemm_stream_bound_tflops = the cells rate times the "
                    "flops a 256 x 256 tile does per streamed byte; mx_kstep_tflops = the MX products' K step "
                    "alone (that stream, fragment reads, block-scaled MFMAs) in four and eight waves and with "
                    "the DMA or the fragment reads removed")
    return out


# ------------------------------------------------------------------ counters and CPU baseline

def step_traffic(cfg):
    """{call: HBM bytes per call} from the workload's counter summary, for the calls whose kernel
    sources are unchanged since the counters were taken (others are left out)."""
    from expert_ffn_layer_top_amd import profsum
    t = profsum.read_step_traffic(os.path.join(ROOT, "profiles", f"hbm_traffic_{workload_tag(cfg)}.txt"))
    if t is None:
        return {}
    dtype = "mxfp8" if cfg.mxfp8 else "bf16"
    return {c: v["traffic_bytes"] for c, v in t.items()
            if v["source_sha256"] == profsum.files_sha256(profsum.call_sources(c, dtype, cfg.logits == "router"))}


def _blas_threads():
    import threadpoolctl
    blas = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    return max((p.get("num_threads", 1) for p in blas), default=1)


def cpu_baseline_bf16(cfg, sample_tokens):
    """The oracle as it stands, on the first `sample_tokens` tokens of the same workload (same
    weights, same routing construction), forward + backward, timed on the host cores."""
    import numpy as np

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
    threads = _blas_threads()
    assert np.isfinite(fwd["y"]).all()
    return dict(value=s / secs, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"first {s} of {cfg.T} tokens, full expert weights, fwd+bwd, float64 numpy "
                       f"({secs:.1f} s; BLAS threads {threads}, affinity {len(os.sched_getaffinity(0))} cores)")


def cpu_baseline_mx(cfg, sample_tokens=1024, sample_rows=128):
    """The MXFP8 oracle chain (oracle.moe_mx) on a bounded sample, scaled to the whole step.

    Its per-step work has three parts that scale differently, each timed on a sample:
      per token   router projection and its backward, route and metadata, permute, combine, their
                  backward, on the first `sample_tokens` tokens (scaled by T / sample);
      per expert  the MX quantisation of one expert's three weights in both directions (x E);
      per row     one expert's forward and backward products on `sample_rows` of its rows, with
                  every activation quantisation (x n / rows)."""
    import numpy as np

    import synth
    from oracle import moe, moe_mx, mxfp8

    s = min(sample_tokens, cfg.T)
    x = synth.gen_x(cfg)[:s]
    dy = synth.gen_dy(cfg)[:s]
    w_r = synth.gen_router_weight(cfg)
    wg, wu, wd = synth.gen_expert_weights(cfg.with_(E=1))      # one expert's shapes, drawn for timing only
    t0 = time.perf_counter()
    logits = moe.router_project(x, w_r)
    idx, gate, _ = moe.route_topk(logits, cfg.k)
    counts, off, dest, row_token, offp = moe.route_metadata(idx, cfg.E)
    xq, xs = mxfp8.quantize_rows(x)
    moe.permute(xq, dest), moe.permute(xs, dest)
    yexp = np.zeros((s * cfg.k, cfg.d))
    y = moe.combine(yexp, gate, dest)
    _, dg = moe.combine_bwd(dy, yexp, gate, dest)
    dl = moe.route_topk_bwd(gate, idx, dg, cfg.E)
    add, _ = moe.router_project_bwd(x, w_r, dl)
    moe.permute_bwd(yexp, dest, addend=add)
    t_tok = time.perf_counter() - t0
    t0 = time.perf_counter()
    qw = moe_mx.quantize_weights(wg, wu, wd)
    t_w = time.perf_counter() - t0
    R = sample_rows
    xr = np.repeat(x, (R + s - 1) // s, axis=0)[:R]
    dyr = np.repeat(dy, (R + s - 1) // s, axis=0)[:R]
    t0 = time.perf_counter()
    rq, rs = mxfp8.quantize_rows(xr)
    G, U, A, Y = moe_mx.expert_forward(rq, rs, qw, 0)
    moe_mx.expert_backward(dyr, G, U, A, xr, qw, 0)
    t_rows = time.perf_counter() - t0
    step_s = t_tok * cfg.T / s + t_w * cfg.E + t_rows * cfg.n / R
    threads = _blas_threads()
    assert np.isfinite(y).all()
    return dict(value=cfg.T / step_s, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=(f"MXFP8 oracle chain, three timed parts scaled to the whole step: per-token work on the first "
                        f"{s} of {cfg.T} tokens ({t_tok:.2f} s, x {cfg.T // s}), one expert's weight quantisation "
                        f"({t_w:.2f} s, x {cfg.E}), one expert's fwd+bwd products on {R} rows ({t_rows:.2f} s, "
                        f"x {cfg.n // R}); estimated {step_s:.0f} s per step; float64 numpy, BLAS threads {threads}, "
                        f"affinity {len(os.sched_getaffinity(0))} cores"))


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (no collectives or sharding); use --gpus 1",
              file=sys.stderr)
        return 2
    cfg = workload_config(args)
    r = run_gpu(cfg, args.steps, args.warmup, args.copy_probe, args.recompute, flush=not args.no_flush)
    K = args.steps
    flops = gemm_flops(cfg)
    dom = r["dom"]
    achieved = flops[dom] / (r["dom_ms"] * 1e-3) / 1e12
    peak = PEAK_MXFP8_TFLOPS if cfg.mxfp8 else PEAK_BF16_TFLOPS
    traffic = step_traffic(cfg)
    from expert_ffn_layer_top_amd import profsum
    dtype = "mxfp8" if cfg.mxfp8 else "bf16"
    flushed = not args.no_flush

    def counter_gbs(calls_ms):
        return {c: round(traffic[c] / (v * 1e-3) / 1e9, 1) for c, v in calls_ms.items() if c in traffic}

    out = {
        "metric": METRIC,
        "value": round(cfg.T * K / r["elapsed"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "instrumented_steps": K,           # untimed pass with every call bracketed
        "ms_per_step": round(r["elapsed"] * 1e3 / K, 4),
        "step_ms": dist(r["step_ms"]),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": describe(cfg), "T": cfg.T, "d_model": cfg.d, "experts": cfg.E,
                   "top_k": cfg.k, "d_ff": cfg.f, "fwd_bwd": not cfg.forward_only,
                   "activation_recompute": bool(args.recompute), "instrumented_pass_flushed": flushed},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic.get(dom),
                     "kernel": f"{profsum.kernel_name(dom, dtype, cfg.d, cfg.f)} ({dom})",
                     "avg_ms": round(r["dom_ms"], 4), "flop_per_launch": flops[dom],
                     "algorithmic_bytes": round(gemm_bytes(cfg, dom))},
    }
    if cfg.mxfp8:
        out["ms_per_step_excl_weight_quant"] = round(r["elapsed_nq"] * 1e3 / K, 4)
        out["step_ms_excl_weight_quant"] = dist(r["step_ms_nq"])
    out["step_ms_flushed"] = dist(r["step_flushed"])
    out["gemm_ms"] = {c: round(v, 4) for c, v in r["gemm_ms"].items()}
    out["gemm_tflops"] = {c: round(flops[c] / (v * 1e-3) / 1e12, 1) for c, v in r["gemm_ms"].items()}
    out["rows_us"] = {c: round(v * 1e3, 1) for c, v in r["row_ms"].items()}
    out["rows_hbm_gbs"] = {c: round(row_bytes(cfg, c) / (v * 1e-3) / 1e9, 1) for c, v in r["row_ms"].items()}
    out["rows_counter_gbs"] = counter_gbs(r["row_ms"])
    if r["aux_ms"]:
        out["aux_us"] = {c: round(v * 1e3, 1) for c, v in r["aux_ms"].items()}
        out["aux_hbm_gbs"] = {c: round(aux_bytes(cfg, c) / (v * 1e-3) / 1e9, 1) for c, v in r["aux_ms"].items()}
        out["aux_counter_gbs"] = counter_gbs(r["aux_ms"])
    out["counter_bytes_over_algorithmic"] = {
        c: round(traffic[c] / (row_bytes(cfg, c) if c in r["row_ms"] else aux_bytes(cfg, c)), 3)
        for c in list(r["row_ms"]) + list(r["aux_ms"]) if c in traffic}
    out["hbm_peak_gbs"] = HBM_PEAK_GBS
    if not args.no_ceilings:
        c = measured_ceilings()
        out["measured_ceilings"] = c
        mf = c["mfma_fp8_tflops_4w" if cfg.mxfp8 else "mfma_bf16_tflops_4w"]
        out["roofline"]["frac_of_measured_mfma_ceiling"] = round(achieved / mf, 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_mx(cfg) if cfg.mxfp8 else cpu_baseline_bf16(cfg, 8192)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
