"""Text summaries of rocprofv3 output (CSV format), for the profiles kept beside the code.

    python -m expert_ffn_layer_top_amd.profsum kernels DIR --title TEXT --command TEXT
        per-kernel calls / total / average / share of a --kernel-trace run
    python -m expert_ffn_layer_top_amd.profsum counters DIR --counter NAME [--counter NAME ...]
            [--match TEXT] --title TEXT --command TEXT
        per-kernel mean of each counter (or derived metric, e.g. MfmaUtil) of a --pmc run
    python -m expert_ffn_layer_top_amd.profsum traffic --fetch DIR --write DIR --kernel NAME
            --call CALL --workload NAME --copy-bytes N --command-fetch TEXT --command-write TEXT
        HBM bytes per dispatch of one kernel from a FETCH_SIZE run and a WRITE_SIZE run, each
        scaled by what the same counter reads for the plain copy kernel (torch's elementwise
        negation of an fp32 buffer of N bytes: N read, N written) dispatched in the same run

    python -m expert_ffn_layer_top_amd.profsum step-traffic --fetch DIR --write DIR --workload NAME
            --copy-bytes N --command-fetch TEXT --command-write TEXT
        HBM bytes per call of one layer step (every routing, row-movement, router, quantiser and
        grouped-GEMM call): the library's dispatches of each complete step are assigned to the
        step's calls in launch order (STEP_SEQUENCE), counter values summed per call and averaged
        over the steps that follow a cache flush (the benchmark's instrumented pass), each
        counter scaled by the copy kernel's reading as above
    python -m expert_ffn_layer_top_amd.profsum step-kernels DIR --workload NAME --title TEXT --command TEXT
        per-call durations of the same steps from a --kernel-trace run

DIR is a rocprofv3 output directory written with `--output-format csv`.  The traffic summary
records the sha256 of the kernel's source files (SOURCES), so a reader can tell whether the
counters still describe the code as it stands.
"""

import argparse
import csv
import glob
import hashlib
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# the files a grouped-GEMM kernel is compiled from, per dtype
SOURCES = {
    "bf16": ("gemm_bf16.hip", "gemm_epilogue.h", "gemm_sched.h", "common.h"),
    "mxfp8": ("gemm_mx.hip", "gemm_epilogue.h", "gemm_sched.h", "common.h", "mx_common.h"),
}

# rocprofv3 kernel name of each grouped-GEMM call (the kernel template's mode number)
CALL_MODE = {"gate_up": 0, "down": 1, "dgrad_down": 2, "dgrad_gate_up": 3, "wgrad_down": 4, "wgrad_gate_up": 5}
COPY_KERNEL = "neg_kernel"

# source files of each kind of call (a summary is valid while their hash is unchanged)
CALL_SOURCES = {
    "route": ("route.hip", "common.h"),
    "rows": ("rows.hip", "common.h", "mx_common.h"),
    "router": ("router.hip", "common.h"),
    "quant": ("mxfp8.hip", "mx_common.h", "common.h"),
}
GEMM_CALLS = ("gate_up", "down", "dgrad_down", "wgrad_down", "dgrad_gate_up", "wgrad_gate_up")


def call_sources(call, dtype, router=False):
    """The csrc files whose code one call of the layer step runs (router: the layer owns its
    router, so the permute backward is the router file's fused kernel)."""
    if call in GEMM_CALLS or call == "recompute":
        return SOURCES[dtype]
    if call in ("route", "route_bwd"):
        return CALL_SOURCES["route"]
    if call in ("router", "router_bwd") or (call == "permute_bwd" and router):
        return CALL_SOURCES["router"]
    if call.startswith("quant_"):
        return CALL_SOURCES["quant"]
    return CALL_SOURCES["rows"]


def files_sha256(names):
    h = hashlib.sha256()
    for name in sorted(set(names)):
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def step_sequence(mxfp8, router, forward_only=False):
    """The library kernels one layer step launches, per call, in launch order (bench.py's step:
    the weights' MXFP8 quantisation, then layer.forward and layer.backward).  Each kernel is
    (base name, template arguments or None for any)."""
    gm = "mx_grouped_gemm_kernel" if mxfp8 else "grouped_gemm_kernel"

    def g(mode):
        return (gm, str(mode)) if not mxfp8 else (gm, f"{mode},")

    seq = []
    if mxfp8:
        seq.append(("quant_w", [("quant_both_kernel", None)] * 3))
    if router:
        seq.append(("router", [("router_fwd_kernel", None)]))
    seq.append(("route", [("route_topk_local", None), ("route_scan", None), ("route_finalize", None)]))
    if mxfp8:
        seq += [("permute", [("permute_mx_kernel", None)]), ("gate_up", [g(0)]),
                ("quant_a", [("quant_rows_grouped_kernel", None)]), ("down", [g(1)])]
    else:
        seq += [("permute", [("permute_kernel", None)]), ("gate_up", [g(0)]), ("down", [g(1)])]
    seq.append(("combine", [("combine_kernel", None)]))
    if forward_only:
        return seq
    seq.append(("combine_bwd", [("combine_bwd_mx_kernel" if mxfp8 else "combine_bwd_kernel", None)]))
    seq.append(("route_bwd", [("route_topk_bwd_kernel", None)]))
    if router:
        seq.append(("router_bwd", [("split_parts", None), ("router_dw_kernel", None), ("reduce_splits", None)]))
    # with a router, the permute backward adds the router's dx term in the same kernel
    pb = ("permute_bwd", [("split_parts", None), ("split_parts", None), ("router_dx_kernel", "true,")] if router
          else [("permute_bwd_kernel", None)])
    if mxfp8:
        qg = ("quant_grouped_kernel", None)
        seq += [("dgrad_down", [g(2)]), ("quant_dyT", [qg]), ("wgrad_down", [g(4)]),
                ("quant_dg", [("quant_rows_grouped_kernel", None)]), ("quant_du", [("quant_rows_grouped_kernel", None)]),
                ("dgrad_gate_up", [g(3)]), pb, ("quant_xT", [qg]), ("wgrad_gate_up", [g(5)])]
    else:
        seq += [("dgrad_down", [g(2)]), ("wgrad_down", [g(4)]), ("dgrad_gate_up", [g(3)]), pb,
                ("wgrad_gate_up", [g(5)])]
    return seq


def workload_router(workload):
    """Whether the named workload's layer owns its router (router-projected logits)."""
    return workload in ("mxfp8", "tiny")


def workload_sequence(workload):
    """step_sequence of a named workload (tiny, balanced, sweep*, skewed, mxfp8)."""
    if workload == "mxfp8":
        return step_sequence(True, True)
    if workload == "tiny":
        return step_sequence(False, True, forward_only=True)
    return step_sequence(False, False)


def _base_targs(short_name):
    """('grouped_gemm_kernel', '5') from 'moe::gg::grouped_gemm_kernel<5>'."""
    head, _, targs = short_name.partition("<")
    return head.rsplit("::", 1)[-1], targs.rstrip(">").replace(" ", "")


def _matches(short_name, pat):
    base, targs = _base_targs(short_name)
    want_base, want_targs = pat
    return base == want_base and (want_targs is None or targs == want_targs or targs.startswith(want_targs))


def _dispatches(d, counter=None):
    """[(dispatch id, short kernel name, value)] in dispatch order: kernel-trace durations (ns)
    when counter is None, else the counter's value."""
    out = []
    if counter is None:
        for f in _csvs(d, "kernel_trace.csv"):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    out.append((int(r["Dispatch_Id"]), short(r["Kernel_Name"]),
                                int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    else:
        for f in _csvs(d, "counter_collection.csv"):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] == counter:
                        out.append((int(r["Dispatch_Id"]), short(r["Kernel_Name"]), float(r["Counter_Value"])))
    out.sort()
    return out


def step_calls(disp, seq):
    """Complete steps found in the dispatch list: [(flushed, {call: summed value})].  A step is
    flushed when the dispatch just before it is not the library's (the benchmark writes 1 GiB
    with a torch kernel before each instrumented step)."""
    flat = [(call, pat) for call, pats in seq for pat in pats]
    L = len(flat)
    steps = []
    i = 0
    while i + L <= len(disp):
        if all(_matches(disp[i + j][1], flat[j][1]) for j in range(L)):
            flushed = i > 0 and not disp[i - 1][1].startswith("moe::")
            per = {}
            for j, (call, _) in enumerate(flat):
                per[call] = per.get(call, 0.0) + disp[i + j][2]
            steps.append((flushed, per))
            i += L
        else:
            i += 1
    return steps


def _chosen_steps(steps, what):
    if not steps:
        raise SystemExit(f"{what}: no complete layer step found (kernel sequence changed?)")
    fl = [p for f, p in steps if f]
    return (fl, True) if fl else ([p for _, p in steps], False)


def mx_scale_groups(call, d, f):
    """Whether the MXFP8 kernel of `call` loads its scales in four-step groups: the library does
    so for the forward and dgrad products whose contraction dim per operand is a multiple of 512."""
    k = {"gate_up": d, "down": f, "dgrad_down": d, "dgrad_gate_up": f}.get(call)
    return k is not None and k % 512 == 0


def kernel_name(call, dtype, d, f):
    """rocprofv3 name of the kernel behind a grouped-GEMM call at model dims d, f."""
    if dtype == "bf16":
        return f"moe::gg::grouped_gemm_kernel<{CALL_MODE[call]}>"
    flag = "true" if mx_scale_groups(call, d, f) else "false"
    return f"moe::gmx::mx_grouped_gemm_kernel<{CALL_MODE[call]}, {flag}>"


def source_sha256(dtype):
    h = hashlib.sha256()
    for name in SOURCES[dtype]:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short(name):
    """Kernel name without its return type and parameter list (template arguments kept)."""
    name = name.replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            name = name[:i]
            break
    return name[5:] if name.startswith("void ") else name


def _csvs(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    return files


def kernel_durations(d):
    """{kernel: [duration ns, ...]} from the kernel trace CSV."""
    out = {}
    for f in _csvs(d, "kernel_trace.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                out.setdefault(short(r["Kernel_Name"]), []).append(ns)
    return out


def counter_values(d, counter):
    """{kernel: [value per dispatch, ...]} of one counter from a --pmc run."""
    out = {}
    for f in _csvs(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    out.setdefault(short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def cmd_kernels(a):
    dur = kernel_durations(a.dir)
    total = sum(sum(v) for v in dur.values())
    print(f"# {a.title}")
    print(f"# command: {a.command}")
    print("# durations in microseconds, from the rocprofv3 kernel trace (end - start of each dispatch)")
    print(f"{'calls':>6} {'total_us':>11} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel")
    for k, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        print(f"{len(v):6d} {sum(v) / 1e3:11.1f} {statistics.mean(v) / 1e3:10.2f} {min(v) / 1e3:10.2f} "
              f"{max(v) / 1e3:10.2f} {100.0 * sum(v) / total:6.2f}  {k}")


def cmd_counters(a):
    """Per-kernel mean over dispatches of each counter of a --pmc run (derived metrics included)."""
    cols = {c: counter_values(a.dir, c) for c in a.counter}
    kernels = sorted({k for v in cols.values() for k in v if a.match in k})
    print(f"# {a.title}")
    print(f"# command: {a.command}")
    print("# mean over dispatches of each counter, per kernel (rocprofv3 --pmc, CSV output)")
    print(f"{'dispatches':>10} " + " ".join(f"{c:>28}" for c in a.counter) + "  kernel")
    for k in kernels:
        n = max(len(cols[c].get(k, [])) for c in a.counter)
        vals = [statistics.mean(cols[c][k]) if cols[c].get(k) else float("nan") for c in a.counter]
        print(f"{n:10d} " + " ".join(f"{v:28.6g}" for v in vals) + f"  {k}")


def _one(values, name, what):
    hits = {k: v for k, v in values.items() if name in k}
    if len(hits) != 1:
        raise SystemExit(f"{what}: expected one kernel matching {name!r}, found {sorted(hits)}")
    (k, v), = hits.items()
    return k, statistics.mean(v), len(v)


def cmd_traffic(a):
    dtype = "mxfp8" if "gmx" in a.kernel else "bf16"
    fetch = counter_values(a.fetch, "FETCH_SIZE")
    write = counter_values(a.write, "WRITE_SIZE")
    k, f_kib, nf = _one(fetch, a.kernel, "FETCH_SIZE")
    _, w_kib, nw = _one(write, a.kernel, "WRITE_SIZE")
    _, cf_kib, _ = _one(fetch, COPY_KERNEL, "FETCH_SIZE copy")
    _, cw_kib, _ = _one(write, COPY_KERNEL, "WRITE_SIZE copy")
    ff = a.copy_bytes / (cf_kib * 1024.0)
    fw = a.copy_bytes / (cw_kib * 1024.0)
    fetch_b = f_kib * 1024.0 * ff
    write_b = w_kib * 1024.0 * fw
    print(f"# HBM traffic per dispatch of {k} ({a.call}), workload {a.workload}")
    print(f"# command (FETCH_SIZE): {a.command_fetch}")
    print(f"# command (WRITE_SIZE): {a.command_write}")
    print(f"# calibration: {COPY_KERNEL} over an fp32 buffer of {a.copy_bytes} bytes in the same runs "
          f"(reads and writes exactly that many bytes)")
    print(f"kernel: {k}")
    print(f"call: {a.call}")
    print(f"workload: {a.workload}")
    print(f"source_sha256: {source_sha256(dtype)}")
    print(f"dispatches: fetch {nf}, write {nw}")
    print(f"fetch_kib_per_dispatch: {f_kib:.1f}")
    print(f"write_kib_per_dispatch: {w_kib:.1f}")
    print(f"copy_fetch_kib: {cf_kib:.1f}")
    print(f"copy_write_kib: {cw_kib:.1f}")
    print(f"fetch_factor: {ff:.4f}")
    print(f"write_factor: {fw:.4f}")
    print(f"fetch_bytes: {fetch_b:.0f}")
    print(f"write_bytes: {write_b:.0f}")
    print(f"traffic_bytes: {fetch_b + write_b:.0f}")


def cmd_step_traffic(a):
    seq = workload_sequence(a.workload.split("_")[0])
    fetch = _dispatches(a.fetch, "FETCH_SIZE")
    write = _dispatches(a.write, "WRITE_SIZE")
    cf = [v for _, k, v in fetch if COPY_KERNEL in k]
    cw = [v for _, k, v in write if COPY_KERNEL in k]
    if not cf or not cw:
        raise SystemExit(f"no {COPY_KERNEL} dispatch (run the benchmark with --copy-probe)")
    ff = a.copy_bytes / (statistics.mean(cf) * 1024.0)
    fw = a.copy_bytes / (statistics.mean(cw) * 1024.0)
    fs, ffl = _chosen_steps(step_calls(fetch, seq), "FETCH_SIZE")
    ws, wfl = _chosen_steps(step_calls(write, seq), "WRITE_SIZE")
    dtype = "mxfp8" if a.workload.startswith("mxfp8") else "bf16"
    print(f"# HBM traffic per call of one layer step, workload {a.workload}")
    print(f"# command (FETCH_SIZE): {a.command_fetch}")
    print(f"# command (WRITE_SIZE): {a.command_write}")
    print(f"# calibration: {COPY_KERNEL} over an fp32 buffer of {a.copy_bytes} bytes in the same runs "
          f"(reads and writes exactly that many bytes): fetch_factor {ff:.4f}, write_factor {fw:.4f}")
    print(f"# steps averaged: fetch {len(fs)} ({'flushed' if ffl else 'not flushed'}), "
          f"write {len(ws)} ({'flushed' if wfl else 'not flushed'}); bytes per call = counter KiB * 1024 * factor")
    print(f"{'call':<14} {'fetch_bytes':>14} {'write_bytes':>14} {'traffic_bytes':>14}  source_sha256  kernels")
    for call, pats in seq:
        fb = statistics.mean(p[call] for p in fs) * 1024.0 * ff
        wb = statistics.mean(p[call] for p in ws) * 1024.0 * fw
        kern = "+".join(b if t is None else f"{b}<{t.rstrip(',')}>" for b, t in pats)
        src = call_sources(call, dtype, workload_router(a.workload.split("_")[0]))
        print(f"{call:<14} {fb:14.0f} {wb:14.0f} {fb + wb:14.0f}  {files_sha256(src)}  {kern}")


def cmd_step_kernels(a):
    seq = workload_sequence(a.workload.split("_")[0])
    steps, flushed = _chosen_steps(step_calls(_dispatches(a.dir), seq), "kernel trace")
    print(f"# {a.title}")
    print(f"# command: {a.command}")
    print(f"# per-call kernel time (sum of the call's dispatches, end - start) over {len(steps)} complete "
          f"{'flushed ' if flushed else ''}steps, microseconds")
    dtype = "mxfp8" if a.workload.startswith("mxfp8") else "bf16"
    print(f"{'call':<14} {'median_us':>10} {'mean_us':>10} {'min_us':>10} {'max_us':>10}  source_sha256  kernels")
    total = 0.0
    for call, pats in seq:
        v = [p[call] / 1e3 for p in steps]
        total += statistics.median(v)
        kern = "+".join(b if t is None else f"{b}<{t.rstrip(',')}>" for b, t in pats)
        print(f"{call:<14} {statistics.median(v):10.1f} {statistics.mean(v):10.1f} {min(v):10.1f} {max(v):10.1f}  "
              f"{files_sha256(call_sources(call, dtype, workload_router(a.workload.split('_')[0])))}  {kern}")
    print(f"{'sum':<14} {total:10.1f}")


def read_step_traffic(path):
    """{call: dict(fetch_bytes, write_bytes, traffic_bytes, source_sha256)} from a step-traffic
    summary, or None if the file is missing."""
    if not os.path.exists(path):
        return None
    out = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or line.startswith("call "):
                continue
            f = line.split()
            if len(f) >= 5:
                out[f[0]] = dict(fetch_bytes=float(f[1]), write_bytes=float(f[2]), traffic_bytes=float(f[3]),
                                 source_sha256=f[4])
    return out


def read_traffic(path):
    """{key: value} of a traffic summary (values as strings), or None if the file is missing."""
    if not os.path.exists(path):
        return None
    out = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or ":" not in line:
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = val.strip()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("dir")
    k.add_argument("--title", required=True)
    k.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--counter", action="append", required=True)
    c.add_argument("--match", default="", help="only kernels whose name contains this")
    c.add_argument("--title", required=True)
    c.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--call", required=True, choices=sorted(CALL_MODE))
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    st = sub.add_parser("step-traffic")
    st.add_argument("--fetch", required=True)
    st.add_argument("--write", required=True)
    st.add_argument("--workload", required=True)
    st.add_argument("--copy-bytes", type=int, required=True)
    st.add_argument("--command-fetch", required=True)
    st.add_argument("--command-write", required=True)
    sk = sub.add_parser("step-kernels")
    sk.add_argument("dir")
    sk.add_argument("--workload", required=True)
    sk.add_argument("--title", required=True)
    sk.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    {"kernels": cmd_kernels, "counters": cmd_counters, "traffic": cmd_traffic, "step-traffic": cmd_step_traffic,
     "step-kernels": cmd_step_kernels}[a.cmd](a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
