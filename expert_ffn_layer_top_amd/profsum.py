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
    a = ap.parse_args(argv)
    {"kernels": cmd_kernels, "counters": cmd_counters, "traffic": cmd_traffic}[a.cmd](a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
