"""Builds the HIP library libmoe_mi355x.so for gfx950 in-tree.

    python -m expert_ffn_layer_top_amd.build [--jobs N] [--verbose]

Each csrc/*.hip is compiled to an object under _build/ (in parallel), then linked into
expert_ffn_layer_top_amd/libmoe_mi355x.so.  The ceiling probes (probe/*.hip: MFMA-only loops and
streaming copies the benchmark times beside the layer) go into a separate libmoe_probe.so, which
is not part of the layer's ABI.  Always recompiles: this is the "does it build" step, and it
must reflect the sources as they are.
"""

import argparse
import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
PROBE = os.path.join(PKG, "probe")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
PROBE_LIB = os.path.join(PKG, "libmoe_probe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall", "-Wno-unused-result",
    # no packed fp32 VALU instructions (v_pk_*_f32) in any device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def _link(srcs, lib, jobs, verbose):
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        futs = [ex.submit(_run, [HIPCC, *CFLAGS, "-c", s, "-o", o], verbose) for s, o in zip(srcs, objs)]
        for fut in futs:
            fut.result()
    tmp = lib + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)


def build(jobs=8, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    _link(srcs, LIB, jobs, verbose)
    _link(sorted(glob.glob(os.path.join(PROBE, "*.hip"))), PROBE_LIB, jobs, verbose)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
