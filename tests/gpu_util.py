"""Helpers shared by the GPU parity tests: host <-> device conversions and the error metric.

Error metric (the layer's parity bar): err = max|out - ref| / max|ref| per tensor, with an
all-zero reference requiring an all-zero output.  Floating-point bars: bf16 outputs and
gradients <= 2e-2 against the float64 oracle; MXFP8 products <= 1e-2 against the oracle on the
same dequantised operands.  Integer, index and byte outputs are compared bit for bit.
"""

import sys

import numpy as np
import torch

BF16_TOL = 2e-2
MX_TOL = 1e-2


def note(msg):
    """Names the case on stdout before a GPU step, so a failure that ends the process is
    attributable from what was printed."""
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def bf16_to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def u8_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def f32_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def i32_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def bits(t):
    """bf16 device tensor -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t):
    return t.detach().cpu().numpy()


def rel_err(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    m = np.max(np.abs(ref)) if ref.size else 0.0
    if m == 0.0:
        return float(np.max(np.abs(out))) if out.size else 0.0
    return float(np.max(np.abs(out - ref)) / m)


def assert_close(out, ref, tol, what):
    e = rel_err(out, ref)
    assert e <= tol, f"{what}: max-rel-to-norm error {e:.3e} > {tol:.1e}"
    return e
