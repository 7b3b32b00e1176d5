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


def gemm_group(K):
    """Bytes per run of the MXFP8 GEMM scale layout for contraction length K."""
    return 16 if K % 512 == 0 else (4 if K % 128 == 0 else 1)


def gemm_scales_to_rows(s, R, K):
    """Host: the GEMM scale layout of one or more [R, K] matrices back to row-major [..., R, K/32]
    (byte (r, b) of a matrix sits at ((b / G) R + r) G + b % G of its R * K/32 bytes).  Leading
    dims are kept when s is shaped [..., R, K/32] (as the bindings return it)."""
    s = np.ascontiguousarray(s)
    G, nb = gemm_group(K), K // 32
    if s.ndim >= 2 and s.shape[-2:] == (R, nb):
        lead = s.shape[:-2]
    else:
        lead = () if s.size == R * nb else (s.size // (R * nb),)
    return s.reshape(-1, nb // G, R, G).transpose(0, 2, 1, 3).reshape(lead + (R, nb))
