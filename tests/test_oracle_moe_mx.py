"""Pins for the oracle's MXFP8 layer chain (oracle/moe_mx.py) against things other than itself:
exact arithmetic where the MX format loses nothing, and the unquantised float64 layer within the
error E4M3 rounding can cause."""

import numpy as np

from oracle import codecs, moe, moe_mx
from synth import to_bf16_bits


def _mx_exact(rows, cols, unit, rng):
    """bf16 values i * unit (integers |i| <= 8) whose every 32-block along either axis holds a
    +-8: amax is 8 * unit in every block, so each element divided by the block scale is an E4M3
    code (32 i) and MX quantisation along rows or columns is exact."""
    i = rng.integers(-7, 8, size=(rows, cols)).astype(np.float32)
    r, c = np.meshgrid(np.arange(rows), np.arange(cols), indexing="ij")
    i[(r % 32) == (c % 32)] = 8 * rng.choice([-1, 1], size=int(np.sum((r % 32) == (c % 32))))
    return to_bf16_bits(i * np.float32(unit))


def test_first_products_exact_on_mx_exact_operands():
    # k = 1 (every gate is exactly 1, so dYexp = dy), MX-exact x, weights and dy: the forward
    # gate/up products and the backward's first product through W_down lose nothing to
    # quantisation, so they equal the exact products of the bf16 values.
    rng = np.random.default_rng(0)
    T, d, f, E, k = 64, 64, 96, 2, 1
    x = _mx_exact(T, d, 1.0, rng)
    dy = _mx_exact(T, d, 0.25, rng)
    wg = np.stack([_mx_exact(f, d, 2.0 ** -6, rng) for _ in range(E)])
    wu = np.stack([_mx_exact(f, d, 2.0 ** -6, rng) for _ in range(E)])
    wd = np.stack([_mx_exact(d, f, 2.0 ** -6, rng) for _ in range(E)])
    logits = rng.standard_normal((T, E)).astype(np.float32)
    qw = moe_mx.quantize_weights(wg, wu, wd)
    fwd = moe_mx.layer_forward_mx(x, None, k, qw, logits=logits)
    bwd = moe_mx.layer_backward_mx(fwd, x, dy, None, qw)
    X = codecs.bf16_to_f64(moe.permute(x, fwd["dest"]))
    dY = codecs.bf16_to_f64(moe.permute(dy, fwd["dest"]))
    assert np.array_equal(codecs.bf16_to_f64(bwd["dyexp"]), dY)
    seen = 0
    for e, r0, r1 in moe._segments(fwd["offsets"]):
        G = X[r0:r1] @ codecs.bf16_to_f64(wg[e]).T
        U = X[r0:r1] @ codecs.bf16_to_f64(wu[e]).T
        assert np.array_equal(fwd["G"][r0:r1], codecs.f64_to_bf16(G))
        assert np.array_equal(fwd["U"][r0:r1], codecs.f64_to_bf16(U))
        dA = dY[r0:r1] @ codecs.bf16_to_f64(wd[e])
        dG, dU = moe.swiglu_bwd(dA, codecs.bf16_to_f64(fwd["G"][r0:r1]), codecs.bf16_to_f64(fwd["U"][r0:r1]))
        assert np.array_equal(bwd["dG"][r0:r1], codecs.f64_to_bf16(dG))
        assert np.array_equal(bwd["dU"][r0:r1], codecs.f64_to_bf16(dU))
        seen += r1 - r0
    assert seen == T * k


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def _rel2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_chain_within_e4m3_error_of_unquantised_layer():
    # Random operands: every result of the MX chain stays within the error E4M3 rounding causes
    # (an element moves by up to 2^-4 of itself, both operands of every product are rounded,
    # and the chain has up to three products in a row: about 8% in norm here), and quantisation
    # did change it.  A dropped term, a wrong sign or a swapped operand moves a result by its own
    # size.
    rng = np.random.default_rng(1)
    T, d, f, E, k = 96, 64, 96, 4, 2
    x = to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    dy = to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    w_r = (0.3 * rng.standard_normal((d, E))).astype(np.float32)
    wg, wu = (to_bf16_bits(0.1 * rng.standard_normal((E, f, d)).astype(np.float32)) for _ in range(2))
    wd = to_bf16_bits(0.1 * rng.standard_normal((E, d, f)).astype(np.float32))
    qw = moe_mx.quantize_weights(wg, wu, wd)
    fwd = moe_mx.layer_forward_mx(x, w_r, k, qw)
    bwd = moe_mx.layer_backward_mx(fwd, x, dy, w_r, qw)
    ref = moe.layer_forward(x, fwd["logits"], k, wg, wu, wd)
    assert np.array_equal(ref["dest"], fwd["dest"])
    rb = moe.layer_backward(ref, dy, wg, wu, wd)
    add, dwr = moe.router_project_bwd(x, w_r, rb["d_logits"])
    rdx = rb["dx"] + add
    for name, got, want in (("y", fwd["y"], ref["y"]), ("dx", bwd["dx"], rdx),
                            ("dw_gate", bwd["dw_gate"], rb["dw_gate"]), ("dw_up", bwd["dw_up"], rb["dw_up"]),
                            ("dw_down", bwd["dw_down"], rb["dw_down"]), ("dw_r", bwd["dw_r"], dwr)):
        e2, em = _rel2(got, want), _rel(got, want)
        assert 1e-3 < e2 < 0.12 and em < 0.3, (name, e2, em)
    # dyexp is bf16(gate * dy): the combine backward's product stored once
    assert _rel(codecs.bf16_to_f64(bwd["dyexp"]), rb["dyexp"]) <= 2.0 ** -8
