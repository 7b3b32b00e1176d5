"""The row/expert-restricted evaluators used for full-size checks agree with the full
oracle on a small problem (each is the same definition restricted to some rows)."""

import numpy as np

from oracle import codecs, moe, sampled
from synth import to_bf16_bits


def test_sampled_helpers_agree_with_full_oracle():
    rng = np.random.default_rng(21)
    T, d, E, k, f = 40, 16, 5, 2, 12
    x = to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    logits = rng.standard_normal((T, E))
    wg = to_bf16_bits((rng.standard_normal((E, f, d)) * 0.2).astype(np.float32))
    wu = to_bf16_bits((rng.standard_normal((E, f, d)) * 0.2).astype(np.float32))
    wd = to_bf16_bits((rng.standard_normal((E, d, f)) * 0.2).astype(np.float32))
    dy = to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    fwd = moe.layer_forward(x, logits, k, wg, wu, wd)
    bwd = moe.layer_backward(fwd, dy, wg, wu, wd)
    rows = np.array([0, 3, 17, 41, 79])
    experts = np.searchsorted(fwd["offsets"], rows, side="right") - 1
    G, U, A, Y = sampled.ffn_forward_rows(fwd["xp"][rows], experts, wg, wu, wd)
    for got, key in ((G, "G"), (U, "U"), (A, "A"), (Y, "yexp")):
        assert np.allclose(got, fwd[key][rows], rtol=1e-13, atol=1e-14)
    dg = sampled.ffn_dgrad_rows(bwd["dyexp"][rows], fwd["G"][rows], fwd["U"][rows], experts, wg, wu, wd)
    for key in ("dA", "dG", "dU", "dxp"):
        assert np.allclose(dg[key], bwd[key][rows], rtol=1e-13, atol=1e-14)
    dxp = sampled.ffn_dxp_rows(bwd["dG"][rows], bwd["dU"][rows], experts, wg, wu)
    assert np.allclose(dxp, bwd["dxp"][rows], rtol=1e-13, atol=1e-14)
    e = int(np.argmax(fwd["counts"]))
    r0, r1 = fwd["offsets"][e], fwd["offsets"][e + 1]
    dwg, dwu, dwd = sampled.wgrad_expert(fwd["xp"][r0:r1], fwd["A"][r0:r1], bwd["dG"][r0:r1],
                                         bwd["dU"][r0:r1], bwd["dyexp"][r0:r1])
    assert np.allclose(dwg, bwd["dw_gate"][e]) and np.allclose(dwu, bwd["dw_up"][e])
    assert np.allclose(dwd, bwd["dw_down"][e])
    assert codecs.bf16_to_f64(x).shape == (T, d)
