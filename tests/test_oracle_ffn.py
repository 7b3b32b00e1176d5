"""Pins for the oracle's permute, expert FFN and combine: a dense SwiGLU FFN computed by
CPU torch (an independent library) for one expert and k = 1, a per-token brute force
with no permutation or grouping, identity experts, k = 1 and empty experts."""

import numpy as np
import pytest
import torch

from oracle import codecs, moe
from synth import to_bf16_bits


def rand_bf16(rng, shape, std=1.0):
    return to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def make_problem(seed, T, d, E, k, f, empty=()):
    rng = np.random.default_rng(seed)
    x = rand_bf16(rng, (T, d))
    logits = rng.standard_normal((T, E))
    for e in empty:
        logits[:, e] -= 100.0
    wg = rand_bf16(rng, (E, f, d), 0.1)
    wu = rand_bf16(rng, (E, f, d), 0.1)
    wd = rand_bf16(rng, (E, d, f), 0.1)
    return x, logits, wg, wu, wd


def test_dense_case_matches_torch():
    x, logits, wg, wu, wd = make_problem(0, 37, 24, 1, 1, 40)
    out = moe.layer_forward(x, logits, 1, wg, wu, wd)
    X = torch.from_numpy(codecs.bf16_to_f64(x))
    Wg = torch.from_numpy(codecs.bf16_to_f64(wg[0]))
    Wu = torch.from_numpy(codecs.bf16_to_f64(wu[0]))
    Wd = torch.from_numpy(codecs.bf16_to_f64(wd[0]))
    ref = torch.matmul(torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T), Wd.T).numpy()
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(out["dest"].ravel(), np.arange(37))


@pytest.mark.parametrize("T,d,E,k,f", [(29, 16, 5, 2, 12), (40, 32, 8, 3, 24), (16, 8, 4, 4, 8)])
def test_per_token_brute_force(T, d, E, k, f):
    x, logits, wg, wu, wd = make_problem(T + E, T, d, E, k, f)
    out = moe.layer_forward(x, logits, k, wg, wu, wd)
    X = codecs.bf16_to_f64(x)
    y = np.zeros((T, d))
    for t in range(T):
        # the k experts with the largest logits, gates from the full softmax renormalised
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        p = np.exp(logits[t] - logits[t].max())
        p /= p.sum()
        for e in order:
            g = p[e] / sum(p[i] for i in order)
            h = X[t] @ codecs.bf16_to_f64(wg[e]).T
            u = X[t] @ codecs.bf16_to_f64(wu[e]).T
            a = h / (1 + np.exp(-h)) * u
            y[t] += g * (a @ codecs.bf16_to_f64(wd[e]).T)
    assert np.allclose(out["y"], y, rtol=1e-11, atol=1e-12)


def test_identity_experts_return_gate_weighted_input():
    x, logits, *_ = make_problem(3, 50, 16, 6, 3, 8)
    idx, gate, _ = moe.route_topk(logits, 3)
    _, _, dest, _, _ = moe.route_metadata(idx, 6)
    xp = moe.permute(x, dest)
    y = moe.combine(xp, gate, dest)          # Yexp := Xp
    assert np.allclose(y, codecs.bf16_to_f64(x), rtol=1e-14, atol=1e-14)


def test_k1_combine_is_the_expert_row():
    x, logits, wg, wu, wd = make_problem(4, 30, 16, 4, 1, 8)
    out = moe.layer_forward(x, logits, 1, wg, wu, wd)
    assert np.array_equal(out["y"], out["yexp"][out["dest"][:, 0]])


def test_empty_experts_take_no_part():
    x, logits, wg, wu, wd = make_problem(5, 40, 16, 6, 2, 8, empty=(1, 4))
    out = moe.layer_forward(x, logits, 2, wg, wu, wd)
    assert out["counts"][1] == 0 and out["counts"][4] == 0
    # changing an empty expert's weights changes nothing
    wg2 = wg.copy(); wg2[1] ^= 0x5555
    out2 = moe.layer_forward(x, logits, 2, wg2, wu, wd)
    assert np.array_equal(out["y"], out2["y"])


def test_permute_is_a_bit_copy_and_column_sums():
    rng = np.random.default_rng(6)
    T, d, E, k = 33, 8, 5, 3
    xi = rng.integers(-50, 50, size=(T, d)).astype(np.float32)
    x = to_bf16_bits(xi)
    idx, _, _ = moe.route_topk(rng.standard_normal((T, E)), k)
    _, _, dest, row_token, _ = moe.route_metadata(idx, E)
    xp = moe.permute(x, dest)
    assert np.array_equal(xp, x[row_token])
    assert np.array_equal(codecs.bf16_to_f64(xp).sum(axis=0), k * xi.astype(np.float64).sum(axis=0))
