"""Pins of the oracle's router balance score and its gradient (oracle/moe.py router_balance,
router_balance_bwd) against closed forms, the gerrymandering case the pages describe, finite
differences and the softmax's shift invariance."""

import numpy as np

from oracle import moe


def _softmax(lg):
    z = lg - lg.max(axis=1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=1, keepdims=True)


def test_uniform_probs_and_balanced_load_give_one():
    T, E, k = 64, 8, 2
    logits = np.zeros((T, E))
    idx = np.stack([(np.arange(T) * k + j) % E for j in range(k)], axis=1)   # round-robin selection
    counts = np.bincount(idx.ravel(), minlength=E)
    b = moe.router_balance(_softmax(logits), counts, k)
    assert b["aux"] == 1.0 and b["load_max"] == 1.0 and b["load_cv"] == 0.0
    assert abs(b["prob_max"] - 1.0) < 1e-15


def test_everything_on_one_expert_gives_E():
    T, E, k = 32, 4, 1
    logits = np.zeros((T, E))
    logits[:, 0] = 80.0                                      # probs = one-hot up to e^-80
    idx, _, probs = moe.route_topk(logits, k)
    counts = np.bincount(idx.ravel(), minlength=E)
    b = moe.router_balance(probs, counts, k)
    assert abs(b["aux"] - E) < 1e-12 and b["load_max"] == E and abs(b["prob_max"] - E) < 1e-12
    assert abs(b["load_cv"] - np.sqrt(E - 1)) < 1e-12       # f = (1, 0, .., 0): std/mean = sqrt(E-1)


def test_gerrymandering_score_blind_to_concentrated_load():
    """Equal logits: every probability is 1/E, so the score sits at its balanced value 1, yet the
    selection (ties to the lower expert id) sends every token to experts 0..k-1."""
    T, E, k = 50, 8, 2
    idx, _, probs = moe.route_topk(np.zeros((T, E)), k)
    counts = np.bincount(idx.ravel(), minlength=E)
    assert list(counts[:k]) == [T] * k and counts[k:].sum() == 0
    b = moe.router_balance(probs, counts, k)
    assert abs(b["aux"] - 1.0) < 1e-12
    assert b["load_max"] == E / k


def test_gradient_matches_finite_differences():
    rng = np.random.default_rng(7)
    T, E, k, wgt = 12, 6, 2, 0.37
    logits = rng.standard_normal((T, E))
    idx, _, _ = moe.route_topk(logits, k)
    counts = np.bincount(idx.ravel(), minlength=E)           # held constant, as in the backward
    g = moe.router_balance_bwd(_softmax(logits), counts, k, wgt)
    h = 1e-6
    num = np.zeros_like(logits)
    for t in range(T):
        for e in range(E):
            lp, lm = logits.copy(), logits.copy()
            lp[t, e] += h
            lm[t, e] -= h
            num[t, e] = wgt * (moe.router_balance(_softmax(lp), counts, k)["aux"]
                               - moe.router_balance(_softmax(lm), counts, k)["aux"]) / (2 * h)
    assert np.max(np.abs(g - num)) <= 1e-8 * max(1.0, np.max(np.abs(num)))
    assert np.max(np.abs(g.sum(axis=1))) < 1e-15            # adding a constant to a row changes nothing


def test_brute_force_loop():
    rng = np.random.default_rng(3)
    T, E, k = 9, 5, 3
    probs = _softmax(rng.standard_normal((T, E)))
    counts = rng.integers(0, 10, size=E)
    aux = 0.0
    for e in range(E):
        fe = counts[e] / (T * k)
        pe = sum(probs[t, e] for t in range(T)) / T
        aux += fe * pe
    assert abs(moe.router_balance(probs, counts, k)["aux"] - E * aux) < 1e-13


def test_gradient_matches_torch_autograd():
    """CPU torch autograd in float64 through softmax and the score, counts held constant."""
    import torch
    rng = np.random.default_rng(11)
    T, E, k, wgt = 40, 9, 3, 1.7
    logits = rng.standard_normal((T, E)) * 2
    idx, _, _ = moe.route_topk(logits, k)
    counts = np.bincount(idx.ravel(), minlength=E)
    lt = torch.tensor(logits, dtype=torch.float64, requires_grad=True)
    p = torch.softmax(lt, dim=1)
    f = torch.tensor(counts / (T * k), dtype=torch.float64)
    aux = E * torch.sum(f * p.mean(dim=0))
    (wgt * aux).backward()
    g = moe.router_balance_bwd(_softmax(logits), counts, k, wgt)
    assert np.max(np.abs(lt.grad.numpy() - g)) < 1e-15
    assert abs(aux.item() - moe.router_balance(_softmax(logits), counts, k)["aux"]) < 1e-14
