"""GPU parity of the router balance score (moe_route_balance) and of the route backward with the
score's gradient (moe_route_topk_bwd_balance), against the oracle (router_balance,
router_balance_bwd, route_topk_bwd) on the GPU's own probabilities and counts."""

import numpy as np
import pytest

from oracle import moe
from tests.gpu_util import assert_close, host, note

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    import torch
    return torch.as_tensor(np.ascontiguousarray(a), dtype=dtype).to("cuda:0")


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (300, 8, 2), (1000, 64, 4), (4097, 128, 8), (513, 256, 16), (257, 3, 3)])
def test_balance_score_and_gradient(T, E, k):
    import torch
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(T * 7 + E)
    logits = (rng.standard_normal((T, E)) * 2.0).astype(np.float32)
    logits[:, 0] += 1.5                                   # an overloaded expert
    note(f"balance T={T} E={E} k={k}")
    r = ops.route_topk(_dev(logits, torch.float32), k, want_probs=True)
    probs, counts = host(r["probs"]), host(r["counts"])
    p_mean, stats = ops.route_balance(r["probs"], r["counts"], k)
    ref = moe.router_balance(probs, counts, k)
    assert_close(host(p_mean), ref["p_mean"], 1e-5, "p_mean")
    got = host(stats)
    for i, key in enumerate(("aux", "load_max", "prob_max", "load_cv")):
        assert abs(got[i] - ref[key]) <= 1e-5 * max(1.0, abs(ref[key])), f"{key}: {got[i]} vs {ref[key]}"
    # bit-reproducible (fixed-order sums)
    p2, s2 = ops.route_balance(r["probs"], r["counts"], k)
    assert torch.equal(p2, p_mean) and torch.equal(s2, stats)
    # backward: route term + weighted balance gradient, counts fixed
    d_gate = _dev(rng.standard_normal((T, k)).astype(np.float32), torch.float32)
    w = 0.01
    dl = ops.route_topk_bwd(r["topk_gate"], r["topk_idx"], d_gate, E, balance=(r["probs"], r["counts"], w))
    dl0 = ops.route_topk_bwd(r["topk_gate"], r["topk_idx"], d_gate, E)
    ref_route = moe.route_topk_bwd(host(r["topk_gate"]), host(r["topk_idx"]), host(d_gate), E)
    ref_bal = moe.router_balance_bwd(probs, counts, k, w)
    assert_close(host(dl0), ref_route, 1e-5, "d_logits (route)")
    assert_close(host(dl), ref_route + ref_bal, 1e-5, "d_logits (route + balance)")
    # the balance term alone (zero upstream gate gradient: the route term is exactly 0), at a
    # weight that makes it comparable in size to the route term
    wb = float(T)
    dlb = ops.route_topk_bwd(r["topk_gate"], r["topk_idx"], torch.zeros_like(d_gate), E,
                             balance=(r["probs"], r["counts"], wb))
    ref_b = moe.router_balance_bwd(probs, counts, k, wb)
    # the term is p (c - <p, c>); where the load is even it vanishes exactly, so the bound scales
    # with the largest coefficient c_e = wb E f_e / T rather than with the term itself
    c_max = wb * E * counts.max() / (T * k) / T
    err = np.max(np.abs(host(dlb) - ref_b))
    assert err <= 1e-5 * max(np.max(np.abs(ref_b)), c_max), f"d_logits balance term: error {err:.3e}"


def test_gerrymandering_equal_logits():
    """Equal logits: the score is at its balanced value 1 while every token lands on experts
    0..k-1 (ties to the lower id): the statistics of the counts show the imbalance."""
    import torch
    from expert_ffn_layer_top_amd import ops
    T, E, k = 2048, 16, 2
    r = ops.route_topk(torch.zeros((T, E), dtype=torch.float32, device="cuda:0"), k, want_probs=True)
    _, stats = ops.route_balance(r["probs"], r["counts"], k)
    aux, load_max, prob_max, _ = host(stats)
    assert abs(aux - 1.0) < 1e-6 and abs(prob_max - 1.0) < 1e-6 and load_max == E / k
