"""Pins for the oracle's backward: CPU torch autograd in float64 over a per-token
formulation with no permutation (an independent derivation), central finite
differences, and invariants (zero-sum logit gradients, zeros off the selected set,
exact-zero weight gradients for empty experts, linearity in dy)."""

import numpy as np
import pytest
import torch

from oracle import codecs, moe
from synth import to_bf16_bits

torch.set_default_dtype(torch.float64)


def problem(seed, T, d, E, k, f, empty=()):
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    w_r = (rng.standard_normal((d, E)) * 0.3).astype(np.float32)
    wg = to_bf16_bits((rng.standard_normal((E, f, d)) * 0.2).astype(np.float32))
    wu = to_bf16_bits((rng.standard_normal((E, f, d)) * 0.2).astype(np.float32))
    wd = to_bf16_bits((rng.standard_normal((E, d, f)) * 0.2).astype(np.float32))
    dy = to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    logits = moe.router_project(x, w_r)
    for e in empty:
        logits[:, e] -= 100.0
    return x, w_r, logits, wg, wu, wd, dy


def oracle_full(x, w_r, logits, k, wg, wu, wd, dy):
    fwd = moe.layer_forward(x, logits, k, wg, wu, wd)
    bwd = moe.layer_backward(fwd, dy, wg, wu, wd)
    add, dwr = moe.router_project_bwd(x, w_r, bwd["d_logits"])
    dx_total = moe.permute_bwd(bwd["dxp"], fwd["dest"], addend=add)
    return fwd, bwd, dx_total, dwr


def torch_reference(x, w_r, k, wg, wu, wd, dy, empty=()):
    """loss = <dy, y> with y built token by token; the selection is taken from the
    forward values and held fixed, as top-k is piecewise constant."""
    X = torch.tensor(codecs.bf16_to_f64(x), requires_grad=True)
    Wr = torch.tensor(w_r.astype(np.float64), requires_grad=True)
    Wg = torch.tensor(codecs.bf16_to_f64(wg), requires_grad=True)
    Wu = torch.tensor(codecs.bf16_to_f64(wu), requires_grad=True)
    Wd = torch.tensor(codecs.bf16_to_f64(wd), requires_grad=True)
    L = X @ Wr
    if empty:
        mask = torch.zeros(L.shape[1])
        mask[list(empty)] = -100.0
        L = L + mask
    L.retain_grad()
    probs = torch.softmax(L, dim=1)
    sel = torch.topk(L.detach(), k, dim=1).indices   # distinct random logits: no ties
    psel = torch.gather(probs, 1, sel)
    g = psel / psel.sum(dim=1, keepdim=True)
    T = X.shape[0]
    y = torch.zeros_like(X)
    for t in range(T):
        acc = torch.zeros(X.shape[1])
        for j in range(k):
            e = int(sel[t, j])
            h = Wg[e] @ X[t]
            u = Wu[e] @ X[t]
            acc = acc + g[t, j] * (Wd[e] @ (torch.nn.functional.silu(h) * u))
        y[t] = acc
    loss = (y * torch.tensor(codecs.bf16_to_f64(dy))).sum()
    loss.backward()
    return dict(y=y.detach().numpy(), dx=X.grad.numpy(), dwr=Wr.grad.numpy(), dl=L.grad.numpy(),
                dwg=Wg.grad.numpy(), dwu=Wu.grad.numpy(), dwd=Wd.grad.numpy())


@pytest.mark.parametrize("T,d,E,k,f", [(12, 16, 4, 2, 8), (20, 8, 6, 3, 12)])
def test_backward_matches_torch_autograd(T, d, E, k, f):
    x, w_r, logits, wg, wu, wd, dy = problem(T * 7 + E, T, d, E, k, f)
    fwd, bwd, dx_total, dwr = oracle_full(x, w_r, logits, k, wg, wu, wd, dy)
    ref = torch_reference(x, w_r, k, wg, wu, wd, dy)
    tol = dict(rtol=1e-10, atol=1e-12)
    assert np.allclose(fwd["y"], ref["y"], **tol)
    assert np.allclose(bwd["d_logits"], ref["dl"], **tol)
    assert np.allclose(dx_total, ref["dx"], **tol)
    assert np.allclose(dwr, ref["dwr"], **tol)
    assert np.allclose(bwd["dw_gate"], ref["dwg"], **tol)
    assert np.allclose(bwd["dw_up"], ref["dwu"], **tol)
    assert np.allclose(bwd["dw_down"], ref["dwd"], **tol)


def test_central_finite_differences():
    T, d, E, k, f = 6, 8, 4, 2, 6
    x, w_r, logits, wg, wu, wd, dy = problem(99, T, d, E, k, f)
    _, bwd, _, _ = oracle_full(x, w_r, logits, k, wg, wu, wd, dy)
    dyf = codecs.bf16_to_f64(dy)
    idx0, _, _ = moe.route_topk(logits, k)

    def loss_from_logits(L):
        out = moe.layer_forward(x, L, k, wg, wu, wd)
        assert np.array_equal(out["topk_idx"], idx0)      # selection must stay fixed
        return np.sum(out["y"] * dyf)

    h = 1e-6
    for (t, e) in [(0, int(idx0[0, 0])), (3, int(idx0[3, 1])), (5, int(idx0[5, 0]))]:
        Lp = logits.copy(); Lp[t, e] += h
        Lm = logits.copy(); Lm[t, e] -= h
        fd = (loss_from_logits(Lp) - loss_from_logits(Lm)) / (2 * h)
        assert abs(fd - bwd["d_logits"][t, e]) < 1e-6 * max(1.0, abs(fd))

    # a weight entry, through float64 weights (the oracle accepts float arrays)
    wdf = codecs.bf16_to_f64(wd)
    e = int(idx0[0, 0])
    for (r, c) in [(0, 0), (3, 5)]:
        def loss_w(delta):
            w = wdf.copy(); w[e, r, c] += delta
            return np.sum(moe.layer_forward(x, logits, k, wg, wu, w)["y"] * dyf)
        fd = (loss_w(h) - loss_w(-h)) / (2 * h)
        assert abs(fd - bwd["dw_down"][e, r, c]) < 1e-6 * max(1.0, abs(fd))


def test_invariants():
    T, d, E, k, f = 30, 16, 6, 2, 8
    x, w_r, logits, wg, wu, wd, dy = problem(5, T, d, E, k, f, empty=(2,))
    fwd, bwd, _, _ = oracle_full(x, w_r, logits, k, wg, wu, wd, dy)
    dl = bwd["d_logits"]
    assert np.allclose(dl.sum(axis=1), 0.0, atol=1e-12)
    mask = np.zeros_like(dl, dtype=bool)
    np.put_along_axis(mask, fwd["topk_idx"].astype(np.int64), True, axis=1)
    assert np.all(dl[~mask] == 0.0)
    assert fwd["counts"][2] == 0
    for key in ("dw_gate", "dw_up", "dw_down"):
        assert np.all(bwd[key][2] == 0.0)
    # linearity in dy
    dy2 = to_bf16_bits((codecs.bf16_to_f64(dy) * 2).astype(np.float32))
    bwd2 = moe.layer_backward(fwd, dy2, wg, wu, wd)
    for key in ("dxp", "dw_gate", "dw_down", "d_logits", "dx"):
        assert np.allclose(bwd2[key], 2 * bwd[key], rtol=1e-12, atol=1e-14)
