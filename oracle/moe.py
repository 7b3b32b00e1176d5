"""The MoE layer's steps, forward and backward, as plain definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

One function per library entry point.  bf16 tensors are uint16 bit arrays; every
floating-point computation is done in float64 on exactly-decoded inputs, with no
blocking, fusion or reordering beyond what the definition states.

Shapes (row-major):  x [T, d] bf16, router weight w_r [d, E] fp32, logits [T, E] fp32,
expert weights w_gate, w_up [E, f, d] and w_down [E, d, f] bf16 (out-features first),
n = T * k routed rows, xp / yexp [n, d], G / U / A [n, f].
"""

import numpy as np

from .codecs import bf16_to_f64


# ------------------------------------------------------------------ router

def router_project(x_bf16, w_r):
    """logits = x @ w_r: the router's linear projection of each token.

    Follows "Ai2 rebuilds Olmo's training stack ..." lead paragraphs (a router scores
    the experts for each token).  float64 on exact inputs; the library accumulates in
    fp32, so parity on logits is a tolerance check.
    """
    return bf16_to_f64(x_bf16) @ np.asarray(w_r, dtype=np.float64)


def route_topk(logits, k):
    """Softmax over all experts, top-k, gates renormalised over the selected k.

    Selection is made on the logits (softmax is strictly increasing, so the top-k of
    the probabilities is the top-k of the logits) in descending order, ties going to
    the lower expert id; that order is also the slot order j.  The renormalised gate
    p_j / sum_{i<k} p_i equals the softmax over the selected logits alone, because the
    full softmax denominator cancels; it is computed here from the full softmax as
    defined, and the closed form is a separate pin in the tests.

    Returns (topk_idx [T,k] int32, topk_gate [T,k] float64, probs [T,E] float64).
    """
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("route_topk: need 1 <= k <= E")
    # Stable argsort of -logits: equal logits keep ascending expert order.
    order = np.argsort(-lg, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    z = lg - lg.max(axis=1, keepdims=True)
    p = np.exp(z)
    probs = p / p.sum(axis=1, keepdims=True)
    psel = np.take_along_axis(probs, idx.astype(np.int64), axis=1)
    gate = psel / psel.sum(axis=1, keepdims=True)
    return idx, gate, probs


def route_metadata(topk_idx, E, pad=32):
    """Device-resident routing metadata, defined as plain counting.

    ("Ai2 rebuilds Olmo's training stack ..." / "Routing work stays on the GPU": the
    metadata that places each routed row stays on the device.)

      counts[e]    number of (token, slot) pairs routed to expert e
      offsets      exclusive prefix sum of counts, length E+1 (offsets[E] = T*k)
      dest[t, j]   row of token t's j-th choice in the expert-major buffer: rows are
                   ordered by expert, and by token within an expert (a token cannot
                   pick one expert twice, so this order is total)
      row_token[r] the token whose row r is
      offsets_pad  like offsets, with each count rounded up to a multiple of `pad`

    Returns int32 arrays (counts [E], offsets [E+1], dest [T,k], row_token [n],
    offsets_pad [E+1]).
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    # Sort all (expert, token) pairs by the key expert * T + token; pair r is row r.
    keys = idx * T + np.arange(T)[:, None]
    order = np.argsort(keys.ravel(), kind="stable")
    dest = np.empty(T * k, dtype=np.int64)
    dest[order] = np.arange(T * k)
    row_token = order // k
    padded = (counts + pad - 1) // pad * pad
    offsets_pad = np.concatenate([[0], np.cumsum(padded)])
    return (counts.astype(np.int32), offsets.astype(np.int32), dest.reshape(T, k).astype(np.int32),
            row_token.astype(np.int32), offsets_pad.astype(np.int32))


# ------------------------------------------------------------------ permute / combine

def permute(x, dest):
    """Rowwise permute: xp[dest[t, j]] = x[t] for every slot j (a bit copy).

    ("Ai2 rebuilds ..." / "Routing work stays on the GPU": routed token rows are
    written straight into the experts' input buffers.)  Works on any row dtype.
    """
    x = np.asarray(x)
    dest = np.asarray(dest, dtype=np.int64)
    T, k = dest.shape
    xp = np.empty((T * k,) + x.shape[1:], dtype=x.dtype)
    for j in range(k):
        xp[dest[:, j]] = x
    return xp


def combine(yexp, gate, dest):
    """Weighted unpermute-combine: y[t] = sum_j gate[t, j] * yexp[dest[t, j]], in slot order.

    yexp may be bf16 bits (uint16) or float.  Returns float64 [T, d].
    """
    ye = _as_f64(yexp)
    g = np.asarray(gate, dtype=np.float64)
    dest = np.asarray(dest, dtype=np.int64)
    T, k = dest.shape
    y = np.zeros((T, ye.shape[1]))
    for j in range(k):
        y += g[:, j:j + 1] * ye[dest[:, j]]
    return y


# ------------------------------------------------------------------ expert FFN

def silu(z):
    return z / (1.0 + np.exp(-z))


def _segments(offsets):
    off = np.asarray(offsets, dtype=np.int64)
    return [(e, off[e], off[e + 1]) for e in range(off.shape[0] - 1) if off[e + 1] > off[e]]


def expert_gate_up(xp, offsets, w_gate, w_up):
    """First grouped product with the SwiGLU activation: for expert e's rows,
    G = X W_gate[e]^T,  U = X W_up[e]^T,  A = silu(G) * U.  Returns float64 (G, U, A)."""
    X = _as_f64(xp)
    f = w_gate.shape[1]
    G = np.zeros((X.shape[0], f)); U = np.zeros_like(G)
    for e, r0, r1 in _segments(offsets):
        G[r0:r1] = X[r0:r1] @ _as_f64(w_gate[e]).T
        U[r0:r1] = X[r0:r1] @ _as_f64(w_up[e]).T
    return G, U, silu(G) * U


def expert_down(a, offsets, w_down):
    """Second grouped product: Yexp = A W_down[e]^T for expert e's rows (float64)."""
    A = _as_f64(a)
    Y = np.zeros((A.shape[0], w_down.shape[1]))
    for e, r0, r1 in _segments(offsets):
        Y[r0:r1] = A[r0:r1] @ _as_f64(w_down[e]).T
    return Y


def expert_ffn(xp, offsets, w_gate, w_up, w_down):
    """SwiGLU expert FFN on each expert's contiguous rows.

    For expert e and rows r in [offsets[e], offsets[e+1]):
        G = X W_gate[e]^T,  U = X W_up[e]^T,  A = silu(G) * U,  Yexp = A W_down[e]^T
    ("Ai2 rebuilds ..." lead paragraphs: feed-forward expert networks; "Routing work
    stays on the GPU": the per-expert products are one grouped operation.)
    Returns float64 (G, U, A, Yexp).
    """
    G, U, A = expert_gate_up(xp, offsets, w_gate, w_up)
    return G, U, A, expert_down(A, offsets, w_down)


# ------------------------------------------------------------------ backward

def combine_bwd(dy, yexp, gate, dest):
    """Gradients of combine: dyexp[dest[t,j]] = gate[t,j] * dy[t];
    d_gate[t,j] = <dy[t], yexp[dest[t,j]]>.  Returns float64 (dyexp [n,d], d_gate [T,k])."""
    dyf = _as_f64(dy)
    ye = _as_f64(yexp)
    g = np.asarray(gate, dtype=np.float64)
    dest = np.asarray(dest, dtype=np.int64)
    T, k = dest.shape
    dyexp = np.zeros((T * k, dyf.shape[1]))
    dgate = np.zeros((T, k))
    for j in range(k):
        dyexp[dest[:, j]] = g[:, j:j + 1] * dyf
        dgate[:, j] = np.sum(dyf * ye[dest[:, j]], axis=1)
    return dyexp, dgate


def swiglu_bwd(dA, G, U):
    """A = silu(G) * U  =>  dG = dA * U * s * (1 + G (1 - s)),  dU = dA * G * s,  s = sigmoid(G)."""
    s = 1.0 / (1.0 + np.exp(-G))
    dG = dA * U * s * (1.0 + G * (1.0 - s))
    dU = dA * G * s
    return dG, dU


def expert_down_bwd(dyexp, a, offsets, w_down, E):
    """Backward of expert_down: dA = dYexp W_down[e]; dW_down[e] = dYexp_e^T A_e (zeros for
    experts with no rows).  Returns float64 (dA [n,f], dW_down [E,d,f])."""
    dY = _as_f64(dyexp); A = _as_f64(a)
    d, f = w_down.shape[1], w_down.shape[2]
    dA = np.zeros((dY.shape[0], f)); dW = np.zeros((E, d, f))
    for e, r0, r1 in _segments(offsets):
        dA[r0:r1] = dY[r0:r1] @ _as_f64(w_down[e])
        dW[e] = dY[r0:r1].T @ A[r0:r1]
    return dA, dW


def expert_gate_up_bwd(xp, dG, dU, offsets, w_gate, w_up, E):
    """Backward of the first product given dG, dU: dXp = dG W_gate[e] + dU W_up[e];
    dW_gate[e] = dG_e^T X_e, dW_up[e] = dU_e^T X_e (zeros for experts with no rows).
    Returns float64 (dXp [n,d], dW_gate [E,f,d], dW_up [E,f,d])."""
    X = _as_f64(xp); dGf = _as_f64(dG); dUf = _as_f64(dU)
    f, d = w_gate.shape[1], w_gate.shape[2]
    dX = np.zeros((dGf.shape[0], d)); dWg = np.zeros((E, f, d)); dWu = np.zeros((E, f, d))
    for e, r0, r1 in _segments(offsets):
        dX[r0:r1] = dGf[r0:r1] @ _as_f64(w_gate[e]) + dUf[r0:r1] @ _as_f64(w_up[e])
        dWg[e] = dGf[r0:r1].T @ X[r0:r1]
        dWu[e] = dUf[r0:r1].T @ X[r0:r1]
    return dX, dWg, dWu


def expert_ffn_bwd(xp, G, U, A, dyexp, offsets, w_gate, w_up, w_down):
    """Backward of expert_ffn for each expert's rows (top-k choices held constant).

        dA  = dYexp W_down[e]                   dW_down[e] = dYexp^T A
        dG, dU from swiglu_bwd(dA, G, U)
        dXp = dG W_gate[e] + dU W_up[e]         dW_gate[e] = dG^T X,  dW_up[e] = dU^T X
    Weight gradients of experts with no rows are exact zeros.
    Returns float64 dict with dA, dG, dU, dxp, dw_gate, dw_up, dw_down.
    """
    E = w_gate.shape[0]
    dA, dWd = expert_down_bwd(dyexp, A, offsets, w_down, E)
    dG, dU = swiglu_bwd(dA, _as_f64(G), _as_f64(U))
    dX, dWg, dWu = expert_gate_up_bwd(xp, dG, dU, offsets, w_gate, w_up, E)
    return dict(dA=dA, dG=dG, dU=dU, dxp=dX, dw_gate=dWg, dw_up=dWu, dw_down=dWd)


def permute_bwd(dxp, dest, addend=None):
    """dx[t] = sum_j dxp[dest[t, j]] (+ addend[t], the router-path term, if given)."""
    dX = _as_f64(dxp)
    dest = np.asarray(dest, dtype=np.int64)
    T, k = dest.shape
    dx = np.zeros((T, dX.shape[1])) if addend is None else np.array(addend, dtype=np.float64)
    for j in range(k):
        dx += dX[dest[:, j]]
    return dx


def route_topk_bwd(gate, topk_idx, d_gate, E):
    """Gradient of the renormalised gates w.r.t. the logits, selection held constant.

    The gates are a softmax over the selected logits, so
        d_logits[t, idx[t,j]] = g_j * (dg_j - sum_i g_i dg_i),  0 for unselected experts.
    """
    g = np.asarray(gate, dtype=np.float64)
    dg = np.asarray(d_gate, dtype=np.float64)
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    inner = np.sum(g * dg, axis=1, keepdims=True)
    dl = np.zeros((T, E))
    np.put_along_axis(dl, idx, g * (dg - inner), axis=1)
    return dl


def router_balance(probs, counts, k):
    """Load-balancing score of the router and balance statistics of the actual load.

    The pages name a routing-balance score and warn that it can improve while the real
    workload grows less balanced ("token gerrymandering"); they give no formula.  Reading:
    the usual auxiliary load-balancing loss of top-k routers, next to statistics of the
    counts themselves, so both views can be compared.
      f_e      = counts[e] / (T k)          share of routed (token, slot) pairs expert e gets
      P_e      = mean over tokens of probs[t, e]   (full softmax over all experts)
      aux      = E * sum_e f_e P_e          1 when f or P is uniform, E when both sit on one expert
      load_max = E * max_e f_e              largest expert load over the mean load
      prob_max = E * max_e P_e
      load_cv  = std_e(f) / mean_e(f)        (population standard deviation)
    Returns dict(aux, load_max, prob_max, load_cv, p_mean [E]) in float64.
    """
    pr = np.asarray(probs, dtype=np.float64)
    T, E = pr.shape
    f = np.asarray(counts, dtype=np.float64) / (T * k)
    P = pr.sum(axis=0) / T
    return dict(aux=E * float(np.sum(f * P)), load_max=E * float(f.max()), prob_max=E * float(P.max()),
                load_cv=float(f.std() / f.mean()), p_mean=P)


def router_balance_bwd(probs, counts, k, weight):
    """Gradient of weight * aux (router_balance) w.r.t. the logits, the counts held constant
    (they come from a discrete selection).  With c_e = weight * E * f_e / T = d(weight aux)/dp[t,e]
    and the softmax Jacobian dp[t,e]/dlogits[t,e'] = p[t,e] (delta_ee' - p[t,e']):
        d_logits[t, e'] = p[t, e'] * (c_e' - sum_e p[t, e] c_e)."""
    pr = np.asarray(probs, dtype=np.float64)
    T, E = pr.shape
    c = weight * E * (np.asarray(counts, dtype=np.float64) / (T * k)) / T
    return pr * (c[None, :] - (pr @ c)[:, None])


def router_project_bwd(x_bf16, w_r, d_logits):
    """Backward of logits = x @ w_r:  dx_router = d_logits @ w_r^T,  dw_r = x^T @ d_logits."""
    X = bf16_to_f64(x_bf16)
    W = np.asarray(w_r, dtype=np.float64)
    dl = np.asarray(d_logits, dtype=np.float64)
    return dl @ W.T, X.T @ dl


# ------------------------------------------------------------------ whole layer

def layer_forward(x, logits, k, w_gate, w_up, w_down):
    """Forward of the whole layer from logits: route, metadata, permute, FFN, combine."""
    E = w_gate.shape[0]
    idx, gate, probs = route_topk(logits, k)
    counts, offsets, dest, row_token, offsets_pad = route_metadata(idx, E)
    xp = permute(x, dest)
    G, U, A, Y = expert_ffn(xp, offsets, w_gate, w_up, w_down)
    y = combine(Y, gate, dest)
    return dict(topk_idx=idx, topk_gate=gate, probs=probs, counts=counts, offsets=offsets, dest=dest,
                row_token=row_token, offsets_pad=offsets_pad, xp=xp, G=G, U=U, A=A, yexp=Y, y=y)


def layer_backward(fwd, dy, w_gate, w_up, w_down):
    """Backward of the whole layer given the forward's saved tensors (float64 chain)."""
    E = w_gate.shape[0]
    dyexp, dgate = combine_bwd(dy, fwd["yexp"], fwd["topk_gate"], fwd["dest"])
    g = expert_ffn_bwd(fwd["xp"], fwd["G"], fwd["U"], fwd["A"], dyexp, fwd["offsets"], w_gate, w_up, w_down)
    dx = permute_bwd(g["dxp"], fwd["dest"])
    dl = route_topk_bwd(fwd["topk_gate"], fwd["topk_idx"], dgate, E)
    out = dict(dyexp=dyexp, d_gate=dgate, dx=dx, d_logits=dl)
    out.update(g)
    return out


def _as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)
