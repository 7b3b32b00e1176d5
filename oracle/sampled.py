"""Evaluators for checking full-size runs on samples (rows, experts).

TEST INFRASTRUCTURE ONLY (see the package docstring).

At full workload sizes the whole float64 oracle would take too long, so the parity
tests recompute chosen rows or chosen experts.  Each helper below is the definition
in `moe` restricted to those rows (most of them call `moe` on a sub-problem made of
just those rows), fed with the library's own stored inputs where a check is chained.
"""

import numpy as np

from . import moe


def _single_expert(rows):
    return np.array([0, rows], dtype=np.int64)


def ffn_forward_rows(xp_rows, experts, w_gate, w_up, w_down):
    """G, U, A, Yexp (float64) for selected rows; experts[i] is the expert of row i."""
    experts = np.asarray(experts, dtype=np.int64)
    m = len(experts)
    f, d = w_gate.shape[1], w_gate.shape[2]
    G = np.zeros((m, f)); U = np.zeros((m, f)); A = np.zeros((m, f)); Y = np.zeros((m, d))
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        g, u, a, y = moe.expert_ffn(xp_rows[sel], _single_expert(len(sel)),
                                    w_gate[e:e + 1], w_up[e:e + 1], w_down[e:e + 1])
        G[sel], U[sel], A[sel], Y[sel] = g, u, a, y
    return G, U, A, Y


def ffn_dgrad_rows(dyexp_rows, G_rows, U_rows, experts, w_gate, w_up, w_down):
    """dA, dG, dU and dXp (float64) for selected rows, from the given dYexp, G, U rows.

    dXp here is computed from the float64 dG, dU; the library computes it from its own
    stored (bf16) dG, dU, which `ffn_dxp_rows` reproduces for chained checks.
    """
    experts = np.asarray(experts, dtype=np.int64)
    m = len(experts)
    f, d = w_gate.shape[1], w_gate.shape[2]
    out = dict(dA=np.zeros((m, f)), dG=np.zeros((m, f)), dU=np.zeros((m, f)), dxp=np.zeros((m, d)))
    zeros_x = np.zeros((m, d), dtype=np.uint16)
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        r = moe.expert_ffn_bwd(zeros_x[sel], G_rows[sel], U_rows[sel], np.zeros((len(sel), f)),
                               dyexp_rows[sel], _single_expert(len(sel)),
                               w_gate[e:e + 1], w_up[e:e + 1], w_down[e:e + 1])
        for key in out:
            out[key][sel] = r[key]
    return out


def ffn_dxp_rows(dG_rows, dU_rows, experts, w_gate, w_up):
    """dXp = dG W_gate[e] + dU W_up[e] for selected rows (float64)."""
    experts = np.asarray(experts, dtype=np.int64)
    dG = moe._as_f64(dG_rows); dU = moe._as_f64(dU_rows)
    out = np.zeros((len(experts), w_gate.shape[2]))
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        out[sel] = dG[sel] @ moe._as_f64(w_gate[e]) + dU[sel] @ moe._as_f64(w_up[e])
    return out


def wgrad_expert(xp_e, A_e, dG_e, dU_e, dyexp_e):
    """Weight gradients of one expert from its rows: dW_gate = dG^T X, dW_up = dU^T X,
    dW_down = dYexp^T A (float64)."""
    X = moe._as_f64(xp_e); A = moe._as_f64(A_e); dG = moe._as_f64(dG_e)
    dU = moe._as_f64(dU_e); dY = moe._as_f64(dyexp_e)
    return dG.T @ X, dU.T @ X, dY.T @ A
