"""The MoE layer with MXFP8 expert products, as a plain chain of definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Ai2 rebuilds Olmo's training stack ..." / "MXFP8 reduces compute and memory costs": the expert
FFN's products run on 8-bit floats that carry one shared scale per small block.  Readings (the
pages name the format, not its use):
  * every operand of every expert product (forward, dgrad and wgrad) is E4M3 with one E8M0 scale
    per 32 elements along that product's contraction dimension, output gradients included; the
    router, permute, combine and their backward stay in bf16 / fp32;
  * a quantiser always reads a bf16 tensor: a value computed in higher precision (A, dYexp, dG,
    dU) is stored to bf16 first, the way an fp32 accumulator is stored (f64_to_bf16), and the
    tensors that cross between steps (G, U, Yexp, dXp) are stored to bf16 as well;
  * wgrad operands are quantised along tokens in blocks that restart at each expert's first row,
    every expert's rows zero-padded to a multiple of 32 (mxfp8.quantize_grouped);
  * each product is the plain product of the dequantised operands (mxfp8.mx_gemm_nt), float64.

Each function is the matching step of `moe` with its operands replaced by their MX values, in
the layer's order; no blocking or fusion beyond that.
"""

import numpy as np

from . import moe, mxfp8
from .codecs import bf16_to_f64, f64_to_bf16


def quantize_weights(w_gate, w_up, w_down):
    """MX copies of the expert weights along each product's contraction dimension.

    Forward products contract over d (gate, up) and f (down): row blocks of W_gate, W_up
    [E, f, d] and W_down [E, d, f].  Dgrad products contract over f (through W_gate, W_up) and
    d (through W_down): column blocks, transposed, [E, d, f] and [E, f, d].
    Returns {name: (q, scale)} for wg, wu, wd (forward) and wg_t, wu_t, wd_t (dgrad).
    """
    return dict(wg=mxfp8.quantize_rows(w_gate), wu=mxfp8.quantize_rows(w_up), wd=mxfp8.quantize_rows(w_down),
                wg_t=mxfp8.quantize_cols(w_gate), wu_t=mxfp8.quantize_cols(w_up),
                wd_t=mxfp8.quantize_cols(w_down))


def _expert(qw, name, e):
    q, s = qw[name]
    return q[e], s[e]


def expert_forward(xq, xs, qw, e):
    """Expert e's forward on its rows: xq, xs are the rows' E4M3 codes and scales (x quantised
    along d before the permute: row blocks commute with the row permutation).
        G = X W_gate^T, U = X W_up^T (stored bf16), A = bf16(silu(G) U) from the unrounded G, U,
        A quantised along f, Yexp = A W_down^T (stored bf16).
    Returns bf16 bits (G, U, A, Yexp)."""
    G = mxfp8.mx_gemm_nt(xq, xs, *_expert(qw, "wg", e))
    U = mxfp8.mx_gemm_nt(xq, xs, *_expert(qw, "wu", e))
    A = f64_to_bf16(moe.silu(G) * U)
    aq, as_ = mxfp8.quantize_rows(A)
    Y = mxfp8.mx_gemm_nt(aq, as_, *_expert(qw, "wd", e))
    return f64_to_bf16(G), f64_to_bf16(U), A, f64_to_bf16(Y)


def expert_backward(dyexp, G, U, A, x_rows, qw, e):
    """Expert e's backward on its rows (all arguments bf16 bits of the expert's rows, in row
    order; x_rows are the tokens' rows of x).
        dA = dYexp W_down (dYexp row blocks along d, W_down blocks along d),
        dG, dU = SwiGLU backward of (dA; stored G, U), stored bf16,
        dXp = dG W_gate + dU W_up (dG, dU row blocks along f), stored bf16,
        dW_down = dYexp^T A, dW_gate = dG^T X, dW_up = dU^T X over token-axis blocks of the
        expert's rows padded to 32.
    Returns dict of dG, dU, dxp (bf16 bits) and dw_gate, dw_up, dw_down (float64)."""
    R = dyexp.shape[0]
    dyq, dys = mxfp8.quantize_rows(dyexp)
    dA = mxfp8.mx_gemm_nt(dyq, dys, *_expert(qw, "wd_t", e))
    dG, dU = moe.swiglu_bwd(dA, bf16_to_f64(G), bf16_to_f64(U))
    dG, dU = f64_to_bf16(dG), f64_to_bf16(dU)
    dgq, dgs = mxfp8.quantize_rows(dG)
    duq, dus = mxfp8.quantize_rows(dU)
    dX = mxfp8.mx_gemm_nt(dgq, dgs, *_expert(qw, "wg_t", e)) + mxfp8.mx_gemm_nt(duq, dus, *_expert(qw, "wu_t", e))
    # weight gradients: one expert group of R rows, padded to a multiple of 32
    off = np.array([0, R])
    offp = np.array([0, (R + 31) // 32 * 32])
    dyT = mxfp8.quantize_grouped(dyexp, off, offp)
    aT = mxfp8.quantize_grouped(A, off, offp)
    dgT = mxfp8.quantize_grouped(dG, off, offp)
    duT = mxfp8.quantize_grouped(dU, off, offp)
    xT = mxfp8.quantize_grouped(x_rows, off, offp)
    return dict(dG=dG, dU=dU, dxp=f64_to_bf16(dX), dw_down=mxfp8.mx_gemm_nt(*dyT, *aT),
                dw_gate=mxfp8.mx_gemm_nt(*dgT, *xT), dw_up=mxfp8.mx_gemm_nt(*duT, *xT))


def layer_forward_mx(x, w_r, k, qw, logits=None):
    """Forward from x [T, d] bf16: router projection (unless logits are given), route and
    metadata, x quantised along d and permuted, each expert's MX products, combine (float64)."""
    E = qw["wg"][0].shape[0]
    if logits is None:
        logits = moe.router_project(x, w_r)
    idx, gate, probs = moe.route_topk(logits, k)
    counts, offsets, dest, row_token, offsets_pad = moe.route_metadata(idx, E)
    xq, xs = mxfp8.quantize_rows(x)
    xpq, xps = moe.permute(xq, dest), moe.permute(xs, dest)
    n, d = xpq.shape
    f = qw["wg"][0].shape[1]
    G = np.zeros((n, f), np.uint16); U = np.zeros_like(G); A = np.zeros_like(G)
    Y = np.zeros((n, d), np.uint16)
    for e, r0, r1 in moe._segments(offsets):
        G[r0:r1], U[r0:r1], A[r0:r1], Y[r0:r1] = expert_forward(xpq[r0:r1], xps[r0:r1], qw, e)
    y = moe.combine(Y, gate, dest)
    return dict(logits=logits, topk_idx=idx, topk_gate=gate, probs=probs, counts=counts, offsets=offsets,
                dest=dest, row_token=row_token, offsets_pad=offsets_pad, G=G, U=U, A=A, yexp=Y, y=y)


def layer_backward_mx(fwd, x, dy, w_r, qw):
    """Backward from dy [T, d] bf16: combine backward (dYexp = bf16(gate dy), stored as the
    quantiser's input), route backward, router backward (when w_r is given), each expert's MX
    backward products, permute backward with the router's dx term (float64)."""
    E = qw["wg"][0].shape[0]
    gate, dest, offsets, row_token = fwd["topk_gate"], fwd["dest"], fwd["offsets"], fwd["row_token"]
    T, k = dest.shape
    d = x.shape[1]
    f = qw["wg"][0].shape[1]
    dyf = bf16_to_f64(dy)
    dyexp = np.zeros((T * k, d), np.uint16)
    for j in range(k):
        dyexp[dest[:, j]] = f64_to_bf16(np.asarray(gate, np.float64)[:, j:j + 1] * dyf)
    _, d_gate = moe.combine_bwd(dy, fwd["yexp"], gate, dest)
    d_logits = moe.route_topk_bwd(gate, fwd["topk_idx"], d_gate, E)
    addend, dw_r = (None, None) if w_r is None else moe.router_project_bwd(x, w_r, d_logits)
    n = T * k
    dG = np.zeros((n, f), np.uint16); dU = np.zeros_like(dG); dXp = np.zeros((n, d), np.uint16)
    dWg = np.zeros((E, f, d)); dWu = np.zeros((E, f, d)); dWd = np.zeros((E, d, f))
    for e, r0, r1 in moe._segments(offsets):
        r = expert_backward(dyexp[r0:r1], fwd["G"][r0:r1], fwd["U"][r0:r1], fwd["A"][r0:r1],
                            x[np.asarray(row_token[r0:r1], np.int64)], qw, e)
        dG[r0:r1], dU[r0:r1], dXp[r0:r1] = r["dG"], r["dU"], r["dxp"]
        dWg[e], dWu[e], dWd[e] = r["dw_gate"], r["dw_up"], r["dw_down"]
    dx = moe.permute_bwd(dXp, dest, addend=addend)
    return dict(dyexp=dyexp, d_gate=d_gate, d_logits=d_logits, dx_router=addend, dw_r=dw_r, dG=dG, dU=dU,
                dxp=dXp, dx=dx, dw_gate=dWg, dw_up=dWu, dw_down=dWd)
