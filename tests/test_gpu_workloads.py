"""GPU parity of the whole layer step at the full sizes of the expert-count sweep (every E), the
skewed-routing workload and the MXFP8 workload, in the launch configuration the benchmark times
(expert_ffn_layer_top_amd.layer.forward / backward, default workgroup count).

Integer outputs (routing indices, destinations, offsets, row order, the permuted rows and the
MXFP8 bytes and scales that are checked) are compared bit for bit.  Float outputs are checked on
samples the float64 oracle recomputes one by one, each on the GPU's own inputs to that step
(chained): rows of every grouped product (random rows plus the first, last and tile-edge rows of
chosen experts), tokens of the combine and its backward, and output rows of the weight gradients
of the hottest, a median, the smallest non-empty and (where one exists) an empty expert.  bf16
bar 2e-2; MXFP8 bar 1e-2 against the oracle on the GPU's dequantised operands.
"""

import numpy as np
import pytest

import synth
from oracle import codecs, moe, mxfp8, sampled
from tests.gpu_util import BF16_TOL, MX_TOL, assert_close, bits, gemm_group, gemm_scales_to_rows, host, note, rel_err

pytestmark = pytest.mark.gpu


def _dev_rows(t, rows):
    """Rows of a device tensor, gathered on the device (only the sample crosses to the host)."""
    import torch
    return t[torch.as_tensor(np.asarray(rows, dtype=np.int64), device=t.device)]


def _gemm_scale_rows(t, rows, R, K):
    """Row-major scale rows [len(rows), K/32] of a device tensor holding R rows' scales in the GEMM
    scale layout (byte (r, b) at ((b / G) R + r) G + b % G), gathered on the device."""
    import torch
    G, nb = gemm_group(K), K // 32
    r = np.asarray(rows, dtype=np.int64)[:, None]
    b = np.arange(nb, dtype=np.int64)[None, :]
    idx = ((b // G) * R + r) * G + b % G
    flat = t.reshape(-1)
    return host(flat[torch.as_tensor(idx.ravel(), device=t.device)]).reshape(len(rows), nb)


def _rows_bits(t, rows):
    return bits(_dev_rows(t, rows))


def _f64(b):
    return codecs.bf16_to_f64(b)


def _run(cfg, inputs):
    import torch
    from expert_ffn_layer_top_amd import layer
    t = synth.to_torch(inputs, torch.device("cuda:0"))
    w = layer.Weights(t["w_gate"], t["w_up"], t["w_down"], w_r=t.get("w_r"))
    if cfg.mxfp8:
        w.quantize_mx()
    ctx = layer.forward(t["x"], w, cfg.k, logits=t.get("logits"), mxfp8=cfg.mxfp8)
    out = layer.backward(ctx, w, t["dy"])
    torch.cuda.synchronize()
    return w, ctx, out


def _chosen_experts(counts):
    """Hottest, median-loaded and smallest non-empty experts, plus an empty one if any."""
    nz = np.nonzero(counts > 0)[0]
    order = nz[np.argsort(counts[nz], kind="stable")]
    chosen = [int(order[-1]), int(order[len(order) // 2]), int(order[0])]
    empty = np.nonzero(counts == 0)[0]
    return list(dict.fromkeys(chosen)), (int(empty[0]) if empty.size else None)


def _sample_rows(off, experts, rng, n_random, pool=None):
    """Random rows (from `pool` experts if given) plus first / last / tile-edge rows of `experts`."""
    n = int(off[-1])
    if pool is None:
        rows = list(rng.choice(n, size=min(n_random, n), replace=False))
    else:
        cand = np.concatenate([np.arange(off[e], off[e + 1]) for e in pool])
        rows = list(rng.choice(cand, size=min(n_random, cand.size), replace=False))
    for e in experts:
        r0, r1 = int(off[e]), int(off[e + 1])
        for r in (r0, r1 - 1, r0 + 255, r0 + 256):
            if r0 <= r < r1:
                rows.append(r)
    rows = np.unique(np.asarray(rows, dtype=np.int64))
    return rows, np.searchsorted(off, rows, side="right") - 1


def _check_routing(cfg, logits, ctx):
    idx, gate, _ = moe.route_topk(logits, cfg.k)
    from expert_ffn_layer_top_amd import layer
    counts, off, dest, row_token, offp = moe.route_metadata(idx, cfg.E, pad=layer.MX_PAD)
    assert np.array_equal(host(ctx["topk_idx"]), idx)
    assert np.array_equal(host(ctx["counts"]), counts) and np.array_equal(host(ctx["offsets"]), off)
    assert np.array_equal(host(ctx["dest"]), dest) and np.array_equal(host(ctx["row_token"]), row_token)
    if cfg.mxfp8:
        assert np.array_equal(host(ctx["offsets_pad"]), offp)
    assert np.max(np.abs(host(ctx["topk_gate"]) - gate)) < 1e-5
    assert counts.sum() == cfg.T * cfg.k
    return counts, off, dest, row_token, offp


def _dyexp_rows(inputs, ctx, out, dest, rows):
    """bf16 bits of dYexp rows: the GPU's own, or under the fused MXFP8 combine backward (which
    never writes them) bf16(gate * dy) formed on the host from the GPU's gates, exactly as that
    kernel forms them (fp32 product, round to nearest even)."""
    if out["dyexp"] is not None:
        return _rows_bits(out["dyexp"], rows)
    T, k = dest.shape
    tok_of, slot_of = np.empty(T * k, np.int64), np.empty(T * k, np.int64)
    tok_of[dest.ravel()] = np.repeat(np.arange(T), k)
    slot_of[dest.ravel()] = np.tile(np.arange(k), T)
    rows = np.asarray(rows)
    tok, slot = tok_of[rows], slot_of[rows]
    g = host(ctx["topk_gate"])[tok, slot].astype(np.float32)
    dyf = codecs.bf16_to_f64(inputs["dy"][tok]).astype(np.float32)
    return synth.to_bf16_bits((dyf * g[:, None]).astype(np.float32))


def _check_combine_and_bwd(cfg, inputs, ctx, out, dest, toks):
    """y, dYexp and d_gate on sampled tokens (GPU's own Yexp and gates); d_logits in full."""
    k = cfg.k
    gate = host(ctx["topk_gate"])
    trow = dest[toks].ravel()
    ye = _rows_bits(ctx["yexp"], trow)
    local = np.arange(len(toks) * k).reshape(len(toks), k)
    assert_close(_f64(_rows_bits(ctx["y"], toks)), moe.combine(ye, gate[toks], local), BF16_TOL, "y tokens")
    rdy, rdg = moe.combine_bwd(inputs["dy"][toks], ye, gate[toks], local)
    assert_close(_f64(_dyexp_rows(inputs, ctx, out, dest, trow)), rdy, BF16_TOL, "dYexp tokens")
    assert_close(host(out["d_gate"])[toks], rdg, 1e-4, "d_gate tokens")
    assert_close(host(out["d_logits"]), moe.route_topk_bwd(gate, host(ctx["topk_idx"]), host(out["d_gate"]), cfg.E),
                 1e-5, "d_logits")


def _check_dx(cfg, out, dest, toks, addend=None):
    k = cfg.k
    dxp = _rows_bits(out["dxp"], dest[toks].ravel())
    local = np.arange(len(toks) * k).reshape(len(toks), k)
    assert_close(_f64(_rows_bits(out["dx"], toks)), moe.permute_bwd(dxp, local, addend=addend), BF16_TOL,
                 "dx tokens")


# ------------------------------------------------------------------ bf16 workloads

def _bf16_layer(cfg):
    rng = np.random.default_rng(100 + cfg.E)
    note(f"layer {cfg.name} inputs T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f}")
    inputs = synth.make_inputs(cfg)
    note(f"layer {cfg.name} fwd+bwd E={cfg.E}")
    w, ctx, out = _run(cfg, inputs)
    counts, off, dest, row_token, _ = _check_routing(cfg, inputs["logits"], ctx)
    # permute: bit-exact, every row
    assert np.array_equal(bits(ctx["xp"]), moe.permute(inputs["x"], dest))

    W = (inputs["w_gate"], inputs["w_up"], inputs["w_down"])
    chosen, empty = _chosen_experts(counts)
    rows, experts = _sample_rows(off, chosen, rng, 64)
    xp_r = _rows_bits(ctx["xp"], rows)
    G, U, A, Y = sampled.ffn_forward_rows(xp_r, experts, *W)
    g_r, u_r = _rows_bits(ctx["g"], rows), _rows_bits(ctx["u"], rows)
    assert_close(_f64(g_r), G, BF16_TOL, "G rows")
    assert_close(_f64(u_r), U, BF16_TOL, "U rows")
    assert_close(_f64(_rows_bits(ctx["a"], rows)), A, BF16_TOL, "A rows")
    assert_close(_f64(_rows_bits(ctx["yexp"], rows)), Y, BF16_TOL, "Yexp rows")

    toks = np.sort(rng.choice(cfg.T, size=32, replace=False))
    _check_combine_and_bwd(cfg, inputs, ctx, out, dest, toks)

    dy_r = _rows_bits(out["dyexp"], rows)
    r = sampled.ffn_dgrad_rows(dy_r, _f64(g_r), _f64(u_r), experts, *W)
    dg_r, du_r = _rows_bits(out["dg"], rows), _rows_bits(out["du"], rows)
    assert_close(_f64(dg_r), r["dG"], BF16_TOL, "dG rows")
    assert_close(_f64(du_r), r["dU"], BF16_TOL, "dU rows")
    assert_close(_f64(_rows_bits(out["dxp"], rows)),
                 sampled.ffn_dxp_rows(dg_r, du_r, experts, inputs["w_gate"], inputs["w_up"]), BF16_TOL, "dXp rows")

    # weight gradients: sampled output rows of chosen experts, on the GPU's own operands
    I = np.sort(rng.choice(cfg.f, size=12, replace=False))
    J = np.sort(rng.choice(cfg.d, size=12, replace=False))
    for e in chosen:
        er = np.arange(off[e], off[e + 1])
        dwg, dwu, dwd = sampled.wgrad_expert(_rows_bits(ctx["xp"], er), _rows_bits(ctx["a"], er),
                                             _rows_bits(out["dg"], er)[:, I], _rows_bits(out["du"], er)[:, I],
                                             _rows_bits(out["dyexp"], er)[:, J])
        assert_close(_f64(bits(out["dw_gate"][e])[I]), dwg, BF16_TOL, f"dW_gate[{e}] rows")
        assert_close(_f64(bits(out["dw_up"][e])[I]), dwu, BF16_TOL, f"dW_up[{e}] rows")
        assert_close(_f64(bits(out["dw_down"][e])[J]), dwd, BF16_TOL, f"dW_down[{e}] rows")
    if empty is not None:
        for key in ("dw_gate", "dw_up", "dw_down"):
            assert not bits(out[key][empty]).any(), f"{key}[{empty}] of an empty expert"
    _check_dx(cfg, out, dest, toks)
    return counts


@pytest.mark.parametrize("E", synth.SWEEP_E)
def test_sweep_full_size(E):
    cfg = synth.CONFIGS["sweep"].with_(E=E)
    counts = _bf16_layer(cfg)
    assert counts.min() > 0


def test_skewed_full_size():
    cfg = synth.CONFIGS["skewed"]
    counts = _bf16_layer(cfg)
    # the workload's shape: a few experts hold more than 10% of the rows, some hold none
    assert counts.max() > 0.1 * cfg.T * cfg.k and (counts == 0).any()


# ------------------------------------------------------------------ MXFP8 workload

def test_mxfp8_full_size():
    import torch
    cfg = synth.CONFIGS["mxfp8"]
    rng = np.random.default_rng(7)
    note(f"layer mxfp8 inputs T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f}")
    inputs = synth.make_inputs(cfg)
    note("layer mxfp8 fwd+bwd")
    w, ctx, out = _run(cfg, inputs)
    x, w_r, k = inputs["x"], inputs["w_r"], cfg.k

    # router projection on sampled tokens; routing bit-exact on the GPU's own logits
    toks = np.sort(rng.choice(cfg.T, size=32, replace=False))
    assert_close(host(_dev_rows(ctx["logits"], toks)), moe.router_project(x[toks], w_r), 1e-5, "logits tokens")
    counts, off, dest, row_token, offp = _check_routing(cfg, host(ctx["logits"]), ctx)

    # x quantised into the expert buffers (row blocks of the routed rows): bytes and scales bit for
    # bit on sampled rows
    chosen, _ = _chosen_experts(counts)
    rows, experts = _sample_rows(off, chosen, rng, 48, pool=chosen)
    n = cfg.T * cfg.k
    xpq_r, xps_r = host(_dev_rows(ctx["xpq"], rows)), _gemm_scale_rows(ctx["xps"], rows, n, cfg.d)
    rq, rs = mxfp8.quantize_rows(x[row_token[rows]])
    assert np.array_equal(xpq_r, rq) and np.array_equal(xps_r, rs)

    # the experts' quantised weights: bit for bit, then dequantised for the products
    q = w.mx
    deq = {}
    for e in chosen:
        for name, src, axis in (("wg", "w_gate", 0), ("wu", "w_up", 0), ("wd", "w_down", 0),
                                ("wg_t", "w_gate", 1), ("wu_t", "w_up", 1), ("wd_t", "w_down", 1)):
            bq = host(q[name][e])
            bs = gemm_scales_to_rows(host(q[name + "_s"][e]), bq.shape[0], bq.shape[1])   # GEMM layout
            ref = mxfp8.quantize_rows(inputs[src][e]) if axis == 0 else mxfp8.quantize_cols(inputs[src][e])
            assert np.array_equal(bq, ref[0]) and np.array_equal(bs, ref[1]), f"{name}[{e}]"
            deq[name, e] = mxfp8.dequantize_blocks(bq, bs)

    def per_expert(fn, m, width):
        res = np.zeros((len(rows), width))
        for e in np.unique(experts):
            sel = np.nonzero(experts == e)[0]
            res[sel] = fn(e, m[sel])
        return res

    # forward products on the GPU's dequantised operands
    X = mxfp8.dequantize_blocks(xpq_r, xps_r)
    G = per_expert(lambda e, m: m @ deq["wg", e].T, X, cfg.f)
    U = per_expert(lambda e, m: m @ deq["wu", e].T, X, cfg.f)
    g_r, u_r, a_r = _rows_bits(ctx["g"], rows), _rows_bits(ctx["u"], rows), _rows_bits(ctx["a"], rows)
    assert_close(_f64(g_r), G, MX_TOL, "G rows (MX)")
    assert_close(_f64(u_r), U, MX_TOL, "U rows (MX)")
    assert_close(_f64(a_r), moe.silu(G) * U, MX_TOL, "A rows (MX)")
    Aq = mxfp8.dequantize_blocks(*mxfp8.quantize_rows(a_r))           # the GPU quantises its bf16 A
    Y = per_expert(lambda e, m: m @ deq["wd", e].T, Aq, cfg.d)
    assert_close(_f64(_rows_bits(ctx["yexp"], rows)), Y, MX_TOL, "Yexp rows (MX, chained)")

    _check_combine_and_bwd(cfg, inputs, ctx, out, dest, toks)

    # dgrad products: operands quantised along the contraction dim, bit for bit, then the products
    mx = out["mx"]
    assert out["dyexp"] is None                                      # fused producer: no bf16 dYexp
    assert np.array_equal(host(out["row_gate"])[dest.ravel()], host(ctx["topk_gate"]).ravel())
    dy_r = _dyexp_rows(inputs, ctx, out, dest, rows)
    dyq_r, dys_r = mxfp8.quantize_rows(dy_r)
    assert np.array_equal(host(_dev_rows(mx["dyq"], rows)), dyq_r)
    assert np.array_equal(_gemm_scale_rows(mx["dys"], rows, n, cfg.d), dys_r)
    dA = per_expert(lambda e, m: m @ deq["wd_t", e].T, mxfp8.dequantize_blocks(dyq_r, dys_r), cfg.f)
    dG, dU = moe.swiglu_bwd(dA, _f64(g_r), _f64(u_r))
    dg_r, du_r = _rows_bits(out["dg"], rows), _rows_bits(out["du"], rows)
    assert_close(_f64(dg_r), dG, MX_TOL, "dG rows (MX)")
    assert_close(_f64(du_r), dU, MX_TOL, "dU rows (MX)")
    dgq, dgs = mxfp8.quantize_rows(dg_r)
    duq, dus = mxfp8.quantize_rows(du_r)
    assert np.array_equal(host(_dev_rows(mx["dgq"], rows)), dgq) and np.array_equal(host(_dev_rows(mx["duq"], rows)), duq)
    assert np.array_equal(_gemm_scale_rows(mx["dgs"], rows, n, cfg.f), dgs)
    assert np.array_equal(_gemm_scale_rows(mx["dus"], rows, n, cfg.f), dus)
    dX = (per_expert(lambda e, m: m @ deq["wg_t", e].T, mxfp8.dequantize_blocks(dgq, dgs), cfg.d)
          + per_expert(lambda e, m: m @ deq["wu_t", e].T, mxfp8.dequantize_blocks(duq, dus), cfg.d))
    assert_close(_f64(_rows_bits(out["dxp"], rows)), dX, MX_TOL, "dXp rows (MX, chained)")

    # weight gradients: grouped token blocks of chosen experts bit for bit, then sampled output rows
    I = np.sort(rng.choice(cfg.f, size=8, replace=False))
    J = np.sort(rng.choice(cfg.d, size=8, replace=False))
    for e in chosen:
        r0, r1, p0 = int(off[e]), int(off[e + 1]), int(offp[e])
        cnt = r1 - r0
        span = int(offp[e + 1]) - p0
        one_off, one_pad = np.array([0, cnt]), np.array([0, span])
        er = np.arange(r0, r1)

        def grouped(dev_q, dev_s, src_rows_bits, C, name):
            gq = host(dev_q[:, p0:p0 + span])
            gs = host(dev_s[p0 // 32:(p0 + span) // 32, :]).T   # scales are block-major
            rq_, rs_ = mxfp8.quantize_grouped(src_rows_bits, one_off, one_pad)
            assert gq.shape == (C, span) and np.array_equal(gq, rq_) and np.array_equal(gs, rs_), f"{name}[{e}]"
            return mxfp8.dequantize_blocks(gq, gs)

        dyT = grouped(mx["dyT"], mx["dyTs"], _dyexp_rows(inputs, ctx, out, dest, er), cfg.d, "dyexp^T")
        aT = grouped(mx["aT"], mx["aTs"], _rows_bits(ctx["a"], er), cfg.f, "a^T")
        dgT = grouped(mx["dgT"], mx["dgTs"], _rows_bits(out["dg"], er), cfg.f, "dg^T")
        duT = grouped(mx["duT"], mx["duTs"], _rows_bits(out["du"], er), cfg.f, "du^T")
        xT = grouped(mx["xT"], mx["xTs"], x[row_token[er]], cfg.d, "x^T")
        assert_close(_f64(bits(out["dw_gate"][e])[I]), dgT[I] @ xT.T, MX_TOL, f"dW_gate[{e}] rows (MX)")
        assert_close(_f64(bits(out["dw_up"][e])[I]), duT[I] @ xT.T, MX_TOL, f"dW_up[{e}] rows (MX)")
        assert_close(_f64(bits(out["dw_down"][e])[J]), dyT[J] @ aT.T, MX_TOL, f"dW_down[{e}] rows (MX)")

    # router backward: dW_r in full; dx (the permuted rows' sum plus the router's dx term, one
    # kernel) on sampled tokens against the oracle's float64 router term
    dl = host(out["d_logits"])
    add, dwr = moe.router_project_bwd(x, w_r, dl)
    assert_close(host(out["dw_r"]), dwr, BF16_TOL, "dW_r")
    _check_dx(cfg, out, dest, toks, addend=add[toks])

    # end-to-end difference of y to the unquantised float64 layer on the sampled tokens (the
    # GPU's routing, bf16 weights, no MXFP8 anywhere): the MXFP8 rounding itself, reported only
    idx, gt = host(ctx["topk_idx"])[toks], host(ctx["topk_gate"])[toks]
    _, _, _, Yu = sampled.ffn_forward_rows(np.repeat(x[toks], k, axis=0), idx.ravel(),
                                           inputs["w_gate"], inputs["w_up"], inputs["w_down"])
    yu = np.einsum("tk,tkd->td", gt, Yu.reshape(len(toks), k, cfg.d))
    e = rel_err(_f64(_rows_bits(ctx["y"], toks)), yu)
    e2 = float(np.linalg.norm(_f64(_rows_bits(ctx["y"], toks)) - yu) / np.linalg.norm(yu))
    print(f"[MXFP8 vs unquantised float64 layer, not gated] y on {len(toks)} sampled tokens: "
          f"max-rel-to-norm {e:.4f}, relative L2 {e2:.4f}", flush=True)
    del torch
