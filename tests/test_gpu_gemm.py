"""GPU parity: the grouped GEMMs of the SwiGLU expert FFN, forward and backward, bf16 and MXFP8.

Shapes span several 256 x 256 tiles with ragged row tails, partial column tiles, an expert that
receives no rows, one expert taking every token, and a single dense expert.  Each product is
checked on the same operands the GPU used (chained: the backward uses the GPU's own bf16 G, U,
A and dG, dU).  bf16 bar: 2e-2; MXFP8 bar: 1e-2 against the oracle on the GPU's dequantised
operands, whose quantised bytes are themselves checked bit for bit."""

import numpy as np
import pytest

from oracle import codecs, moe, mxfp8
from synth import to_bf16_bits
from tests.gpu_util import BF16_TOL, MX_TOL, assert_close, bf16_to_dev, bits, host, i32_to_dev, note

pytestmark = pytest.mark.gpu


def problem(T, d, E, k, f, seed, empty=(), hot=None, wstd=0.05, pad=128):
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    logits = rng.standard_normal((T, E))
    for e in empty:
        logits[:, e] -= 100.0
    if hot is not None:
        logits[:, hot] += 100.0
    idx, gate, _ = moe.route_topk(logits, k)
    counts, off, dest, row_token, offp = moe.route_metadata(idx, E, pad=pad)
    wg = to_bf16_bits((rng.standard_normal((E, f, d)) * wstd).astype(np.float32))
    wu = to_bf16_bits((rng.standard_normal((E, f, d)) * wstd).astype(np.float32))
    wd = to_bf16_bits((rng.standard_normal((E, d, f)) * wstd).astype(np.float32))
    dyexp = to_bf16_bits(rng.standard_normal((T * k, d)).astype(np.float32))
    return dict(x=x, counts=counts, off=off, dest=dest, row_token=row_token, offp=offp, wg=wg, wu=wu, wd=wd,
                xp=moe.permute(x, dest), dyexp=dyexp, E=E, n=T * k, T=T, d=d, f=f)


BF16_CASES = [
    dict(T=600, d=512, E=5, k=2, f=384, seed=1, empty=(2,)),
    dict(T=256, d=128, E=8, k=2, f=256, seed=2),
    dict(T=700, d=256, E=4, k=2, f=192, seed=3, hot=1),
    dict(T=300, d=320, E=1, k=1, f=448, seed=4),
    dict(T=1100, d=256, E=16, k=4, f=256, seed=5, empty=(0, 15)),
    # fewer rows than one 256-row tile
    dict(T=1, d=128, E=4, k=1, f=128, seed=6),
    dict(T=3, d=192, E=8, k=2, f=256, seed=7),
    # one expert far above twice the mean rows (every token picks expert 0): the weight
    # gradients deal their tiles round-robin in snake order
    dict(T=700, d=256, E=8, k=2, f=256, seed=8, hot=0),
    # expert 0 holds 4200 rows (17 m-tiles: the gate/up product takes its tiles n-fastest), the
    # others about 1400 (6 m-tiles: in cells), within one launch; the weight gradients stay in
    # contiguous runs (4200 is not above twice the mean)
    dict(T=4200, d=128, E=4, k=2, f=256, seed=9, hot=0),
    # every token picks expert 0 alone: seven experts without rows, whose weight gradients are
    # written as zeros outside the K-step stream, beside the dealt tiles of the hot expert
    dict(T=700, d=256, E=8, k=1, f=256, seed=10, hot=0),
    # 200 experts, top-1 of 300 tokens: empty experts in all four groups of 64
    dict(T=300, d=128, E=200, k=1, f=128, seed=11),
]


def case_id(c):
    return "-".join(f"{k}{v}" for k, v in c.items() if k != "seed")


@pytest.mark.parametrize("case", BF16_CASES, ids=case_id)
def test_grouped_gemm_bf16_forward_backward(case):
    from expert_ffn_layer_top_amd import ops
    p = problem(**case)
    E = p["E"]
    note(f"gg bf16 fwd {case}")
    off_d = i32_to_dev(p["off"])
    xp_d = bf16_to_dev(p["xp"])
    W = [bf16_to_dev(p[w]) for w in ("wg", "wu", "wd")]
    g, u, a, yexp = ops.grouped_gemm_swiglu(xp_d, off_d, *W)
    G, U, A = moe.expert_gate_up(p["xp"], p["off"], p["wg"], p["wu"])
    assert_close(codecs.bf16_to_f64(bits(g)), G, BF16_TOL, "G")
    assert_close(codecs.bf16_to_f64(bits(u)), U, BF16_TOL, "U")
    assert_close(codecs.bf16_to_f64(bits(a)), A, BF16_TOL, "A")
    assert_close(codecs.bf16_to_f64(bits(yexp)), moe.expert_down(bits(a), p["off"], p["wd"]), BF16_TOL, "Yexp (chained)")
    assert_close(codecs.bf16_to_f64(bits(yexp)), moe.expert_down(A, p["off"], p["wd"]), BF16_TOL, "Yexp")

    note(f"gg bf16 bwd {case}")
    out = ops.grouped_gemm_swiglu_bwd(xp_d, g, u, a, bf16_to_dev(p["dyexp"]), off_d, *W)
    dA, dWd = moe.expert_down_bwd(p["dyexp"], bits(a), p["off"], p["wd"], E)
    dG, dU = moe.swiglu_bwd(dA, codecs.bf16_to_f64(bits(g)), codecs.bf16_to_f64(bits(u)))
    assert_close(codecs.bf16_to_f64(bits(out["dg"])), dG, BF16_TOL, "dG")
    assert_close(codecs.bf16_to_f64(bits(out["du"])), dU, BF16_TOL, "dU")
    assert_close(codecs.bf16_to_f64(bits(out["dw_down"])), dWd, BF16_TOL, "dW_down")
    dX, dWg, dWu = moe.expert_gate_up_bwd(p["xp"], bits(out["dg"]), bits(out["du"]), p["off"], p["wg"], p["wu"], E)
    assert_close(codecs.bf16_to_f64(bits(out["dxp"])), dX, BF16_TOL, "dXp (chained)")
    assert_close(codecs.bf16_to_f64(bits(out["dw_gate"])), dWg, BF16_TOL, "dW_gate (chained)")
    assert_close(codecs.bf16_to_f64(bits(out["dw_up"])), dWu, BF16_TOL, "dW_up (chained)")
    for e in np.nonzero(p["counts"] == 0)[0]:
        for key in ("dw_gate", "dw_up", "dw_down"):
            assert np.all(bits(out[key])[e] == 0), f"{key}[{e}] of an empty expert is not zero"


def test_grouped_gemm_bf16_deterministic():
    from expert_ffn_layer_top_amd import ops
    p = problem(T=600, d=512, E=5, k=2, f=384, seed=9)
    note("gg bf16 determinism")
    args = (bf16_to_dev(p["xp"]), i32_to_dev(p["off"]), bf16_to_dev(p["wg"]), bf16_to_dev(p["wu"]), bf16_to_dev(p["wd"]))
    r1 = [bits(t) for t in ops.grouped_gemm_swiglu(*args)]
    r2 = [bits(t) for t in ops.grouped_gemm_swiglu(*args)]
    assert all(np.array_equal(a, b) for a, b in zip(r1, r2))


# ------------------------------------------------------------------ MXFP8

def deq_w(q, s):
    return mxfp8.dequantize_blocks(host(q), host(s))


def gemm_weights(ops, Wd):
    """The experts' weights quantised for the MX products along each dim: Q with row-major
    scales (mxfp8_quantize, for the oracle) and QG with the same scales in the GEMM scale layout
    (the products' operands); "_t" = quantised along the weight's rows (the dgrad direction)."""
    Q, QG = {}, {}
    for w in ("wg", "wu", "wd"):
        Q[w] = ops.mxfp8_quantize(Wd[w], 0)
        Q[w + "_t"] = ops.mxfp8_quantize(Wd[w], 1)
        R, C = Wd[w].shape[1], Wd[w].shape[2]
        QG[w] = (Q[w][0], ops.mxfp8_scales_to_gemm(Q[w][1], C))
        QG[w + "_t"] = (Q[w + "_t"][0], ops.mxfp8_scales_to_gemm(Q[w + "_t"][1], R))
    return Q, QG


MX_CASES = [
    # experts padded to 32 tokens on the weight gradients' token axis (the rest: 128)
    dict(T=600, d=512, E=5, k=2, f=384, seed=11, empty=(2,), pad=32),
    dict(T=300, d=256, E=4, k=2, f=256, seed=12, hot=0),
    dict(T=1000, d=384, E=9, k=3, f=128, seed=13, empty=(4,), pad=32),
    # contraction dims multiples of 512: the forward and dgrad products load scales in groups
    dict(T=700, d=1024, E=6, k=2, f=512, seed=14, empty=(3,)),
    # fewer rows than one tile; a single dense expert; top-1 routing
    dict(T=1, d=128, E=4, k=1, f=128, seed=15),
    dict(T=3, d=256, E=8, k=2, f=128, seed=16),
    dict(T=200, d=256, E=1, k=1, f=256, seed=17),
    dict(T=500, d=128, E=6, k=1, f=256, seed=18),
    # a hot expert far above twice the mean: round-robin (snake) deal of the weight gradients
    dict(T=600, d=256, E=8, k=2, f=256, seed=19, hot=0),
]


@pytest.mark.parametrize("case", MX_CASES, ids=case_id)
def test_grouped_gemm_mxfp8_forward_backward(case):
    from expert_ffn_layer_top_amd import ops
    p = problem(**case)
    E = p["E"]
    note(f"gg mxfp8 quantise {case}")
    x_d = bf16_to_dev(p["x"])
    xq, xs = ops.mxfp8_quantize(x_d, 0)
    rq, rs = mxfp8.quantize_rows(p["x"])
    assert np.array_equal(host(xq), rq) and np.array_equal(host(xs), rs)
    dest_d = i32_to_dev(p["dest"])
    xpq, xps = ops.permute(xq, dest_d, x_scale=xs)
    xps_g = ops.mxfp8_scales_to_gemm(xps, p["d"])             # the products read GEMM-layout scales
    Wd = {w: bf16_to_dev(p[w]) for w in ("wg", "wu", "wd")}
    Q, QG = gemm_weights(ops, Wd)
    for w in ("wg", "wu", "wd"):
        fq, fs = mxfp8.quantize_rows(p[w])
        assert np.array_equal(host(Q[w][0]), fq) and np.array_equal(host(Q[w][1]), fs)
        tq, ts = mxfp8.quantize_cols(p[w])
        assert np.array_equal(host(Q[w + "_t"][0]), tq) and np.array_equal(host(Q[w + "_t"][1]), ts)
    off_d = i32_to_dev(p["off"])

    note(f"gg mxfp8 fwd {case}")
    g, u, a, yexp = ops.grouped_gemm_swiglu(xpq, off_d, QG["wg"][0], QG["wu"][0], QG["wd"][0],
                                            scales=(xps_g, QG["wg"][1], QG["wu"][1], QG["wd"][1]))
    Xd = mxfp8.dequantize_blocks(host(xpq), host(xps))
    G, U, A = moe.expert_gate_up(Xd, p["off"], deq_w(*Q["wg"]), deq_w(*Q["wu"]))
    assert_close(codecs.bf16_to_f64(bits(g)), G, MX_TOL, "G (MX)")
    assert_close(codecs.bf16_to_f64(bits(u)), U, MX_TOL, "U (MX)")
    assert_close(codecs.bf16_to_f64(bits(a)), A, MX_TOL, "A (MX)")
    aq, as_ = mxfp8.quantize_rows(bits(a))                     # the GPU quantises its own bf16 A
    Y = moe.expert_down(mxfp8.dequantize_blocks(aq, as_), p["off"], deq_w(*Q["wd"]))
    assert_close(codecs.bf16_to_f64(bits(yexp)), Y, MX_TOL, "Yexp (MX, chained)")
    # the down product on A quantised by the one-read rows + grouped quantiser: the same bytes
    aq_d, as_d, _, _ = ops.mxfp8_quantize_rows_grouped(a, off_d, i32_to_dev(p["offp"]))
    y2 = ops.grouped_gemm_down_mx(aq_d, as_d, off_d, QG["wd"][0], QG["wd"][1])
    assert np.array_equal(bits(y2), bits(yexp)), "down on pre-quantised A differs from the composite"

    note(f"gg mxfp8 bwd {case}")
    offp_d = i32_to_dev(p["offp"])
    out = ops.grouped_gemm_swiglu_bwd(x_d, g, u, a, bf16_to_dev(p["dyexp"]), off_d, QG["wg_t"][0], QG["wu_t"][0],
                                      QG["wd_t"][0], scales=(QG["wg_t"][1], QG["wu_t"][1], QG["wd_t"][1]),
                                      offsets_pad=offp_d, row_token=i32_to_dev(p["row_token"]))
    dyq, dys = mxfp8.quantize_rows(p["dyexp"])
    dA = moe.expert_down(mxfp8.dequantize_blocks(dyq, dys), p["off"], deq_w(*Q["wd_t"]))
    dG, dU = moe.swiglu_bwd(dA, codecs.bf16_to_f64(bits(g)), codecs.bf16_to_f64(bits(u)))
    assert_close(codecs.bf16_to_f64(bits(out["dg"])), dG, MX_TOL, "dG (MX)")
    assert_close(codecs.bf16_to_f64(bits(out["du"])), dU, MX_TOL, "dU (MX)")
    dgq = mxfp8.dequantize_blocks(*mxfp8.quantize_rows(bits(out["dg"])))
    duq = mxfp8.dequantize_blocks(*mxfp8.quantize_rows(bits(out["du"])))
    dX = moe.expert_down(dgq, p["off"], deq_w(*Q["wg_t"])) + moe.expert_down(duq, p["off"], deq_w(*Q["wu_t"]))
    assert_close(codecs.bf16_to_f64(bits(out["dxp"])), dX, MX_TOL, "dXp (MX, chained)")
    # weight gradients: operands quantised along grouped tokens
    def grouped(t_bits, row_token=None):
        q, s = mxfp8.quantize_grouped(t_bits, p["off"], p["offp"], row_token=row_token)
        return mxfp8.dequantize_blocks(q, s)
    dyT, aT = grouped(p["dyexp"]), grouped(bits(a))
    dgT, duT = grouped(bits(out["dg"])), grouped(bits(out["du"]))
    xT = grouped(p["x"], row_token=p["row_token"])
    dWd = np.zeros((E, p["d"], p["f"])); dWg = np.zeros((E, p["f"], p["d"])); dWu = np.zeros_like(dWg)
    for e in range(E):
        a0, a1 = p["offp"][e], p["offp"][e + 1]
        dWd[e] = dyT[:, a0:a1] @ aT[:, a0:a1].T
        dWg[e] = dgT[:, a0:a1] @ xT[:, a0:a1].T
        dWu[e] = duT[:, a0:a1] @ xT[:, a0:a1].T
    assert_close(codecs.bf16_to_f64(bits(out["dw_down"])), dWd, MX_TOL, "dW_down (MX)")
    assert_close(codecs.bf16_to_f64(bits(out["dw_gate"])), dWg, MX_TOL, "dW_gate (MX)")
    assert_close(codecs.bf16_to_f64(bits(out["dw_up"])), dWu, MX_TOL, "dW_up (MX)")
    for e in np.nonzero(p["counts"] == 0)[0]:
        for key in ("dw_gate", "dw_up", "dw_down"):
            assert np.all(bits(out[key])[e] == 0)


# ------------------------------------------------ one kernel per call = the composite

@pytest.mark.parametrize("mx", [False, True], ids=["bf16", "mxfp8"])
def test_backward_per_kernel_calls_match_composite(mx):
    """The four backward products called one by one (on operands quantised by the standalone
    quantisers, for MXFP8) give the composite's bytes exactly."""
    from expert_ffn_layer_top_amd import ops
    p = problem(T=600, d=512, E=5, k=2, f=384, seed=21, empty=(3,))
    n = p["n"]
    note(f"gg per-kernel backward, mx={mx}")
    off_d = i32_to_dev(p["off"])
    dy_d = bf16_to_dev(p["dyexp"])
    Wd = {w: bf16_to_dev(p[w]) for w in ("wg", "wu", "wd")}
    if not mx:
        xp_d = bf16_to_dev(p["xp"])
        g, u, a, _ = ops.grouped_gemm_swiglu(xp_d, off_d, Wd["wg"], Wd["wu"], Wd["wd"])
        ref = ops.grouped_gemm_swiglu_bwd(xp_d, g, u, a, dy_d, off_d, Wd["wg"], Wd["wu"], Wd["wd"])
        dg, du = ops.grouped_gemm_dgrad_down(dy_d, off_d, Wd["wd"], g, u)
        dwd = ops.grouped_gemm_wgrad_down(dy_d, a, off_d, n)
        dxp = ops.grouped_gemm_dgrad_gate_up(dg, du, off_d, Wd["wg"], Wd["wu"])
        dwg, dwu = ops.grouped_gemm_wgrad_gate_up(dg, du, xp_d, off_d, n)
    else:
        x_d = bf16_to_dev(p["x"])
        xpq, xps = ops.permute_quant_mx(x_d, i32_to_dev(p["dest"]))
        _, Q = gemm_weights(ops, Wd)
        g, u, a, _ = ops.grouped_gemm_swiglu(xpq, off_d, Q["wg"][0], Q["wu"][0], Q["wd"][0],
                                             scales=(xps, Q["wg"][1], Q["wu"][1], Q["wd"][1]))
        offp_d = i32_to_dev(p["offp"])
        rt_d = i32_to_dev(p["row_token"])
        ref = ops.grouped_gemm_swiglu_bwd(x_d, g, u, a, dy_d, off_d, Q["wg_t"][0], Q["wu_t"][0], Q["wd_t"][0],
                                          scales=(Q["wg_t"][1], Q["wu_t"][1], Q["wd_t"][1]),
                                          offsets_pad=offp_d, row_token=rt_d)
        dyq, dys = ops.mxfp8_quantize_gemm(dy_d)
        dg, du = ops.grouped_gemm_dgrad_down(dyq, off_d, Q["wd_t"][0], g, u, scales=(dys, Q["wd_t"][1]))
        dyT, dyTs = ops.mxfp8_quantize_grouped(dy_d, off_d, offp_d, n)
        aT, aTs = ops.mxfp8_quantize_grouped(a, off_d, offp_d, n)
        dwd = ops.grouped_gemm_wgrad_down(dyT, aT, off_d, n, offsets_pad=offp_d, scales=(dyTs, aTs))
        dgq, dgs = ops.mxfp8_quantize_gemm(dg)
        duq, dus = ops.mxfp8_quantize_gemm(du)
        dxp = ops.grouped_gemm_dgrad_gate_up(dgq, duq, off_d, Q["wg_t"][0], Q["wu_t"][0],
                                             scales=(dgs, dus, Q["wg_t"][1], Q["wu_t"][1]))
        dgT, dgTs = ops.mxfp8_quantize_grouped(dg, off_d, offp_d, n)
        duT, duTs = ops.mxfp8_quantize_grouped(du, off_d, offp_d, n)
        xT, xTs = ops.mxfp8_quantize_grouped(x_d, off_d, offp_d, n, row_token=rt_d)
        dwg, dwu = ops.grouped_gemm_wgrad_gate_up(dgT, duT, xT, off_d, n, offsets_pad=offp_d,
                                                  scales=(dgTs, duTs, xTs))
    got = dict(dg=dg, du=du, dxp=dxp, dw_gate=dwg, dw_up=dwu, dw_down=dwd)
    for key, t in got.items():
        assert np.array_equal(bits(t), bits(ref[key])), f"{key}: per-kernel call differs from the composite"


# ------------------------------------------------ persistent launch: many tiles per workgroup

@pytest.mark.parametrize("case", [BF16_CASES[i] for i in (0, 2, 4, 7, 8, 9, 10)], ids=case_id)
def test_bf16_few_workgroups_bit_identical(case, monkeypatch):
    """With 8 workgroups each runs many tiles in a row (the next tile's first K steps stream in
    during the previous tile's epilogue); every output must match the default launch bit for bit,
    and the default launch matches the oracle (test above)."""
    from expert_ffn_layer_top_amd import ops
    p = problem(**case)
    n = p["n"]
    off_d = i32_to_dev(p["off"])
    xp_d = bf16_to_dev(p["xp"])
    dy_d = bf16_to_dev(p["dyexp"])
    W = [bf16_to_dev(p[w]) for w in ("wg", "wu", "wd")]

    def run():
        g, u, a, y = ops.grouped_gemm_swiglu(xp_d, off_d, *W)
        b = ops.grouped_gemm_swiglu_bwd(xp_d, g, u, a, dy_d, off_d, *W)
        return [bits(t) for t in (g, u, a, y, b["dg"], b["du"], b["dxp"], b["dw_gate"], b["dw_up"], b["dw_down"])]

    note(f"gg bf16 default launch {case}")
    ref = run()
    monkeypatch.setenv("MOE_GG_WORKGROUPS", "8")
    note(f"gg bf16 8 workgroups {case}")
    got = run()
    names = ("g", "u", "a", "yexp", "dg", "du", "dxp", "dw_gate", "dw_up", "dw_down")
    for nm, r, o in zip(names, ref, got):
        assert np.array_equal(r, o), f"{nm}: 8-workgroup launch differs from the default launch"


@pytest.mark.parametrize("case", MX_CASES, ids=case_id)
def test_mxfp8_few_workgroups_bit_identical(case, monkeypatch):
    """MXFP8 products with 8 workgroups (many tiles each, empty experts among them) give the
    default launch's bytes exactly."""
    from expert_ffn_layer_top_amd import ops
    p = problem(**case)
    x_d = bf16_to_dev(p["x"])
    xpq, xps = ops.permute_quant_mx(x_d, i32_to_dev(p["dest"]))
    Wd = {w: bf16_to_dev(p[w]) for w in ("wg", "wu", "wd")}
    _, Q = gemm_weights(ops, Wd)
    off_d = i32_to_dev(p["off"])
    offp_d = i32_to_dev(p["offp"])
    rt_d = i32_to_dev(p["row_token"])
    dy_d = bf16_to_dev(p["dyexp"])

    def run():
        g, u, a, y = ops.grouped_gemm_swiglu(xpq, off_d, Q["wg"][0], Q["wu"][0], Q["wd"][0],
                                             scales=(xps, Q["wg"][1], Q["wu"][1], Q["wd"][1]))
        b = ops.grouped_gemm_swiglu_bwd(x_d, g, u, a, dy_d, off_d, Q["wg_t"][0], Q["wu_t"][0], Q["wd_t"][0],
                                        scales=(Q["wg_t"][1], Q["wu_t"][1], Q["wd_t"][1]),
                                        offsets_pad=offp_d, row_token=rt_d)
        return [bits(t) for t in (g, u, a, y, b["dg"], b["du"], b["dxp"], b["dw_gate"], b["dw_up"], b["dw_down"])]

    note(f"gg mxfp8 default launch {case}")
    ref = run()
    monkeypatch.setenv("MOE_GG_WORKGROUPS", "8")
    note(f"gg mxfp8 8 workgroups {case}")
    got = run()
    names = ("g", "u", "a", "yexp", "dg", "du", "dxp", "dw_gate", "dw_up", "dw_down")
    for nm, r, o in zip(names, ref, got):
        assert np.array_equal(r, o), f"{nm}: 8-workgroup launch differs from the default launch"


@pytest.mark.parametrize("case", [MX_CASES[0], MX_CASES[2], MX_CASES[8]], ids=case_id)
def test_mxfp8_wgrad_pad_independent(case):
    """The MXFP8 weight gradients with each expert padded to 32, 64 and 128 tokens on the token
    axis: the 32-token scale blocks and the 128-token K steps start at the same rows of each
    expert every way, so every weight gradient is bit-identical."""
    from expert_ffn_layer_top_amd import ops
    p = problem(**{**case, "pad": 32})
    n = p["n"]
    off_d = i32_to_dev(p["off"])
    rt_d = i32_to_dev(p["row_token"])
    x_d = bf16_to_dev(p["x"])
    dy_d = bf16_to_dev(p["dyexp"])
    rng = np.random.default_rng(case["seed"] + 100)
    dg_d, du_d, a_d = (bf16_to_dev(to_bf16_bits(rng.standard_normal((n, p["f"])).astype(np.float32)))
                       for _ in range(3))
    outs = {}
    for pad in (32, 64, 128):
        offp_d = i32_to_dev(p["offp"] if pad == 32 else problem(**{**case, "pad": pad})["offp"])
        note(f"gg mxfp8 wgrad pad {pad} {case}")
        dyT, dyTs = ops.mxfp8_quantize_grouped(dy_d, off_d, offp_d, n)
        aT, aTs = ops.mxfp8_quantize_grouped(a_d, off_d, offp_d, n)
        dgT, dgTs = ops.mxfp8_quantize_grouped(dg_d, off_d, offp_d, n)
        duT, duTs = ops.mxfp8_quantize_grouped(du_d, off_d, offp_d, n)
        xT, xTs = ops.mxfp8_quantize_grouped(x_d, off_d, offp_d, n, row_token=rt_d)
        dwd = ops.grouped_gemm_wgrad_down(dyT, aT, off_d, n, offsets_pad=offp_d, scales=(dyTs, aTs))
        dwg, dwu = ops.grouped_gemm_wgrad_gate_up(dgT, duT, xT, off_d, n, offsets_pad=offp_d,
                                                  scales=(dgTs, duTs, xTs))
        outs[pad] = [bits(t) for t in (dwd, dwg, dwu)]
    for pad in (64, 128):
        for nm, r, o in zip(("dw_down", "dw_gate", "dw_up"), outs[32], outs[pad]):
            assert np.array_equal(r, o), f"{nm}: pad {pad} differs from pad 32"
