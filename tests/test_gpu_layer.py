"""GPU parity of the whole layer step (forward + backward) through expert_ffn_layer_top_amd.layer.

  tiny      (256 tokens, d 128, 8 experts, top-2, d_ff 256, router weight): the float64 oracle
            runs the whole layer independently, router included.
  mxfp8     small MXFP8 layers (router weight, every expert product on E4M3 operands): the
            oracle's MXFP8 chain runs the whole layer from the GPU's logits, and the difference
            to the unquantised float64 layer is reported (not gated).
  balanced  (8192 tokens, d 2048, 64 experts, top-4, d_ff 1024, round-robin logits): the
            benchmarked workload, at full size, in the same launch configuration the benchmark
            times.  Integer outputs are checked in full; float outputs on sampled rows, tokens
            and experts the oracle recomputes one by one, each on the GPU's own inputs to that
            step (chained), plus independent per-token checks of y.
"""

import numpy as np
import pytest

import synth
from oracle import codecs, moe, moe_mx, sampled
from tests.gpu_util import BF16_TOL, assert_close, bits, host, note, rel_err

pytestmark = pytest.mark.gpu


def _run_layer(cfg, inputs):
    import torch
    from expert_ffn_layer_top_amd import layer
    t = synth.to_torch(inputs, torch.device("cuda:0"))
    w = layer.Weights(t["w_gate"], t["w_up"], t["w_down"], w_r=t.get("w_r"))
    ctx = layer.forward(t["x"], w, cfg.k, logits=t.get("logits"), mxfp8=cfg.mxfp8)
    out = layer.backward(ctx, w, t["dy"])
    torch.cuda.synchronize()
    return ctx, out


def test_tiny_layer_end_to_end_independent():
    cfg = synth.CONFIGS["tiny"]
    inputs = synth.make_inputs(cfg)
    note("layer tiny fwd+bwd")
    ctx, out = _run_layer(cfg, inputs)
    x, w_r, wg, wu, wd, dy = (inputs[k] for k in ("x", "w_r", "w_gate", "w_up", "w_down", "dy"))
    logits = moe.router_project(x, w_r)
    assert_close(host(ctx["logits"]), logits, 1e-5, "logits")
    # routing: bit-exact on the GPU's own fp32 logits, and equal to the independent routing
    # unless a k-th / (k+1)-th gap is below the fp32 noise of the logits
    idx_c, gate_c, _ = moe.route_topk(host(ctx["logits"]), cfg.k)
    assert np.array_equal(host(ctx["topk_idx"]), idx_c)
    srt = np.sort(logits, axis=1)[:, ::-1]
    gap = srt[:, cfg.k - 1] - srt[:, cfg.k]
    near = gap < 1e-5 * np.max(np.abs(logits))
    idx_i, _, _ = moe.route_topk(logits, cfg.k)
    assert np.array_equal(host(ctx["topk_idx"])[~near], idx_i[~near])
    assert not near.any(), "near-tie tokens: compare those in chained mode only"

    fwd = moe.layer_forward(x, logits, cfg.k, wg, wu, wd)
    assert np.array_equal(host(ctx["dest"]), fwd["dest"])
    assert_close(codecs.bf16_to_f64(bits(ctx["y"])), fwd["y"], BF16_TOL, "y")
    bwd = moe.layer_backward(fwd, dy, wg, wu, wd)
    add, dwr = moe.router_project_bwd(x, w_r, bwd["d_logits"])
    dx = moe.permute_bwd(bwd["dxp"], fwd["dest"], addend=add)
    assert_close(codecs.bf16_to_f64(bits(out["dx"])), dx, BF16_TOL, "dx")
    assert_close(host(out["d_logits"]), bwd["d_logits"], BF16_TOL, "d_logits")
    assert_close(host(out["dw_r"]), dwr, BF16_TOL, "dw_r")
    for key in ("dw_gate", "dw_up", "dw_down"):
        assert_close(codecs.bf16_to_f64(bits(out[key])), bwd[key], BF16_TOL, key)


def _check_mx_chain(cfg, inputs, ctx, out, what):
    """The GPU's MXFP8 layer against the oracle's MXFP8 chain run independently on the same
    inputs (routing from the GPU's own fp32 logits, which are checked against the oracle first):
    every float output within the bf16 bar.  Also prints the end-to-end difference to the
    unquantised float64 layer (MXFP8 rounding itself; reported, not gated)."""
    x, w_r, wg, wu, wd, dy = (inputs[k] for k in ("x", "w_r", "w_gate", "w_up", "w_down", "dy"))
    lg = host(ctx["logits"])
    assert_close(lg, moe.router_project(x, w_r), 1e-5, f"{what}: logits")
    qw = moe_mx.quantize_weights(wg, wu, wd)
    fwd = moe_mx.layer_forward_mx(x, w_r, cfg.k, qw, logits=lg)
    assert np.array_equal(host(ctx["dest"]), fwd["dest"])
    bwd = moe_mx.layer_backward_mx(fwd, x, dy, w_r, qw)
    got = dict(y=codecs.bf16_to_f64(bits(ctx["y"])), dx=codecs.bf16_to_f64(bits(out["dx"])),
               d_logits=host(out["d_logits"]), dw_r=host(out["dw_r"]),
               dw_gate=codecs.bf16_to_f64(bits(out["dw_gate"])), dw_up=codecs.bf16_to_f64(bits(out["dw_up"])),
               dw_down=codecs.bf16_to_f64(bits(out["dw_down"])))
    want = dict(y=fwd["y"], dx=bwd["dx"], d_logits=bwd["d_logits"], dw_r=bwd["dw_r"], dw_gate=bwd["dw_gate"],
                dw_up=bwd["dw_up"], dw_down=bwd["dw_down"])
    for key in got:
        assert_close(got[key], want[key], BF16_TOL, f"{what}: {key} (MXFP8 chain)")
    # end-to-end difference to the unquantised layer (same routing), reported only
    ref = moe.layer_forward(x, lg, cfg.k, wg, wu, wd)
    rb = moe.layer_backward(ref, dy, wg, wu, wd)
    add, dwr = moe.router_project_bwd(x, w_r, rb["d_logits"])
    unq = dict(y=ref["y"], dx=rb["dx"] + add, d_logits=rb["d_logits"], dw_r=dwr, dw_gate=rb["dw_gate"],
               dw_up=rb["dw_up"], dw_down=rb["dw_down"])
    report = ", ".join(f"{k} {rel_err(got[k], unq[k]):.3f}" for k in got)
    print(f"[MXFP8 vs unquantised float64 layer, max-rel-to-norm, not gated] {what}: {report}", flush=True)


MX_LAYER_SHAPES = [dict(T=640, d=512, E=6, k=2, f=512), dict(T=200, d=256, E=1, k=1, f=256),
                   dict(T=300, d=256, E=8, k=1, f=384)]


@pytest.mark.parametrize("shape", MX_LAYER_SHAPES, ids=lambda s: "-".join(f"{k}{v}" for k, v in s.items()))
def test_mxfp8_layer_against_oracle_chain(shape):
    cfg = synth.CONFIGS["mxfp8"].with_(**shape)
    inputs = synth.make_inputs(cfg)
    note(f"layer mxfp8 fwd+bwd {shape}")
    ctx, out = _run_layer(cfg, inputs)
    _check_mx_chain(cfg, inputs, ctx, out, f"mxfp8 {shape}")


def test_mxfp8_weights_requantised_after_in_place_update():
    """An in-place change of a bf16 expert weight between two steps reaches the MXFP8 products:
    the second step equals a step of fresh Weights built from the updated tensors."""
    import torch
    from expert_ffn_layer_top_amd import layer
    cfg = synth.CONFIGS["mxfp8"].with_(T=256, d=256, E=4, k=2, f=256)
    inputs = synth.make_inputs(cfg)
    t = synth.to_torch(inputs, torch.device("cuda:0"))
    w = layer.Weights(t["w_gate"], t["w_up"], t["w_down"], w_r=t["w_r"])
    note("layer mxfp8 weight update between steps")
    y0 = layer.forward(t["x"], w, cfg.k, mxfp8=True)["y"].clone()
    with torch.no_grad():
        w.w_gate.mul_(0.5)
        w.w_down.add_(0.01)
    ctx1 = layer.forward(t["x"], w, cfg.k, mxfp8=True)
    out1 = layer.backward(ctx1, w, t["dy"])
    fresh = layer.Weights(w.w_gate.clone(), w.w_up.clone(), w.w_down.clone(), w_r=t["w_r"])
    ctx2 = layer.forward(t["x"], fresh, cfg.k, mxfp8=True)
    out2 = layer.backward(ctx2, fresh, t["dy"])
    torch.cuda.synchronize()
    assert not torch.equal(ctx1["y"], y0)
    assert torch.equal(ctx1["y"], ctx2["y"])
    for key in ("dx", "dw_gate", "dw_up", "dw_down"):
        assert torch.equal(out1[key], out2[key]), key


@pytest.fixture(scope="module")
def balanced_run():
    cfg = synth.CONFIGS["balanced"]
    inputs = synth.make_inputs(cfg)
    note(f"layer balanced fwd+bwd T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f}")
    ctx, out = _run_layer(cfg, inputs)
    return cfg, inputs, ctx, out


def test_balanced_full_size_routing_and_permute(balanced_run):
    cfg, inputs, ctx, _ = balanced_run
    idx, gate, _ = moe.route_topk(inputs["logits"], cfg.k)
    counts, off, dest, row_token, _ = moe.route_metadata(idx, cfg.E)
    assert np.all(counts == 512)
    assert np.array_equal(host(ctx["topk_idx"]), idx) and np.array_equal(host(ctx["dest"]), dest)
    assert np.array_equal(host(ctx["offsets"]), off) and np.array_equal(host(ctx["row_token"]), row_token)
    assert np.max(np.abs(host(ctx["topk_gate"]) - gate)) < 1e-5
    assert np.array_equal(bits(ctx["xp"]), moe.permute(inputs["x"], dest))


def test_balanced_full_size_forward_samples(balanced_run):
    cfg, inputs, ctx, _ = balanced_run
    rng = np.random.default_rng(0)
    off = host(ctx["offsets"])
    rows = np.sort(rng.choice(cfg.n, size=96, replace=False))
    rows = np.concatenate([rows, [0, 511, 512, cfg.n - 1]])              # tile edges
    experts = np.searchsorted(off, rows, side="right") - 1
    xp = bits(ctx["xp"])
    W = (inputs["w_gate"], inputs["w_up"], inputs["w_down"])
    G, U, A, Y = sampled.ffn_forward_rows(xp[rows], experts, *W)
    assert_close(codecs.bf16_to_f64(bits(ctx["g"])[rows]), G, BF16_TOL, "G rows")
    assert_close(codecs.bf16_to_f64(bits(ctx["u"])[rows]), U, BF16_TOL, "U rows")
    assert_close(codecs.bf16_to_f64(bits(ctx["a"])[rows]), A, BF16_TOL, "A rows")
    assert_close(codecs.bf16_to_f64(bits(ctx["yexp"])[rows]), Y, BF16_TOL, "Yexp rows")
    # y for sampled tokens, independently: sum_j g_j FFN_{e_j}(x_t)
    toks = np.sort(rng.choice(cfg.T, size=24, replace=False))
    dest = host(ctx["dest"])
    gate = moe.route_topk(inputs["logits"][toks], cfg.k)[1]
    trow = dest[toks].ravel()
    texp = np.searchsorted(off, trow, side="right") - 1
    _, _, _, Yt = sampled.ffn_forward_rows(xp[trow], texp, *W)
    y_ref = np.einsum("tj,tjd->td", gate, Yt.reshape(len(toks), cfg.k, -1))
    assert_close(codecs.bf16_to_f64(bits(ctx["y"])[toks]), y_ref, BF16_TOL, "y tokens")


def test_balanced_full_size_backward_samples(balanced_run):
    cfg, inputs, ctx, out = balanced_run
    rng = np.random.default_rng(1)
    off = host(ctx["offsets"])
    dest = host(ctx["dest"])
    gate = host(ctx["topk_gate"])
    yexp = bits(ctx["yexp"])
    # combine backward: full tensors, on the GPU's own yexp and gates
    rdy, rdg = moe.combine_bwd(inputs["dy"], yexp, gate, dest)
    assert_close(codecs.bf16_to_f64(bits(out["dyexp"])), rdy, BF16_TOL, "dyexp")
    assert_close(host(out["d_gate"]), rdg, 1e-4, "d_gate")
    assert_close(host(out["d_logits"]), moe.route_topk_bwd(gate, host(ctx["topk_idx"]), host(out["d_gate"]), cfg.E),
                 1e-5, "d_logits")
    W = (inputs["w_gate"], inputs["w_up"], inputs["w_down"])
    rows = np.sort(rng.choice(cfg.n, size=96, replace=False))
    experts = np.searchsorted(off, rows, side="right") - 1
    dyexp = bits(out["dyexp"])
    r = sampled.ffn_dgrad_rows(dyexp[rows], codecs.bf16_to_f64(bits(ctx["g"])[rows]),
                               codecs.bf16_to_f64(bits(ctx["u"])[rows]), experts, *W)
    assert_close(codecs.bf16_to_f64(bits(out["dg"])[rows]), r["dG"], BF16_TOL, "dG rows")
    assert_close(codecs.bf16_to_f64(bits(out["du"])[rows]), r["dU"], BF16_TOL, "dU rows")
    dg, du = bits(out["dg"]), bits(out["du"])
    dxp_ref = sampled.ffn_dxp_rows(dg[rows], du[rows], experts, inputs["w_gate"], inputs["w_up"])
    assert_close(codecs.bf16_to_f64(bits(out["dxp"])[rows]), dxp_ref, BF16_TOL, "dXp rows")
    # weight gradients of sampled experts, on the GPU's own xp, A, dG, dU, dYexp
    xp, a = bits(ctx["xp"]), bits(ctx["a"])
    for e in (0, 37, cfg.E - 1):
        r0, r1 = off[e], off[e + 1]
        dwg, dwu, dwd = sampled.wgrad_expert(xp[r0:r1], a[r0:r1], dg[r0:r1], du[r0:r1], dyexp[r0:r1])
        assert_close(codecs.bf16_to_f64(bits(out["dw_gate"])[e]), dwg, BF16_TOL, f"dW_gate[{e}]")
        assert_close(codecs.bf16_to_f64(bits(out["dw_up"])[e]), dwu, BF16_TOL, f"dW_up[{e}]")
        assert_close(codecs.bf16_to_f64(bits(out["dw_down"])[e]), dwd, BF16_TOL, f"dW_down[{e}]")
    # dx for sampled tokens, on the GPU's own dXp
    toks = np.sort(rng.choice(cfg.T, size=64, replace=False))
    dxp = bits(out["dxp"])
    dx_ref = moe.permute_bwd(dxp, dest[toks])
    assert_close(codecs.bf16_to_f64(bits(out["dx"])[toks]), dx_ref, BF16_TOL, "dx tokens")


@pytest.mark.parametrize("mx", [False, True], ids=["bf16", "mxfp8"])
def test_activation_recompute_bit_identical(mx):
    """Per-layer activation recompute: the forward keeps no G, U, A and the backward runs the
    gate/up product again; every backward output equals the stored-activation run bit for bit."""
    import torch
    from expert_ffn_layer_top_amd import layer
    base = synth.CONFIGS["mxfp8" if mx else "tiny"]
    cfg = base.with_(T=640, d=512, E=6, k=2, f=512) if mx else base
    inputs = synth.make_inputs(cfg)
    t = synth.to_torch(inputs, torch.device("cuda:0"))
    w = layer.Weights(t["w_gate"], t["w_up"], t["w_down"], w_r=t.get("w_r"))
    outs = []
    for rc in (False, True):
        note(f"layer recompute={rc} mxfp8={mx} T={cfg.T} d={cfg.d} E={cfg.E} f={cfg.f}")
        ctx = layer.forward(t["x"], w, cfg.k, logits=t.get("logits"), mxfp8=mx, recompute=rc)
        assert (ctx["g"] is None) == rc and (ctx["a"] is None) == rc
        outs.append((ctx, layer.backward(ctx, w, t["dy"])))
    torch.cuda.synchronize()
    (c0, o0), (c1, o1) = outs
    assert torch.equal(c0["y"], c1["y"])
    for key in ("dx", "d_logits", "dw_gate", "dw_up", "dw_down", "dg", "du", "dxp"):
        assert torch.equal(o0[key], o1[key]), f"{key}: recompute run differs"
    if mx:
        # and the recompute run itself against the oracle's MXFP8 chain at this shape
        _check_mx_chain(cfg, inputs, c1, o1, "mxfp8 recompute")


def test_layer_balance_score_in_step():
    """balance_weight: the forward reports the balance score and load statistics, and the
    backward's d_logits carries the score's gradient on top of the route term."""
    import torch
    from expert_ffn_layer_top_amd import layer
    cfg = synth.CONFIGS["tiny"]
    inputs = synth.make_inputs(cfg)
    t = synth.to_torch(inputs, torch.device("cuda:0"))
    w = layer.Weights(t["w_gate"], t["w_up"], t["w_down"], w_r=t["w_r"])
    note("layer tiny with balance score")
    wb = 0.5
    ctx = layer.forward(t["x"], w, cfg.k, balance_weight=wb)
    out = layer.backward(ctx, w, t["dy"])
    torch.cuda.synchronize()
    probs, counts = host(ctx["probs"]), host(ctx["counts"])
    ref = moe.router_balance(probs, counts, cfg.k)
    stats = host(ctx["balance"]["stats"])
    assert abs(stats[0] - ref["aux"]) < 1e-5 * ref["aux"] and stats[1] == np.float32(ref["load_max"])
    d_ref = (moe.route_topk_bwd(host(ctx["topk_gate"]), host(ctx["topk_idx"]), host(out["d_gate"]), cfg.E)
             + moe.router_balance_bwd(probs, counts, cfg.k, wb))
    assert_close(host(out["d_logits"]), d_ref, 1e-5, "d_logits with balance term")


@pytest.mark.parametrize("mx", [False, True], ids=["bf16", "mxfp8"])
def test_step_captured_in_hip_graph(mx):
    """Nothing in the step waits on the host (routing metadata stays on the device), so the whole
    forward + backward can be captured in one HIP graph; three replays, with eager steps between
    them, each reproduce the eager results bit for bit."""
    import torch
    from expert_ffn_layer_top_amd import layer
    cfg = synth.CONFIGS["mxfp8" if mx else "balanced"].with_(T=1024, d=512, E=8, k=2, f=512)
    inputs = synth.make_inputs(cfg)
    t = synth.to_torch(inputs, torch.device("cuda:0"))
    w = layer.Weights(t["w_gate"], t["w_up"], t["w_down"], w_r=t.get("w_r"))
    keys = ("dx", "d_logits", "dw_gate", "dw_up", "dw_down")

    def step():
        if mx:
            w.quantize_mx()
        ctx = layer.forward(t["x"], w, cfg.k, logits=t.get("logits"), mxfp8=mx)
        return ctx, layer.backward(ctx, w, t["dy"])

    note(f"graph capture mxfp8={mx} T={cfg.T} d={cfg.d} E={cfg.E}")
    ctx, out = step()
    torch.cuda.synchronize()
    ref = {k: out[k].clone() for k in keys}
    ref["y"] = ctx["y"].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gctx, gout = step()
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gctx["y"], ref["y"]), f"replay {i}: y"
        for k in keys:
            assert torch.equal(gout[k], ref[k]), f"replay {i}: {k}"
        step()                                   # eager work between replays
        torch.cuda.synchronize()
