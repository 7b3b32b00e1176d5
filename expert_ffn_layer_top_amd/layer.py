"""One MoE layer step (forward + backward) on one GPU's share, composed from the C entry points.

Forward:  [router_project] -> route_topk -> permute -> grouped_gemm_swiglu -> unpermute_combine
Backward: unpermute_combine_bwd -> grouped_gemm_swiglu_bwd -> route_topk_bwd
          -> [router_project_bwd] -> permute_bwd (+ the router's dx term)
MXFP8 adds the block quantisation of x (before the permute; row blocks commute with the row
permutation) and of the expert weights in both contraction directions; router, combine,
permute-backward and route-backward stay bf16/fp32.

Every step is a library call on the current stream; this module only sequences them and holds
the tensors one step passes to the next.  ([news] "Ai2 rebuilds Olmo's training stack ...",
"Routing work stays on the GPU": the metadata never leaves the device, so the host enqueues
the whole step without waiting.)
"""

from dataclasses import dataclass, field

import torch

from . import ops


@dataclass
class Weights:
    w_gate: torch.Tensor                 # [E, f, d] bf16
    w_up: torch.Tensor                   # [E, f, d] bf16
    w_down: torch.Tensor                 # [E, d, f] bf16
    w_r: torch.Tensor = None             # [d, E] fp32, when the layer owns its router
    mx: dict = field(default_factory=dict)

    @property
    def E(self):
        return self.w_gate.shape[0]

    def quantize_mx(self):
        """MXFP8 copies of the expert weights, blocks along each product's contraction dim:
        forward (gate/up along d, down along f) and dgrad (gate/up along f, down along d)."""
        q = {}
        q["wg"], q["wg_s"] = ops.mxfp8_quantize(self.w_gate, 0)
        q["wu"], q["wu_s"] = ops.mxfp8_quantize(self.w_up, 0)
        q["wd"], q["wd_s"] = ops.mxfp8_quantize(self.w_down, 0)
        q["wg_t"], q["wg_t_s"] = ops.mxfp8_quantize(self.w_gate, 1)
        q["wu_t"], q["wu_t_s"] = ops.mxfp8_quantize(self.w_up, 1)
        q["wd_t"], q["wd_t_s"] = ops.mxfp8_quantize(self.w_down, 1)
        self.mx = q
        return q


def forward(x, weights, k, logits=None, mxfp8=False, want_probs=False, gate_up_events=None):
    """Layer forward.  x [T, d] bf16; logits [T, E] fp32 unless weights.w_r is given.
    Returns the context dict that `backward` consumes (all intermediate tensors), with y.
    gate_up_events: optional (start, end) torch.cuda.Event pair recorded on the current stream
    around the first grouped product (the benchmark times that kernel with them)."""
    ctx = dict(x=x, k=k, mxfp8=mxfp8)
    if logits is None:
        logits = ops.router_project(x, weights.w_r)
    ctx["logits"] = logits
    r = ops.route_topk(logits, k, want_probs=want_probs, pad=32 if mxfp8 else None)
    ctx.update(r)
    ev0, ev1 = gate_up_events if gate_up_events is not None else (None, None)
    if not mxfp8:
        xp = ops.permute(x, r["dest"])
        ctx["xp"] = xp
        if ev0 is not None:
            ev0.record()
        g, u, a = ops.grouped_gemm_gate_up(xp, r["offsets"], weights.w_gate, weights.w_up)
        if ev1 is not None:
            ev1.record()
        yexp = ops.grouped_gemm_down(a, r["offsets"], weights.w_down)
    else:
        q = weights.mx or weights.quantize_mx()
        xq, xs = ops.mxfp8_quantize(x, 0)
        xpq, xps = ops.permute(xq, r["dest"], x_scale=xs)
        ctx["xq"], ctx["xs"], ctx["xpq"], ctx["xps"] = xq, xs, xpq, xps
        if ev0 is not None:
            ev0.record()
        g, u, a = ops.grouped_gemm_gate_up(xpq, r["offsets"], q["wg"], q["wu"], scales=(xps, q["wg_s"], q["wu_s"]))
        if ev1 is not None:
            ev1.record()
        yexp = ops.grouped_gemm_down(a, r["offsets"], q["wd"], w_down_scale=q["wd_s"])
    ctx.update(g=g, u=u, a=a, yexp=yexp)
    ctx["y"] = ops.unpermute_combine(yexp, r["topk_gate"], r["dest"])
    return ctx


def backward(ctx, weights, dy):
    """Layer backward from dy [T, d] bf16.  Returns dict with dx, d_logits, dw_gate, dw_up,
    dw_down (and dw_r, dx_router when the layer owns its router) plus the intermediates."""
    out = {}
    dyexp, dgate = ops.unpermute_combine_bwd(dy, ctx["yexp"], ctx["topk_gate"], ctx["dest"])
    out.update(dyexp=dyexp, d_gate=dgate)
    if not ctx["mxfp8"]:
        gb = ops.grouped_gemm_swiglu_bwd(ctx["xp"], ctx["g"], ctx["u"], ctx["a"], dyexp, ctx["offsets"],
                                         weights.w_gate, weights.w_up, weights.w_down)
    else:
        q = weights.mx
        gb = ops.grouped_gemm_swiglu_bwd(ctx["x"], ctx["g"], ctx["u"], ctx["a"], dyexp, ctx["offsets"],
                                         q["wg_t"], q["wu_t"], q["wd_t"],
                                         scales=(q["wg_t_s"], q["wu_t_s"], q["wd_t_s"]),
                                         offsets_pad=ctx["offsets_pad"], row_token=ctx["row_token"])
    out.update(gb)
    E = ctx["logits"].shape[1]
    out["d_logits"] = ops.route_topk_bwd(ctx["topk_gate"], ctx["topk_idx"], dgate, E)
    addend = None
    if weights.w_r is not None:
        addend, out["dw_r"] = ops.router_project_bwd(ctx["x"], weights.w_r, out["d_logits"])
        out["dx_router"] = addend
    out["dx"] = ops.permute_bwd(gb["dxp"], ctx["dest"], addend=addend)
    return out
