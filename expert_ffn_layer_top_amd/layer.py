"""One MoE layer step (forward + backward) on one GPU's share, composed from the C entry points.

Forward:  [router_project] -> route_topk -> permute -> grouped_gemm_gate_up -> grouped_gemm_down
          -> unpermute_combine
Backward: unpermute_combine_bwd -> route_topk_bwd -> [router_project_bwd: dw_r]
          -> grouped_gemm_dgrad_down -> grouped_gemm_wgrad_down -> grouped_gemm_dgrad_gate_up
          -> permute_bwd (permute_bwd_router: with the router's dx term, computed in the same
          kernel) -> grouped_gemm_wgrad_gate_up
The grouped products are issued one kernel per call (the same kernels, in the same order, as the
composite grouped_gemm_swiglu / grouped_gemm_swiglu_bwd), so each can be timed on its own.
MXFP8 adds the block quantisation of x (inside the permute, which writes the row blocks straight
into the expert buffers; row blocks commute with the row permutation) and of the expert weights
in both contraction directions; router, combine,
permute-backward and route-backward stay bf16/fp32.  Its combine backward is the fused producer
(unpermute_combine_bwd_mx): dYexp leaves as MXFP8 row blocks and per-row gates, and the grouped
token blocks of dYexp are rebuilt from dy and those gates, so the bf16 dYexp is never written.

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
    mx_key: tuple = None                 # the bf16 weights the MXFP8 copies were made from

    @property
    def E(self):
        return self.w_gate.shape[0]

    def _key(self):
        # storage and in-place version of each bf16 weight: an optimizer step that updates a
        # weight in place bumps its version, a new tensor changes its storage
        return tuple((t.data_ptr(), t._version) for t in (self.w_gate, self.w_up, self.w_down))

    def quantize_mx(self):
        """MXFP8 copies of the expert weights, blocks along each product's contraction dim:
        forward (gate/up along d, down along f) and dgrad (gate/up along f, down along d), both
        from one read of each weight."""
        q = {}
        for name, w in (("wg", self.w_gate), ("wu", self.w_up), ("wd", self.w_down)):
            q[name], q[name + "_s"], q[name + "_t"], q[name + "_t_s"] = ops.mxfp8_quantize_both(w)
        self.mx = q
        self.mx_key = self._key()
        return q

    def mx_current(self):
        """The MXFP8 copies of the weights as they are now: quantised again whenever a bf16 weight
        was replaced or modified in place since the copies were made."""
        if not self.mx or self.mx_key != self._key():
            return self.quantize_mx()
        return self.mx


class _Span:
    """Records an optional (start, end) torch.cuda.Event pair on the current stream around one
    library call: events[name] if the caller asked for that name."""

    def __init__(self, events, name):
        self.pair = events.get(name) if events else None

    def __enter__(self):
        if self.pair is not None:
            self.pair[0].record()

    def __exit__(self, *exc):
        if self.pair is not None:
            self.pair[1].record()
        return False


# names of the calls `forward` and `backward` can bracket with events: each grouped-GEMM call is
# one kernel ("recompute" is the gate/up product again, in the backward of a forward run with
# recompute=True); ROW_CALLS are the routing and row-movement calls (route: its three kernels)
GEMM_CALLS = ("gate_up", "down", "dgrad_down", "wgrad_down", "dgrad_gate_up", "wgrad_gate_up")
RECOMPUTE_CALL = "recompute"
# the router products (layers that own their router) and the MXFP8 quantiser calls of the forward
# and the backward (each one kernel; "quant_a" gives A's row blocks and grouped token blocks from
# one read, "quant_dyT" gathers dy with the combine backward's row gates)
ROUTER_CALLS = ("router", "router_bwd")
QUANT_CALLS_FWD = ("quant_a",)
QUANT_CALLS = ("quant_dg", "quant_du", "quant_dyT", "quant_xT")
ROW_CALLS = ("route", "permute", "combine", "combine_bwd", "permute_bwd", "route_bwd")
# MXFP8: each expert's rows start at a multiple of MX_PAD on the padded token axis of the
# weight-gradient operands.  128 = one K step of those products: every step's 128-byte piece of an
# operand row is then one whole cache line (with 32, each straddles two: both weight gradients
# ran about 20% slower at T 32768, d 7168, 64 experts)
MX_PAD = 128


def forward(x, weights, k, logits=None, mxfp8=False, want_probs=False, events=None, recompute=False,
            balance_weight=None):
    """Layer forward.  x [T, d] bf16; logits [T, E] fp32 unless weights.w_r is given.
    Returns the context dict that `backward` consumes (all intermediate tensors), with y.
    events: optional {name: (start, end)} of torch.cuda.Event pairs, recorded on the current
    stream around the calls named in GEMM_CALLS and ROW_CALLS.
    recompute: keep neither G, U nor A (3 n f bf16 values) for the backward, which then runs the
    gate/up product again on the kept permuted input (per-layer activation recompute, [card]
    "Supercharging Olmo-core ...": used at the largest scale).  The kernels are deterministic,
    so the backward's results are bit-identical either way.
    mxfp8: the expert products run on MXFP8 operands; the weights' MXFP8 copies are made on the
    first such forward and again whenever a bf16 weight was replaced or changed in place
    (Weights.mx_current), so an optimizer step between two forwards is always seen.
    balance_weight: also compute the router's load-balancing score and the balance statistics of
    the actual load (ctx["balance"]: p_mean [E], stats [aux, load_max, prob_max, load_cv]), and
    add the gradient of balance_weight * aux to d_logits in the backward."""
    ctx = dict(x=x, k=k, mxfp8=mxfp8, balance_weight=balance_weight)
    want_probs = want_probs or balance_weight is not None
    if logits is None:
        with _Span(events, "router"):
            logits = ops.router_project(x, weights.w_r)
    ctx["logits"] = logits
    with _Span(events, "route"):
        r = ops.route_topk(logits, k, want_probs=want_probs, pad=MX_PAD if mxfp8 else None)
    ctx.update(r)
    if balance_weight is not None:
        p_mean, stats = ops.route_balance(r["probs"], r["counts"], k)
        ctx["balance"] = dict(p_mean=p_mean, stats=stats)
    if not mxfp8:
        with _Span(events, "permute"):
            xp = ops.permute(x, r["dest"])
        ctx["xp"] = xp
        with _Span(events, "gate_up"):
            g, u, a = ops.grouped_gemm_gate_up(xp, r["offsets"], weights.w_gate, weights.w_up)
        with _Span(events, "down"):
            yexp = ops.grouped_gemm_down(a, r["offsets"], weights.w_down)
    else:
        q = weights.mx_current()
        # x quantised along d on its way into the expert buffers (no token-major E4M3 copy)
        with _Span(events, "permute"):
            xpq, xps = ops.permute_quant_mx(x, r["dest"])
        ctx["xpq"], ctx["xps"] = xpq, xps
        ctx["mx_weights"] = q            # the backward uses the copies this forward used
        with _Span(events, "gate_up"):
            g, u, a = ops.grouped_gemm_gate_up(xpq, r["offsets"], q["wg"], q["wu"],
                                               scales=(xps, q["wg_s"], q["wu_s"]))
        # A read once for both its MXFP8 layouts: row blocks for the down product now, grouped
        # token blocks for the down weight gradient (kept for the backward, recompute or not)
        with _Span(events, "quant_a"):
            aq, as_, aT, aTs = ops.mxfp8_quantize_rows_grouped(a, r["offsets"], r["offsets_pad"])
        ctx["aT"], ctx["aTs"] = aT, aTs
        with _Span(events, "down"):
            yexp = ops.grouped_gemm_down_mx(aq, as_, r["offsets"], q["wd"], q["wd_s"])
    if recompute:
        del g, u, a
        ctx.update(g=None, u=None, a=None, yexp=yexp)
    else:
        ctx.update(g=g, u=u, a=a, yexp=yexp)
    with _Span(events, "combine"):
        ctx["y"] = ops.unpermute_combine(yexp, r["topk_gate"], r["dest"])
    return ctx


def backward(ctx, weights, dy, events=None):
    """Layer backward from dy [T, d] bf16.  Returns dict with dx, d_logits, dw_gate, dw_up,
    dw_down (and dw_r when the layer owns its router) plus the intermediates (under
    MXFP8, "mx" holds the quantised backward operands: row blocks dyq/dgq/duq, grouped token
    blocks dyT/aT/dgT/duT/xT, each with its scales).
    events: as for `forward`.

    Each call follows the call that produced its input where the dependencies allow (the router
    gradients right after the combine backward, the permute backward right after the product
    that writes dXp), so its input is still in the last-level cache; the arithmetic does not
    depend on the order."""
    out = {}
    with _Span(events, "combine_bwd"):
        if not ctx["mxfp8"]:
            dyexp, dgate = ops.unpermute_combine_bwd(dy, ctx["yexp"], ctx["topk_gate"], ctx["dest"])
        else:
            # fused MXFP8 producer: dYexp leaves as row blocks only (bf16 rows never written)
            dyexp = None
            dyq, dys, row_gate, dgate = ops.unpermute_combine_bwd_mx(dy, ctx["yexp"], ctx["topk_gate"], ctx["dest"])
    out.update(dyexp=dyexp, d_gate=dgate)
    E = ctx["logits"].shape[1]
    with _Span(events, "route_bwd"):
        bal = None
        if ctx.get("balance_weight") is not None:
            bal = (ctx["probs"], ctx["counts"], ctx["balance_weight"])
        out["d_logits"] = ops.route_topk_bwd(ctx["topk_gate"], ctx["topk_idx"], dgate, E, balance=bal)
    if weights.w_r is not None:
        with _Span(events, "router_bwd"):
            _, out["dw_r"] = ops.router_project_bwd(ctx["x"], weights.w_r, out["d_logits"], want_dx=False)

    def permute_bwd(dxp):
        # the router's dx term, when the layer owns its router, joins the permuted rows' sum
        if weights.w_r is None:
            return ops.permute_bwd(dxp, ctx["dest"])
        return ops.permute_bwd_router(dxp, ctx["dest"], weights.w_r, out["d_logits"])
    off = ctx["offsets"]
    g, u, a = ctx["g"], ctx["u"], ctx["a"]
    if g is None:
        # activation recompute: the forward's gate/up product again (same kernel, same inputs)
        with _Span(events, RECOMPUTE_CALL):
            if not ctx["mxfp8"]:
                g, u, a = ops.grouped_gemm_gate_up(ctx["xp"], off, weights.w_gate, weights.w_up)
            else:
                q = ctx["mx_weights"]
                g, u, a = ops.grouped_gemm_gate_up(ctx["xpq"], off, q["wg"], q["wu"],
                                                   scales=(ctx["xps"], q["wg_s"], q["wu_s"]))
    if not ctx["mxfp8"]:
        with _Span(events, "dgrad_down"):
            dg, du = ops.grouped_gemm_dgrad_down(dyexp, off, weights.w_down, g, u)
        with _Span(events, "wgrad_down"):
            dw_down = ops.grouped_gemm_wgrad_down(dyexp, a, off, g.shape[0])
        with _Span(events, "dgrad_gate_up"):
            dxp = ops.grouped_gemm_dgrad_gate_up(dg, du, off, weights.w_gate, weights.w_up)
        with _Span(events, "permute_bwd"):
            out["dx"] = permute_bwd(dxp)
        with _Span(events, "wgrad_gate_up"):
            dw_gate, dw_up = ops.grouped_gemm_wgrad_gate_up(dg, du, ctx["xp"], off, g.shape[0])
    else:
        # MXFP8: every operand quantised along its product's contraction dim (rows for the dgrads,
        # grouped tokens padded to MX_PAD for the wgrads), then one kernel per product
        q = ctx["mx_weights"]
        n = g.shape[0]
        pad = ctx["offsets_pad"]
        with _Span(events, "dgrad_down"):
            dg, du = ops.grouped_gemm_dgrad_down(dyq, off, q["wd_t"], g, u, scales=(dys, q["wd_t_s"]))
        with _Span(events, "quant_dyT"):
            dyT, dyTs = ops.mxfp8_quantize_grouped(dy, off, pad, n, row_token=ctx["row_token"], row_gate=row_gate)
        aT, aTs = ctx["aT"], ctx["aTs"]          # the forward's grouped token blocks of A
        with _Span(events, "wgrad_down"):
            dw_down = ops.grouped_gemm_wgrad_down(dyT, aT, off, n, offsets_pad=pad, scales=(dyTs, aTs))
        # dG and dU each read once for both layouts: row blocks for the gate/up dgrad, grouped
        # token blocks for the gate/up weight gradient
        with _Span(events, "quant_dg"):
            dgq, dgs, dgT, dgTs = ops.mxfp8_quantize_rows_grouped(dg, off, pad)
        with _Span(events, "quant_du"):
            duq, dus, duT, duTs = ops.mxfp8_quantize_rows_grouped(du, off, pad)
        with _Span(events, "dgrad_gate_up"):
            dxp = ops.grouped_gemm_dgrad_gate_up(dgq, duq, off, q["wg_t"], q["wu_t"],
                                                 scales=(dgs, dus, q["wg_t_s"], q["wu_t_s"]))
        with _Span(events, "permute_bwd"):
            out["dx"] = permute_bwd(dxp)
        with _Span(events, "quant_xT"):
            xT, xTs = ops.mxfp8_quantize_grouped(ctx["x"], off, pad, n, row_token=ctx["row_token"])
        with _Span(events, "wgrad_gate_up"):
            dw_gate, dw_up = ops.grouped_gemm_wgrad_gate_up(dgT, duT, xT, off, n, offsets_pad=pad,
                                                            scales=(dgTs, duTs, xTs))
        out["row_gate"] = row_gate
        out["mx"] = dict(dyq=dyq, dys=dys, dyT=dyT, dyTs=dyTs, aT=aT, aTs=aTs, dgq=dgq, dgs=dgs, duq=duq,
                         dus=dus, dgT=dgT, dgTs=dgTs, duT=duT, duTs=duTs, xT=xT, xTs=xTs)
    out.update(dg=dg, du=du, dxp=dxp, dw_gate=dw_gate, dw_up=dw_up, dw_down=dw_down)
    return out
