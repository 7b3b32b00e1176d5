"""GPU parity: router top-k + routing metadata (bit-exact), route backward and the router
projection (tolerance), against the oracle on the same inputs."""

import numpy as np
import pytest

import synth
from oracle import codecs, moe
from tests.gpu_util import BF16_TOL, assert_close, bf16_to_dev, bits, f32_to_dev, host, i32_to_dev, note

pytestmark = pytest.mark.gpu


def _logits(kind, T, E, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":        # small integers: many exact ties, including -0.0 vs +0.0
        L = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
        L[rng.random((T, E)) < 0.1] = -0.0
        return L
    if kind == "equal":
        return np.zeros((T, E), dtype=np.float32)
    if kind == "skew":        # some experts never chosen
        L = rng.standard_normal((T, E)).astype(np.float32)
        L[:, ::3] -= 100.0
        return L
    raise ValueError(kind)


CASES = [
    ("normal", 1, 1, 1), ("normal", 7, 3, 2), ("ties", 300, 8, 2), ("equal", 257, 16, 4),
    ("normal", 1000, 64, 4), ("skew", 513, 128, 8), ("normal", 2000, 256, 16), ("ties", 777, 5, 5),
    ("normal", 64, 256, 1),
]


@pytest.mark.parametrize("kind,T,E,k", CASES)
def test_route_topk_bitexact(kind, T, E, k):
    from expert_ffn_layer_top_amd import ops
    L = _logits(kind, T, E, T + E + k)
    note(f"route_topk kind={kind} T={T} E={E} k={k}")
    r = ops.route_topk(f32_to_dev(L), k, want_probs=True, pad=32)
    idx, gate, probs = moe.route_topk(L, k)
    counts, off, dest, row_token, offp = moe.route_metadata(idx, E, pad=32)
    assert np.array_equal(host(r["topk_idx"]), idx)
    assert np.array_equal(host(r["counts"]), counts)
    assert np.array_equal(host(r["offsets"]), off)
    assert np.array_equal(host(r["offsets_pad"]), offp)
    assert np.array_equal(host(r["dest"]), dest)
    assert np.array_equal(host(r["row_token"]), row_token)
    assert np.max(np.abs(host(r["topk_gate"]) - gate)) < 1e-5
    assert np.max(np.abs(host(r["probs"]) - probs)) < 1e-6


@pytest.mark.parametrize("name", ["balanced", "skewed"])
def test_route_topk_workload_logits(name):
    from expert_ffn_layer_top_amd import ops
    cfg = synth.CONFIGS[name]
    L = synth.gen_logits(cfg)
    note(f"route_topk workload={name} T={cfg.T} E={cfg.E} k={cfg.k}")
    r = ops.route_topk(f32_to_dev(L), cfg.k)
    idx, gate, _ = moe.route_topk(L, cfg.k)
    counts, off, dest, row_token, _ = moe.route_metadata(idx, cfg.E)
    assert np.array_equal(host(r["topk_idx"]), idx) and np.array_equal(host(r["dest"]), dest)
    assert np.array_equal(host(r["counts"]), counts) and np.array_equal(host(r["row_token"]), row_token)
    assert np.max(np.abs(host(r["topk_gate"]) - gate)) < 1e-5


@pytest.mark.parametrize("T,E,k", [(5, 4, 2), (300, 64, 4), (1000, 128, 8), (64, 16, 16)])
def test_route_topk_bwd(T, E, k):
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(T * k)
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx, gate, _ = moe.route_topk(L, k)
    dgate = rng.standard_normal((T, k)).astype(np.float32)
    gate32 = gate.astype(np.float32)
    note(f"route_topk_bwd T={T} E={E} k={k}")
    dl = ops.route_topk_bwd(f32_to_dev(gate32), i32_to_dev(idx), f32_to_dev(dgate), E)
    ref = moe.route_topk_bwd(gate32, idx, dgate, E)
    out = host(dl)
    assert np.max(np.abs(out - ref)) <= 1e-6 * max(1.0, np.max(np.abs(ref)))
    mask = np.zeros((T, E), dtype=bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
    assert np.all(out[~mask] == 0.0)


@pytest.mark.parametrize("T,d,E", [(256, 128, 8), (300, 512, 64), (1000, 7168, 64), (130, 200, 5), (257, 136, 12),
                                   (64, 8, 1), (70, 64, 256)])
def test_router_project_and_bwd(T, d, E):
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(d + E)
    x = synth.to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    w_r = (rng.standard_normal((d, E)) * 0.02).astype(np.float32)
    dl = rng.standard_normal((T, E)).astype(np.float32)
    note(f"router_project T={T} d={d} E={E}")
    xd, wd = bf16_to_dev(x), f32_to_dev(w_r)
    logits = ops.router_project(xd, wd)
    dx, dw = ops.router_project_bwd(xd, wd, f32_to_dev(dl))
    assert_close(host(logits), moe.router_project(x, w_r), 1e-5, "logits")
    rdx, rdw = moe.router_project_bwd(x, w_r, dl)
    assert_close(host(dx), rdx, 1e-5, "dx_router")
    assert_close(host(dw), rdw, 1e-5, "dw_r")
    # fixed-order split-K reduction: a repeat gives the same bits
    dx2, dw2 = ops.router_project_bwd(xd, wd, f32_to_dev(dl))
    assert np.array_equal(host(dw2), host(dw)) and np.array_equal(host(dx2), host(dx))


@pytest.mark.parametrize("T,d,E,k", [(300, 192, 8, 2), (1000, 512, 64, 4), (257, 256, 5, 1), (100, 128, 16, 8),
                                     (70, 64, 32, 16), (1, 64, 4, 3), (513, 7168, 64, 4),
                                     # more than 64 experts: several 64-expert chunks, a ragged last one
                                     (130, 128, 256, 8), (64, 320, 96, 2)])
def test_permute_bwd_with_router_term(T, d, E, k):
    """The permute backward with the router's dx term in one kernel: byte-identical to the router
    backward's fp32 dx followed by the permute backward with it as the addend, and within the bf16
    bar of the oracle (ragged token tiles, partial 128-channel tiles, k = 1..16, E up to 256)."""
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(T + d + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, _, _ = moe.route_topk(logits, k)
    _, _, dest, _, _ = moe.route_metadata(idx, E)
    x = synth.to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    w_r = (rng.standard_normal((d, E)) * 0.02).astype(np.float32)
    dl = rng.standard_normal((T, E)).astype(np.float32)
    dxp = synth.to_bf16_bits(rng.standard_normal((T * k, d)).astype(np.float32))
    note(f"permute_bwd_router T={T} d={d} E={E} k={k}")
    dxp_d, dest_d, w_d, dl_d = bf16_to_dev(dxp), i32_to_dev(dest), f32_to_dev(w_r), f32_to_dev(dl)
    fused = ops.permute_bwd_router(dxp_d, dest_d, w_d, dl_d)
    addend, _ = ops.router_project_bwd(bf16_to_dev(x), w_d, dl_d, want_dw=False)
    two = ops.permute_bwd(dxp_d, dest_d, addend=addend)
    assert np.array_equal(bits(fused), bits(two)), "fused call differs from the two calls"
    rdx, _ = moe.router_project_bwd(x, w_r, dl)
    ref = moe.permute_bwd(dxp, dest, addend=rdx)
    assert_close(codecs.bf16_to_f64(bits(fused)), ref, BF16_TOL, "dx")
