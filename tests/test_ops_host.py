"""Host-side argument checks of the torch wrappers (no GPU needed): every size the kernels index
is compared across the call's tensors before anything reaches the library, so a mismatch is a
ValueError on the host, never an out-of-range device access.  CPU tensors are used throughout;
with consistent shapes the wrappers stop at the device check, before calling the library."""

import pytest
import torch

from expert_ffn_layer_top_amd import ops

bf, u8, i32, f32 = torch.bfloat16, torch.uint8, torch.int32, torch.float32


def z(*shape, dt=bf):
    return torch.zeros(shape, dtype=dt)


def mismatch(fn, *args, name, **kw):
    with pytest.raises(ValueError, match=name):
        fn(*args, **kw)


def consistent(fn, *args, **kw):
    # consistent shapes: the only complaint left is the device
    with pytest.raises(ValueError, match="GPU"):
        fn(*args, **kw)


T, d, E, k, f = 8, 64, 4, 2, 128
n = T * k


def test_router():
    consistent(ops.router_project, z(T, d), z(d, E, dt=f32))
    mismatch(ops.router_project, z(T, d), z(d + 1, E, dt=f32), name="w_r")
    consistent(ops.router_project_bwd, z(T, d), z(d, E, dt=f32), z(T, E, dt=f32))
    mismatch(ops.router_project_bwd, z(T, d), z(d, E, dt=f32), z(T, E + 1, dt=f32), name="d_logits")


def test_route():
    consistent(ops.route_topk, z(T, E, dt=f32), k)
    dest = z(T, k, dt=i32)
    consistent(ops.route_topk_bwd, z(T, k, dt=f32), dest, z(T, k, dt=f32), E)
    mismatch(ops.route_topk_bwd, z(T, k, dt=f32), dest, z(T, k + 1, dt=f32), E, name="d_gate")
    mismatch(ops.route_topk_bwd, z(T, k, dt=f32), dest, z(T, k, dt=f32), E,
             balance=(z(T, E + 1, dt=f32), z(E, dt=i32), 0.1), name="probs")
    mismatch(ops.route_balance, z(T, E, dt=f32), z(E - 1, dt=i32), k, name="counts")


def test_rows():
    dest = z(T, k, dt=i32)
    consistent(ops.permute, z(T, d), dest)
    mismatch(ops.permute, z(T + 1, d), dest, name="x")
    mismatch(ops.permute, z(T, d, dt=u8), dest, x_scale=z(T, d // 32 + 1, dt=u8), name="x_scale")
    consistent(ops.unpermute_combine, z(n, d), z(T, k, dt=f32), dest)
    mismatch(ops.unpermute_combine, z(n - 1, d), z(T, k, dt=f32), dest, name="yexp")
    mismatch(ops.unpermute_combine, z(n, d), z(T, k + 1, dt=f32), dest, name="topk_gate")
    consistent(ops.unpermute_combine_bwd, z(T, d), z(n, d), z(T, k, dt=f32), dest)
    mismatch(ops.unpermute_combine_bwd, z(T, d), z(n, d + 64), z(T, k, dt=f32), dest, name="yexp")
    mismatch(ops.unpermute_combine_bwd_mx, z(T - 1, d), z(n, d), z(T, k, dt=f32), dest, name="dy")
    consistent(ops.permute_bwd, z(n, d), dest, addend=z(T, d, dt=f32))
    mismatch(ops.permute_bwd, z(n + 1, d), dest, name="dxp")
    mismatch(ops.permute_bwd, z(n, d), dest, addend=z(T, d + 1, dt=f32), name="addend")


def test_quantisers():
    off = z(E + 1, dt=i32)
    consistent(ops.mxfp8_quantize, z(4, d), 0)
    mismatch(ops.mxfp8_quantize, z(40, 48), 0, name="multiple of 32")
    consistent(ops.mxfp8_quantize_grouped, z(n, d), off, off, n)
    mismatch(ops.mxfp8_quantize_grouped, z(n + 1, d), off, off, n, name="x")
    mismatch(ops.mxfp8_quantize_grouped, z(n, d), off, z(E, dt=i32), n, name="offsets_pad")
    mismatch(ops.mxfp8_quantize_grouped, z(T, d), off, off, n, row_token=z(n - 1, dt=i32), name="row_token")
    mismatch(ops.mxfp8_quantize_grouped, z(T, d), off, off, n, row_token=z(n, dt=i32),
             row_gate=z(n + 1, dt=f32), name="row_gate")


def test_grouped_gemms_bf16():
    off = z(E + 1, dt=i32)
    wg, wu, wd = z(E, f, d), z(E, f, d), z(E, d, f)
    consistent(ops.grouped_gemm_gate_up, z(n, d), off, wg, wu)
    mismatch(ops.grouped_gemm_gate_up, z(n, d + 64), off, wg, wu, name="xp")
    mismatch(ops.grouped_gemm_gate_up, z(n, d), z(E, dt=i32), wg, wu, name="offsets")
    mismatch(ops.grouped_gemm_gate_up, z(n, d), off, wg, z(E, f + 64, d), name="w_up")
    consistent(ops.grouped_gemm_down, z(n, f), off, wd)
    mismatch(ops.grouped_gemm_down, z(n, f + 64), off, wd, name="a")
    consistent(ops.grouped_gemm_swiglu, z(n, d), off, wg, wu, wd)
    mismatch(ops.grouped_gemm_swiglu, z(n, d), off, wg, wu, z(E, d, f + 64), name="w_down")
    consistent(ops.grouped_gemm_dgrad_down, z(n, d), off, wd, z(n, f), z(n, f))
    mismatch(ops.grouped_gemm_dgrad_down, z(n, d), off, wd, z(n, f), z(n + 1, f), name="u")
    mismatch(ops.grouped_gemm_dgrad_down, z(n, d), off, z(E, f, d), z(n, f), z(n, f), name="w_down_t")
    consistent(ops.grouped_gemm_wgrad_down, z(n, d), z(n, f), off, n)
    mismatch(ops.grouped_gemm_wgrad_down, z(n, d), z(n - 1, f), off, n, name="a_t")
    consistent(ops.grouped_gemm_dgrad_gate_up, z(n, f), z(n, f), off, wg, wu)
    mismatch(ops.grouped_gemm_dgrad_gate_up, z(n, f), z(n, f), off, wg, z(E, f, d + 64), name="w_up_t")
    consistent(ops.grouped_gemm_wgrad_gate_up, z(n, f), z(n, f), z(n, d), off, n)
    mismatch(ops.grouped_gemm_wgrad_gate_up, z(n, f), z(n, f), z(n + 1, d), off, n, name="xp_t")
    args = (z(n, d), z(n, f), z(n, f), z(n, f), z(n, d), off, wg, wu, wd)
    consistent(ops.grouped_gemm_swiglu_bwd, *args)
    mismatch(ops.grouped_gemm_swiglu_bwd, z(n, d), z(n, f), z(n, f), z(n - 1, f), z(n, d), off, wg, wu, wd, name="a")


def test_grouped_gemms_mxfp8():
    off = z(E + 1, dt=i32)
    wg, wu, wd = z(E, f, d, dt=u8), z(E, f, d, dt=u8), z(E, d, f, dt=u8)
    sx, sg, su, sd = z(n, d // 32, dt=u8), z(E, f, d // 32, dt=u8), z(E, f, d // 32, dt=u8), z(E, d, f // 32, dt=u8)
    consistent(ops.grouped_gemm_gate_up, z(n, d, dt=u8), off, wg, wu, scales=(sx, sg, su))
    mismatch(ops.grouped_gemm_gate_up, z(n, d, dt=u8), off, wg, wu, scales=(z(n + 1, d // 32, dt=u8), sg, su),
             name="xp_scale")
    consistent(ops.grouped_gemm_down, z(n, f), off, wd, w_down_scale=sd)
    mismatch(ops.grouped_gemm_down, z(n, f), off, wd, w_down_scale=z(E, d, f // 32 - 1, dt=u8), name="w_down_scale")
    consistent(ops.grouped_gemm_swiglu, z(n, d, dt=u8), off, wg, wu, wd, scales=(sx, sg, su, sd))
    P = ops._mx_pad_cap(n, E)
    dyT, aT = z(d, P, dt=u8), z(f, P, dt=u8)
    consistent(ops.grouped_gemm_wgrad_down, dyT, aT, off, n, offsets_pad=off,
               scales=(z(P // 32, d, dt=u8), z(P // 32, f, dt=u8)))
    mismatch(ops.grouped_gemm_wgrad_down, dyT, z(f, P - 128, dt=u8), off, n, offsets_pad=off,
             scales=(z(P // 32, d, dt=u8), z(P // 32, f, dt=u8)), name="a_t")
    mismatch(ops.grouped_gemm_wgrad_down, dyT, aT, off, n, offsets_pad=off,
             scales=(z(P // 32, d, dt=u8), z(P // 32, f + 1, dt=u8)), name="a_t_scale")
    # dgrad-direction weights are [E, d, f] (gate, up) and [E, f, d] (down)
    wgt, wdt_ = z(E, d, f, dt=u8), z(E, f, d, dt=u8)
    consistent(ops.grouped_gemm_dgrad_down, z(n, d, dt=u8), off, wdt_, z(n, f), z(n, f),
               scales=(sx, z(E, f, d // 32, dt=u8)))
    mismatch(ops.grouped_gemm_dgrad_down, z(n, d, dt=u8), off, wd, z(n, f), z(n, f),
             scales=(sx, z(E, f, d // 32, dt=u8)), name="w_down_t")
    sdg = z(n, f // 32, dt=u8)
    consistent(ops.grouped_gemm_dgrad_gate_up, z(n, f, dt=u8), z(n, f, dt=u8), off, wgt, wgt,
               scales=(sdg, sdg, z(E, d, f // 32, dt=u8), z(E, d, f // 32, dt=u8)))
    mismatch(ops.grouped_gemm_dgrad_gate_up, z(n, f, dt=u8), z(n, f, dt=u8), off, wg, wg,
             scales=(sdg, sdg, z(E, d, f // 32, dt=u8), z(E, d, f // 32, dt=u8)), name="w_gate_t")
