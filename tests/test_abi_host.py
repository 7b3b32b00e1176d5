"""Host-side checks of the C ABI (no GPU needed): the built library loads, exports every function
declared in include/*.h with the binding's signature, and rejects bad host-visible arguments with
the documented status before anything is enqueued (every call below fails argument checks, so
no kernel is launched)."""

import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

try:
    from expert_ffn_layer_top_amd import _lib
except ImportError as exc:      # library not built: the build step is part of the check
    pytest.fail(f"libmoe_mi355x.so not importable: {exc}", pytrace=False)

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b([a-z_][a-z0-9_]*)\s*\(", text):
            name = m.group(1)
            if name.startswith(("moe_", "mxfp8_")):
                names.add(name)
    return names


def test_every_declared_function_is_exported_and_bound():
    names = declared_functions()
    assert len(names) >= 25
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
        assert n in _lib.SIGNATURES, f"{n} exported but has no binding signature"
    assert set(_lib.SIGNATURES) == names


def test_version_and_status_strings():
    assert _lib.lib.moe_abi_version() == 2
    assert _lib.lib.moe_status_string(0) == b"ok"
    assert b"workspace" in _lib.lib.moe_status_string(3)
    assert _lib.lib.moe_status_string(99) == b"unknown status"


def test_workspace_sizes_from_host_scalars():
    L = _lib.lib
    assert L.moe_route_workspace_bytes(8192, 64, 4) == (8192 // 64) * 64 * 4     # one histogram per 64 tokens
    assert L.moe_route_workspace_bytes(1, 1, 1) == 4
    assert L.moe_gg_workspace_bytes(0, 64, 32768, 2048, 1024) == 0          # bf16 needs none
    mx = L.moe_gg_workspace_bytes(1, 64, 131072, 7168, 2048)
    assert mx > 131072 * (7168 + 2 * 2048)                                    # monotone, covers the row operands
    assert L.moe_gg_workspace_bytes(1, 64, 131072, 7168, 2048) <= L.moe_gg_workspace_bytes(1, 64, 131072 * 2, 7168, 2048)
    assert L.moe_mx_pad_cap(512, 8) == 1536 and L.moe_mx_pad_cap(100, 1) == 256
    # dw_r partials over 2048-token splits, then the bf16 parts of d_logits and of w_r (experts
    # padded to 64), each region 256-byte aligned
    al = lambda b: (b + 255) // 256 * 256
    for T, d, E in ((32768, 7168, 64), (1000, 136, 5), (70, 64, 256)):
        S, EP = -(-T // 2048), -(-E // 64) * 64
        assert L.moe_router_bwd_workspace_bytes(T, d, E) == al(S * d * EP * 4) + al(3 * T * EP * 2) + al(3 * d * EP * 2)


def test_argument_checks_return_status_without_launching():
    L = _lib.lib
    fake = ctypes.c_void_p(0x1000)           # never dereferenced: every call fails its checks first
    # route: T = 0, E too large, k > E, null pointer
    assert L.moe_route_topk(fake, 0, 8, 2, *[fake] * 6, 0, fake, None, fake, 1 << 20, None) == UNSUPPORTED
    assert L.moe_route_topk(fake, 16, 300, 2, *[fake] * 6, 0, fake, None, fake, 1 << 20, None) == UNSUPPORTED
    assert L.moe_route_topk(fake, 16, 4, 5, *[fake] * 6, 0, fake, None, fake, 1 << 20, None) == UNSUPPORTED
    assert L.moe_route_topk(None, 16, 8, 2, *[fake] * 6, 0, fake, None, fake, 1 << 20, None) == INVALID
    # route: workspace too small
    assert L.moe_route_topk(fake, 1000, 8, 2, *[fake] * 6, 32, fake, None, fake, 4, None) == WORKSPACE
    assert L.moe_route_topk(fake, 1000, 8, 2, *[fake] * 6, 0, fake, None, fake, 1 << 20, None) == INVALID  # pad 0
    # misaligned pointer
    assert L.moe_unpermute_combine(ctypes.c_void_p(0x1002), fake, fake, 16, 64, 2, fake, None) == INVALID
    # d not a multiple of 64
    assert L.moe_permute(0, fake, None, fake, 16, 100, 2, fake, None, None) == UNSUPPORTED
    # bf16 permute must not get scales; unknown dtype
    assert L.moe_permute(0, fake, fake, fake, 16, 128, 2, fake, fake, None) == INVALID
    assert L.moe_permute(7, fake, None, fake, 16, 128, 2, fake, None, None) == UNSUPPORTED
    # quantiser: bad axis, cols not a multiple of 32
    assert L.mxfp8_quantize(fake, 1, 64, 64, 2, 0, fake, fake, None) == INVALID
    assert L.mxfp8_quantize(fake, 1, 64, 48, 0, 0, fake, fake, None) == UNSUPPORTED
    assert L.mxfp8_quantize(fake, 1, 64, 64, 0, 2, fake, fake, None) == INVALID       # scale_mode 0 or 1
    assert L.mxfp8_quantize(fake, 1, 64, 64, 0, -1, fake, fake, None) == INVALID
    # grouped GEMM: MXFP8 needs d, f multiples of 128 and a workspace
    args = [fake] * 14
    assert L.moe_grouped_gemm_swiglu(1, 8, 256, 192, 256, *args, 0, None) == UNSUPPORTED
    assert L.moe_grouped_gemm_swiglu(1, 8, 256, 256, 256, *args, 0, None) == WORKSPACE
    assert L.moe_grouped_gemm_swiglu(0, 8, 256, 128, 256, fake, fake, fake, *[fake] * 11, 0, None) == INVALID
    # per-kernel backward GEMMs: bf16 takes no scales nor offsets_pad; MXFP8 needs them; null outputs
    assert L.moe_grouped_gemm_dgrad_down(0, 8, 256, 128, 256, fake, fake, fake, fake, None, fake, fake, fake,
                                         fake, None) == INVALID
    assert L.moe_grouped_gemm_dgrad_down(1, 8, 256, 128, 256, fake, fake, None, fake, fake, fake, fake, fake,
                                         fake, None) == INVALID
    assert L.moe_grouped_gemm_wgrad_down(0, 8, 256, 128, 256, fake, fake, fake, None, fake, None, fake,
                                         None) == INVALID
    assert L.moe_grouped_gemm_wgrad_down(1, 8, 256, 128, 256, fake, None, fake, fake, fake, fake, fake,
                                         None) == INVALID
    assert L.moe_grouped_gemm_dgrad_gate_up(0, 8, 256, 128, 256, fake, fake, None, fake, None, fake, None,
                                            fake, None, None, None) == INVALID
    assert L.moe_grouped_gemm_wgrad_gate_up(1, 8, 256, 192, 256, fake, fake, *[fake] * 8, None) == UNSUPPORTED
    assert L.moe_grouped_gemm_wgrad_gate_up(0, 8, 256, 128, 256, fake, None, fake, None, fake, None, fake, None,
                                            fake, None, None) == INVALID
    # two-layout quantiser: rows % 32, cols % 64
    assert L.mxfp8_quantize_both(fake, 1, 48, 64, fake, fake, fake, fake, None) == UNSUPPORTED
    assert L.mxfp8_quantize_both(fake, 1, 64, 96, fake, fake, fake, fake, None) == UNSUPPORTED
    assert L.mxfp8_quantize_both(fake, 1, 64, 64, fake, None, fake, fake, None) == INVALID
    # GEMM-layout quantiser and scale conversion: blocked dim % 32, pointers, no aliasing
    assert L.mxfp8_quantize_gemm(fake, 1, 8, 48, fake, fake, None) == UNSUPPORTED
    assert L.mxfp8_quantize_gemm(fake, 1, 8, 64, fake, None, None) == INVALID
    assert L.mxfp8_quantize_gemm(fake, 0, 8, 64, fake, fake, None) == INVALID
    assert L.mxfp8_scales_to_gemm(fake, 1, 8, 48, ctypes.c_void_p(0x2000), None) == UNSUPPORTED
    assert L.mxfp8_scales_to_gemm(fake, 1, 8, 64, fake, None) == INVALID
    assert L.mxfp8_scales_to_gemm(fake, 1, 8, 64, None, None) == INVALID
    # quantising permute: d % 64, k range, pointers, alignment
    assert L.moe_permute_quant_mx(fake, fake, 8, 96, 2, fake, fake, None) == UNSUPPORTED
    assert L.moe_permute_quant_mx(fake, fake, 8, 128, 17, fake, fake, None) == UNSUPPORTED
    assert L.moe_permute_quant_mx(fake, fake, 8, 128, 2, fake, None, None) == INVALID
    assert L.moe_permute_quant_mx(ctypes.c_void_p(0x1008), fake, 8, 128, 2, fake, fake, None) == INVALID
    # rows + grouped quantiser: C % 64, E range, row outputs required
    assert L.mxfp8_quantize_rows_grouped(fake, fake, fake, 4, 100, 96, fake, fake, fake, fake, None) == UNSUPPORTED
    assert L.mxfp8_quantize_rows_grouped(fake, fake, fake, 0, 100, 128, fake, fake, fake, fake, None) == UNSUPPORTED
    assert L.mxfp8_quantize_rows_grouped(fake, fake, fake, 4, 100, 128, None, fake, fake, fake, None) == INVALID
    assert L.mxfp8_quantize_rows_grouped(fake, fake, fake, 4, 100, 128, fake, None, fake, fake, None) == INVALID
    assert L.mxfp8_quantize_rows_grouped(fake, fake, fake, 4, 100, 128, ctypes.c_void_p(0x1008), fake, fake, fake,
                                         None) == INVALID
    # router: d a multiple of 8, x 16-byte aligned
    assert L.moe_router_project(fake, fake, 64, 12, 8, fake, None) == UNSUPPORTED
    assert L.moe_router_project(ctypes.c_void_p(0x1008), fake, 64, 128, 8, fake, None) == INVALID
    assert L.moe_router_project_bwd(fake, fake, fake, 64, 12, 8, fake, None, None, 0, None) == UNSUPPORTED
    # router backward: either output requested without workspace
    assert L.moe_router_project_bwd(fake, fake, fake, 64, 128, 8, None, fake, None, 0, None) == WORKSPACE
    msg = L.moe_last_error_string().decode()
    assert "workspace" in msg
    assert L.moe_router_project_bwd(fake, fake, fake, 64, 128, 8, fake, None, None, 0, None) == WORKSPACE
    # nothing requested: nothing to do
    assert L.moe_router_project_bwd(fake, fake, fake, 64, 128, 8, None, None, None, 0, None) == 0
    # MXFP8 down product on quantised A: the MXFP8 shape rule, pointers, alignment, scales
    gdm = L.moe_grouped_gemm_down_mx
    assert gdm(4, 256, 192, 256, fake, fake, fake, fake, fake, fake, None) == UNSUPPORTED   # d % 128
    assert gdm(0, 256, 256, 256, fake, fake, fake, fake, fake, fake, None) == UNSUPPORTED   # E = 0
    assert gdm(4, 256, 256, 256, fake, None, fake, fake, fake, fake, None) == INVALID
    assert gdm(4, 256, 256, 256, fake, fake, None, fake, fake, fake, None) == INVALID       # a scale
    assert gdm(4, 256, 256, 256, fake, fake, fake, fake, ctypes.c_void_p(0x1008), fake, None) == INVALID
    assert gdm(4, 256, 256, 256, fake, ctypes.c_void_p(0x1008), fake, fake, fake, fake, None) == INVALID
    # permute backward with the router's dx term: the rows' limits, the router's, the workspace
    pbr = L.moe_permute_bwd_router
    assert pbr(fake, fake, 64, 128, 0, fake, fake, 8, fake, fake, 1 << 30, None) == UNSUPPORTED    # k = 0
    assert pbr(fake, fake, 64, 128, 17, fake, fake, 8, fake, fake, 1 << 30, None) == UNSUPPORTED   # k > 16
    assert pbr(fake, fake, 64, 96, 4, fake, fake, 8, fake, fake, 1 << 30, None) == UNSUPPORTED     # d % 64
    assert pbr(fake, fake, 64, 128, 4, fake, fake, 0, fake, fake, 1 << 30, None) == UNSUPPORTED    # E = 0
    assert pbr(fake, fake, 64, 128, 4, fake, fake, 257, fake, fake, 1 << 30, None) == UNSUPPORTED  # E > 256
    assert pbr(fake, fake, 0, 128, 4, fake, fake, 8, fake, fake, 1 << 30, None) == UNSUPPORTED     # T = 0
    assert pbr(None, fake, 64, 128, 4, fake, fake, 8, fake, fake, 1 << 30, None) == INVALID
    assert pbr(fake, fake, 64, 128, 4, None, fake, 8, fake, fake, 1 << 30, None) == INVALID
    assert pbr(fake, fake, 64, 128, 4, fake, fake, 8, None, fake, 1 << 30, None) == INVALID
    assert pbr(fake, fake, 64, 128, 4, fake, fake, 8, ctypes.c_void_p(0x1008), fake, 1 << 30, None) == INVALID
    need = L.moe_router_bwd_workspace_bytes(64, 128, 8)
    assert pbr(fake, fake, 64, 128, 4, fake, fake, 8, fake, fake, need - 1, None) == WORKSPACE
    assert pbr(fake, fake, 64, 128, 4, fake, fake, 8, fake, None, need, None) == WORKSPACE


def test_argument_checks_of_balance_and_fused_producer():
    L = _lib.lib
    fake = ctypes.c_void_p(0x1000)
    # balance score: shape, null pointers, workspace
    assert L.moe_route_balance(fake, fake, 0, 8, 2, fake, fake, fake, 1 << 20, None) == UNSUPPORTED
    assert L.moe_route_balance(fake, fake, 64, 300, 2, fake, fake, fake, 1 << 20, None) == UNSUPPORTED
    assert L.moe_route_balance(fake, None, 64, 8, 2, fake, fake, fake, 1 << 20, None) == INVALID
    assert L.moe_route_balance(fake, fake, 1000, 8, 2, fake, fake, fake, 4, None) == WORKSPACE
    assert L.moe_route_balance_workspace_bytes(1000, 8) == 4 * 8 * 4          # 4 blocks of 256 tokens
    # route backward with the balance term: null probs, non-finite weight, k > E
    assert L.moe_route_topk_bwd_balance(fake, fake, fake, None, fake, 0.1, 64, 8, 2, fake, None) == INVALID
    assert L.moe_route_topk_bwd_balance(fake, fake, fake, fake, fake, float("nan"), 64, 8, 2, fake, None) == INVALID
    assert L.moe_route_topk_bwd_balance(fake, fake, fake, fake, fake, 0.1, 64, 4, 5, fake, None) == UNSUPPORTED
    # fused MXFP8 combine backward: d a multiple of 64, every output pointer given
    assert L.moe_unpermute_combine_bwd_mx(fake, fake, fake, fake, 16, 96, 2, fake, fake, fake, fake, None) == UNSUPPORTED
    assert L.moe_unpermute_combine_bwd_mx(fake, fake, fake, fake, 16, 128, 2, fake, fake, None, fake, None) == INVALID
    # gated grouped quantiser: row_token and row_gate required, C a multiple of 64
    assert L.mxfp8_quantize_grouped_gated(fake, None, fake, fake, fake, 8, 64, 128, fake, fake, None) == INVALID
    assert L.mxfp8_quantize_grouped_gated(fake, fake, None, fake, fake, 8, 64, 128, fake, fake, None) == INVALID
    assert L.mxfp8_quantize_grouped_gated(fake, fake, fake, fake, fake, 8, 64, 96, fake, fake, None) == UNSUPPORTED


def test_noalloc_route_rejects_sizes_beyond_its_scratch():
    L = _lib.lib
    fake = ctypes.c_void_p(0x1000)
    # ceil(T/64) * E * 4 bytes of per-block counts must fit the fixed scratch (4 MiB): T = 262144
    # at E = 256 fits exactly, one more block does not; rejected before anything is enqueued
    assert L.moe_route_topk_noalloc(fake, 262144 + 64, 256, 2, *[fake] * 6, 32, fake, None, None) == UNSUPPORTED
    assert b"scratch" in L.moe_last_error_string()
    # the route's own argument checks come first
    assert L.moe_route_topk_noalloc(fake, 0, 8, 2, *[fake] * 6, 32, fake, None, None) == UNSUPPORTED
    assert L.moe_route_topk_noalloc(None, 64, 8, 2, *[fake] * 6, 32, fake, None, None) == INVALID
