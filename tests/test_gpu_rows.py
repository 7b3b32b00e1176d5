"""GPU parity: rowwise permute (bit-exact, bf16 and E4M3 + scales), weighted combine, combine
backward and permute backward (tolerance, on the same inputs as the oracle)."""

import numpy as np
import pytest

from oracle import codecs, moe
from synth import to_bf16_bits
from tests.gpu_util import (BF16_TOL, assert_close, bf16_to_dev, bits, f32_to_dev, host, i32_to_dev, note,
                            u8_to_dev)

pytestmark = pytest.mark.gpu

SHAPES = [(1, 64, 1, 1), (37, 128, 8, 2), (300, 2048, 64, 4), (513, 4096, 128, 8), (64, 7168, 16, 16),
          (129, 192, 5, 5)]


def _routing(T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx, gate, _ = moe.route_topk(rng.standard_normal((T, E)), k)
    _, _, dest, _, _ = moe.route_metadata(idx, E)
    return gate.astype(np.float32), dest


@pytest.mark.parametrize("T,d,E,k", SHAPES)
def test_permute_bf16_bitexact(T, d, E, k):
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(T + d)
    x = to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    _, dest = _routing(T, E, k, T * 3)
    note(f"permute bf16 T={T} d={d} k={k}")
    xp = ops.permute(bf16_to_dev(x), i32_to_dev(dest))
    assert np.array_equal(bits(xp), moe.permute(x, dest))


@pytest.mark.parametrize("T,d,E,k", SHAPES)
def test_permute_e4m3_bitexact(T, d, E, k):
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(T + d + 1)
    q = rng.integers(0, 256, size=(T, d), dtype=np.uint8)
    s = rng.integers(0, 255, size=(T, d // 32), dtype=np.uint8)
    _, dest = _routing(T, E, k, T * 5)
    note(f"permute e4m3 T={T} d={d} k={k}")
    xp, xps = ops.permute(u8_to_dev(q), i32_to_dev(dest), x_scale=u8_to_dev(s))
    assert np.array_equal(host(xp), moe.permute(q, dest))
    assert np.array_equal(host(xps), moe.permute(s, dest))


@pytest.mark.parametrize("T,d,E,k", SHAPES)
def test_combine_and_backward(T, d, E, k):
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(T * d)
    gate, dest = _routing(T, E, k, T * 7)
    yexp = to_bf16_bits(rng.standard_normal((T * k, d)).astype(np.float32))
    dy = to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    note(f"combine T={T} d={d} k={k}")
    yd, gd, dd = bf16_to_dev(yexp), f32_to_dev(gate), i32_to_dev(dest)
    y = ops.unpermute_combine(yd, gd, dd)
    dyexp, dgate = ops.unpermute_combine_bwd(bf16_to_dev(dy), yd, gd, dd)
    assert_close(codecs.bf16_to_f64(bits(y)), moe.combine(yexp, gate, dest), BF16_TOL, "y")
    rdy, rdg = moe.combine_bwd(dy, yexp, gate, dest)
    assert_close(codecs.bf16_to_f64(bits(dyexp)), rdy, BF16_TOL, "dyexp")
    assert_close(host(dgate), rdg, 1e-4, "d_gate")
    # each dyexp element is one fp32 product g * dy rounded once to bf16 (nearest-even): the
    # bits are fixed, which pins the kernels' fp32 -> bf16 rounding exactly
    prod = gate.astype(np.float32)[:, :, None] * codecs.bf16_to_f64(dy).astype(np.float32)[:, None, :]
    want = np.zeros((T * k, d), np.uint16)
    want[dest.reshape(-1)] = codecs.f32_to_bf16(prod).reshape(T * k, d)
    assert np.array_equal(bits(dyexp), want), "dyexp is not the bf16 rounding of the fp32 product"


@pytest.mark.parametrize("T,d,E,k", SHAPES)
@pytest.mark.parametrize("with_addend", [False, True])
def test_permute_bwd(T, d, E, k, with_addend):
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(T + 11 * d)
    _, dest = _routing(T, E, k, T * 9)
    dxp = to_bf16_bits(rng.standard_normal((T * k, d)).astype(np.float32))
    add = rng.standard_normal((T, d)).astype(np.float32) if with_addend else None
    note(f"permute_bwd T={T} d={d} k={k} addend={with_addend}")
    dx = ops.permute_bwd(bf16_to_dev(dxp), i32_to_dev(dest), addend=None if add is None else f32_to_dev(add))
    assert_close(codecs.bf16_to_f64(bits(dx)), moe.permute_bwd(dxp, dest, addend=add), BF16_TOL, "dx")


def test_identity_experts_combine_returns_input():
    """Yexp := Xp (identity experts): the combine returns the gate-weighted sum of identical
    rows, i.e. x itself, to within one bf16 rounding."""
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(3)
    T, d, E, k = 500, 1024, 32, 4
    x = to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    gate, dest = _routing(T, E, k, 17)
    note("identity experts combine")
    xd, dd = bf16_to_dev(x), i32_to_dev(dest)
    y = ops.unpermute_combine(ops.permute(xd, dd), f32_to_dev(gate), dd)
    xf = codecs.bf16_to_f64(x)
    err = np.abs(codecs.bf16_to_f64(bits(y)) - xf)
    assert np.all(err <= 2.0 ** -8 * np.abs(xf) + 1e-6)
