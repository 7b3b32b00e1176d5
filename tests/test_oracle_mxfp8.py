"""Pins for the oracle's MXFP8 block quantiser: the scale over every amax exponent, the
round-trip error bound of an E4M3 block, idempotence, hand-worked edge blocks, the
permute/quantise commutation, a pure-Python loop for the grouped token-axis layout, and
exactness of the MX product on exactly-representable operands."""

import numpy as np
import pytest

from oracle import codecs, moe, mxfp8
from synth import to_bf16_bits


def block_of(values):
    return to_bf16_bits(np.asarray(values, dtype=np.float32).reshape(1, 32))


def test_scale_every_amax_exponent():
    # amax = 1.5 * 2^e for every e a bf16 normal can have, plus bf16 subnormals
    for e in range(-133, 128):
        amax = 1.5 * 2.0 ** e if e >= -126 else 2.0 ** e
        if not np.isfinite(np.float32(amax)):
            continue
        v = np.zeros(32, dtype=np.float32)
        v[7] = amax
        v[3] = -amax / 4
        q, s = mxfp8.quantize_blocks(block_of(v))
        X = 2.0 ** (int(s[0, 0]) - 127)
        # property: unless the scale hits its floor, amax / X lies in [256, 512), i.e. the
        # block's largest element uses E4M3's top binade
        if s[0, 0] > 0:
            assert 256 <= amax / X < 512, (e, s)
        else:
            assert amax / X < 512
        assert int(s[0, 0]) == max(0, min(254, e - 8 + 127))


def test_zero_block_and_signed_zero():
    v = np.zeros(32, dtype=np.float32)
    v[5] = -0.0
    q, s = mxfp8.quantize_blocks(block_of(v))
    assert s[0, 0] == 0
    assert q[0, 5] == 0x80 and np.all(np.delete(q[0], 5) == 0)


def test_single_nonzero_and_exact_448_multiple():
    for m in (-20, 0, 3, 50):
        v = np.zeros(32, dtype=np.float32)
        v[0] = np.float32(448.0 * 2.0 ** m)
        q, s = mxfp8.quantize_blocks(block_of(v))
        assert s[0, 0] == 127 + m and q[0, 0] == 0x7E


def test_rne_midpoints_tie_to_even():
    # amax 256 gives shared exponent 0 (no scaling); 1.0625 and 1.1875 are E4M3 midpoints
    v = np.zeros(32, dtype=np.float32)
    v[:4] = [256.0, 1.0625, 1.1875, -3 * 2.0 ** -10]
    q, s = mxfp8.quantize_blocks(block_of(v))
    assert s[0, 0] == 127
    assert list(q[0, :4]) == [0x78, 0x38, 0x3A, 0x82]


def test_saturation_region_just_below_power_of_two():
    # amax = 508 (largest bf16 below 2^9): shared exponent 0, elements in (448, 512) saturate
    v = np.zeros(32, dtype=np.float32)
    v[:3] = [508.0, 470.0, -460.0]
    q, s = mxfp8.quantize_blocks(block_of(v))
    assert s[0, 0] == 127
    assert list(q[0, :3]) == [0x7E, 0x7E, 0xFE]


def test_roundtrip_bound_random():
    rng = np.random.default_rng(7)
    for scale in (1e-30, 1e-3, 1.0, 37.0, 1e20):
        v = (rng.standard_normal((64, 256)) * scale).astype(np.float32)
        v[rng.random(v.shape) < 0.05] *= 100     # spread within blocks
        b = to_bf16_bits(v)
        q, s = mxfp8.quantize_rows(b)
        deq = mxfp8.dequantize_blocks(q, s)
        vv = codecs.bf16_to_f64(b)
        X = np.repeat(codecs.e8m0_to_f64(s), 32, axis=1)
        bound = np.maximum.reduce([2.0 ** -4 * np.abs(vv), 2.0 ** -10 * X, np.abs(vv) - 448 * X])
        assert np.all(np.abs(deq - vv) <= bound)


def test_idempotent_on_top_binade_blocks():
    rng = np.random.default_rng(8)
    v = (rng.standard_normal((32, 128))).astype(np.float32)
    q, s = mxfp8.quantize_rows(to_bf16_bits(v))
    deq = mxfp8.dequantize_blocks(q, s)
    q2, s2 = mxfp8.quantize_rows(codecs.f64_to_bf16(deq))
    # every nonzero block has its max code in [256, 448] after the first pass
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_cols_layout_is_blocks_along_the_strided_dim():
    rng = np.random.default_rng(9)
    x = to_bf16_bits(rng.standard_normal((64, 96)).astype(np.float32))
    qT, sT = mxfp8.quantize_cols(x)
    assert qT.shape == (96, 64) and sT.shape == (96, 2)
    # brute force: column c, rows 32*b .. 32*b+31 form one block
    for c in (0, 17, 95):
        for blk in range(2):
            col = x[32 * blk:32 * blk + 32, c]
            qb, sb = mxfp8.quantize_blocks(col.reshape(1, 32))
            assert np.array_equal(qT[c, 32 * blk:32 * blk + 32], qb[0]) and sT[c, blk] == sb[0, 0]


def test_quantize_then_permute_equals_permute_then_quantize():
    rng = np.random.default_rng(10)
    T, d, E, k = 40, 64, 6, 3
    x = to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    idx, _, _ = moe.route_topk(rng.standard_normal((T, E)), k)
    _, _, dest, _, _ = moe.route_metadata(idx, E)
    q, s = mxfp8.quantize_rows(x)
    qp, sp = mxfp8.quantize_rows(moe.permute(x, dest))
    assert np.array_equal(moe.permute(q, dest), qp) and np.array_equal(moe.permute(s, dest), sp)


@pytest.mark.parametrize("gather", [False, True])
def test_grouped_token_blocks_loop(gather):
    rng = np.random.default_rng(11)
    T, d, E, k = 50, 64, 5, 2
    logits = rng.standard_normal((T, E))
    logits[:, 4] -= 100.0                                  # expert 4 gets no rows
    idx, _, _ = moe.route_topk(logits, k)
    counts, off, dest, row_token, offp = moe.route_metadata(idx, E, pad=32)
    x = to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    xp = moe.permute(x, dest)
    if gather:
        qT, sT = mxfp8.quantize_grouped(x, off, offp, row_token=row_token)
    else:
        qT, sT = mxfp8.quantize_grouped(xp, off, offp)
    assert qT.shape == (d, offp[E]) and sT.shape == (d, offp[E] // 32)
    # pure-Python loop: for each expert, each column, each 32-row block of the padded group
    for e in range(E):
        for c in range(0, d, 7):
            for b0 in range(offp[e], offp[e + 1], 32):
                blk = np.zeros(32, dtype=np.uint16)
                for i in range(32):
                    r = off[e] + (b0 - offp[e]) + i
                    if r < off[e + 1]:
                        blk[i] = xp[r, c]
                qb, sb = mxfp8.quantize_blocks(blk.reshape(1, 32))
                assert np.array_equal(qT[c, b0:b0 + 32], qb[0])
                assert sT[c, b0 // 32] == sb[0, 0]
    assert counts[4] == 0 and offp[4] == offp[5]


def test_mx_product_exact_on_representable_operands():
    rng = np.random.default_rng(12)
    # small integers are exact E4M3 codes; with the matrix max forced to 256 in every
    # block the scale is 2^0 and the quantised operands equal the inputs exactly
    a = rng.integers(-8, 9, size=(16, 64)).astype(np.float32)
    b = rng.integers(-8, 9, size=(24, 64)).astype(np.float32)
    a[:, ::32] = 256.0
    b[:, ::32] = 256.0
    qa, sa = mxfp8.quantize_rows(to_bf16_bits(a))
    qb, sb = mxfp8.quantize_rows(to_bf16_bits(b))
    assert np.all(sa == 127) and np.all(sb == 127)
    got = mxfp8.mx_gemm_nt(qa, sa, qb, sb)
    want = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(got, want.astype(np.float64))


# ---------------------------------------------------------------- scale_mode 1 (rounded-up scale)

def test_ceil_scale_is_smallest_power_of_two_without_saturation():
    # every bf16 significand (1 + M/128) at several exponents: the scale X of mode 1 is the
    # smallest power of two with amax / X <= 448
    for e in (-120, -10, 0, 3, 50, 119):
        for M in range(128):
            amax = (1 + M / 128) * 2.0 ** e
            v = np.zeros(32, dtype=np.float32)
            v[11] = -amax
            q, s = mxfp8.quantize_blocks(block_of(v), scale_mode=1)
            X = 2.0 ** (int(s[0, 0]) - 127)
            assert amax / X <= 448, (e, M)
            if s[0, 0] > 0:                  # (the scale byte's floor 2^-127 may bind below that)
                assert amax / (X / 2) > 448, (e, M)


def test_ceil_scale_against_floor_rule():
    # mode 1 equals mode 0 except when amax's significand exceeds 1.75 (bf16 mantissa field
    # above 96), where the scale is one larger; equal scales give equal codes
    rng = np.random.default_rng(5)
    x = to_bf16_bits((rng.standard_normal((400, 64)) * np.exp2(rng.integers(-30, 30, (400, 1)))).astype(np.float32))
    q0, s0 = mxfp8.quantize_rows(x)
    q1, s1 = mxfp8.quantize_rows(x, scale_mode=1)
    amax_bits = np.max(x.reshape(400, 2, 32) & 0x7FFF, axis=-1)
    up = (amax_bits & 0x7F) > 96
    assert up.any() and (~up).any()
    assert np.array_equal(s1.astype(int) - s0.astype(int), up.astype(int))
    same = np.repeat(~up, 32, axis=1)
    assert np.array_equal(q1[same], q0[same])


def test_ceil_scale_roundtrip_never_saturates():
    rng = np.random.default_rng(6)
    x = to_bf16_bits((rng.standard_normal((300, 96)) * 100).astype(np.float32))
    q, s = mxfp8.quantize_rows(x, scale_mode=1)
    v = codecs.bf16_to_f64(x)
    r = mxfp8.dequantize_blocks(q, s)
    X = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
    assert np.all(np.abs(r - v) <= np.maximum(2.0 ** -4 * np.abs(v), 2.0 ** -10 * X))
    assert not np.any((q & 0x7F) == 0x7E) or np.all(np.abs(v[(q & 0x7F) == 0x7E]) <= 448 * X[(q & 0x7F) == 0x7E])
