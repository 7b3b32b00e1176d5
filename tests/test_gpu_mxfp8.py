"""GPU parity: MXFP8 block quantisation, bit-exact against the oracle — every finite bf16 bit
pattern, edge blocks (zeros, signed zeros, subnormals, saturation, midpoints), random data in
the row, column (transposed) and grouped token-axis layouts."""

import numpy as np
import pytest

from oracle import codecs, moe, mxfp8
from synth import to_bf16_bits
from tests.gpu_util import bf16_to_dev, gemm_scales_to_rows, host, i32_to_dev, note, u8_to_dev

pytestmark = pytest.mark.gpu


def finite_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = codecs.bf16_to_f64(b)
    b = b.copy()
    b[~np.isfinite(v)] = 0          # NaN / Inf inputs are outside the supported set
    return b


def check_rows(x_bits, scale_mode=0):
    from expert_ffn_layer_top_amd import ops
    q, s = ops.mxfp8_quantize(bf16_to_dev(x_bits), 0, scale_mode=scale_mode)
    rq, rs = mxfp8.quantize_rows(x_bits, scale_mode=scale_mode)
    assert np.array_equal(host(s), rs), "scales differ"
    assert np.array_equal(host(q), rq), "elements differ"


def test_every_bf16_pattern_in_natural_blocks():
    b = finite_patterns()
    note("mxfp8 rows: all bf16 patterns")
    check_rows(b.reshape(2048, 32))
    # the same patterns under a different block grouping (neighbours from far-apart exponents)
    check_rows(np.ascontiguousarray(b.reshape(32, 2048).T).reshape(64, 1024))


@pytest.mark.parametrize("scale_mode", [0, 1])
def test_every_bf16_pattern_against_every_block_scale(scale_mode):
    """Each bf16 pattern next to an anchor that fixes the block's scale, for anchors spanning the
    scale range: exercises subnormal, normal and saturating encodes of every mantissa.  Under
    scale_mode 1 the anchors with a significand above 1.75 raise the scale by one."""
    b = finite_patterns()
    mags = b & 0x7FFF
    for anchor_exp in (-120, -60, -10, 0, 7, 60, 120):
        for sig in (1.5, 1.75, 1.7578125, 1.9921875):
            anchor = to_bf16_bits(np.array([sig * 2.0 ** anchor_exp], dtype=np.float32))[0]
            sel = b[mags <= anchor]                              # values not above the anchor
            sel = sel[: (len(sel) // 31) * 31].reshape(-1, 31)
            blocks = np.concatenate([np.full((sel.shape[0], 1), anchor, dtype=np.uint16), sel], axis=1)
            nb = blocks.shape[0] // 32 * 32                      # rows of 32 blocks each
            note(f"mxfp8 rows mode {scale_mode}: anchor {sig} * 2^{anchor_exp}, {nb} blocks")
            check_rows(blocks[:nb].reshape(-1, 1024), scale_mode)


@pytest.mark.parametrize("scale_mode", [0, 1])
def test_edge_blocks(scale_mode):
    vals = np.zeros((8, 32), dtype=np.float32)
    vals[1, 5] = -0.0                                     # signed zero, all-zero block
    vals[2, 0] = 448.0 * 2.0 ** 20                        # exact 448 multiple
    vals[3, :4] = [256.0, 1.0625, 1.1875, -3 * 2.0 ** -10]  # RNE midpoints
    vals[4, :3] = [508.0, 470.0, -460.0]                  # saturation region
    vals[5, :2] = [2.0 ** -130, -2.0 ** -133]             # bf16 subnormals only
    vals[6, :3] = [1e30, 1e-30, -1e20]                    # wide dynamic range
    vals[7] = np.linspace(-1, 1, 32)
    note(f"mxfp8 rows mode {scale_mode}: edge blocks")
    check_rows(to_bf16_bits(vals.reshape(1, 256)), scale_mode)


@pytest.mark.parametrize("R,C", [(1, 32), (3, 64), (300, 2048), (1025, 7168)])
def test_rows_random(R, C):
    rng = np.random.default_rng(R + C)
    v = rng.standard_normal((R, C)).astype(np.float32) * np.exp(rng.standard_normal((R, 1)) * 4).astype(np.float32)
    note(f"mxfp8 rows random R={R} C={C}")
    check_rows(to_bf16_bits(v))


@pytest.mark.parametrize("B,R,C", [(1, 32, 64), (1, 288, 192), (3, 256, 128), (2, 2048, 1024), (1, 7168, 2048)])
@pytest.mark.parametrize("scale_mode", [0, 1])
def test_cols_transposed(B, R, C, scale_mode):
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(B * R + C)
    x = to_bf16_bits(rng.standard_normal((B, R, C)).astype(np.float32))
    note(f"mxfp8 cols B={B} R={R} C={C} mode {scale_mode}")
    q, s = ops.mxfp8_quantize(bf16_to_dev(x), 1, scale_mode=scale_mode)
    rq, rs = mxfp8.quantize_cols(x, scale_mode=scale_mode)
    assert np.array_equal(host(s), rs) and np.array_equal(host(q), rq)


@pytest.mark.parametrize("B,R,C", [(1, 32, 64), (1, 288, 192), (3, 256, 128), (2, 160, 320), (5, 96, 320), (4, 2048, 1024),
                                   (1, 7168, 2048)])
def test_rows_and_cols_from_one_read(B, R, C):
    """The two-layout quantiser (used for the weights) against the oracle in both layouts, on
    shapes with partial 128 x 128 tiles in either dimension and a per-row dynamic range."""
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(7 * B + R + C)
    v = rng.standard_normal((B, R, C)).astype(np.float32) * np.exp(rng.standard_normal((B, R, 1)) * 3).astype(np.float32)
    x = to_bf16_bits(v)
    note(f"mxfp8 both B={B} R={R} C={C}")
    q, s, qT, sT = ops.mxfp8_quantize_both(bf16_to_dev(x))
    rq, rs = mxfp8.quantize_rows(x)
    cq, cs = mxfp8.quantize_cols(x)
    # scales in the GEMM scale layout of each matrix (R = rows, K = cols; transposed: R = cols, K = rows)
    assert np.array_equal(gemm_scales_to_rows(host(s), R, C), rs) and np.array_equal(host(q), rq)
    assert np.array_equal(gemm_scales_to_rows(host(sT), C, R), cs) and np.array_equal(host(qT), cq)


@pytest.mark.parametrize("B,R,C", [(1, 32, 64), (3, 100, 128), (2, 257, 512), (1, 96, 7168), (4, 40, 2048)])
def test_gemm_scale_layout_producers(B, R, C):
    """Row blocks with GEMM-layout scales (mxfp8_quantize_gemm) and the conversion of row-major
    scales into that layout (mxfp8_scales_to_gemm), against the oracle's row blocks."""
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(B * R + C)
    v = rng.standard_normal((B, R, C)).astype(np.float32) * np.exp(rng.standard_normal((B, R, 1)) * 3).astype(np.float32)
    x = to_bf16_bits(v)
    note(f"mxfp8 gemm-layout scales B={B} R={R} C={C}")
    q, s = ops.mxfp8_quantize_gemm(bf16_to_dev(x))
    rq, rs = mxfp8.quantize_rows(x)
    assert np.array_equal(host(q), rq) and np.array_equal(gemm_scales_to_rows(host(s), R, C), rs)
    s2 = ops.mxfp8_scales_to_gemm(u8_to_dev(rs), C)
    assert np.array_equal(host(s2), host(s))


@pytest.mark.parametrize("T,E,k,C", [(40, 5, 2, 64), (700, 6, 2, 256), (1000, 64, 4, 128), (300, 16, 8, 192)])
@pytest.mark.parametrize("pad", [32, 64, 128])
def test_rows_and_grouped_from_one_read(T, E, k, C, pad):
    """Both layouts of a grouped tensor from one read (the backward's dG, dU) against the oracle's
    row blocks and grouped token blocks, with an empty expert group and ragged group sizes."""
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(3 * T + E + C)
    logits = rng.standard_normal((T, E))
    logits[:, E // 2] -= 100.0                            # an empty expert group
    idx, _, _ = moe.route_topk(logits, k)
    _, off, dest, row_token, offp = moe.route_metadata(idx, E, pad=pad)
    n = T * k
    v = rng.standard_normal((n, C)).astype(np.float32) * np.exp(rng.standard_normal((n, 1)) * 3).astype(np.float32)
    xp = to_bf16_bits(v)
    note(f"mxfp8 rows+grouped T={T} E={E} k={k} C={C} pad={pad}")
    q, s, qT, sT = ops.mxfp8_quantize_rows_grouped(bf16_to_dev(xp), i32_to_dev(off), i32_to_dev(offp))
    rq, rs = mxfp8.quantize_rows(xp)
    assert np.array_equal(host(q), rq) and np.array_equal(gemm_scales_to_rows(host(s), n, C), rs)
    gq, gs = mxfp8.quantize_grouped(xp, off, offp)
    qT, sT = host(qT), host(sT).T
    assert np.array_equal(qT[:, : offp[E]], gq) and np.array_equal(sT[:, : offp[E] // 32], gs)
    assert np.all(qT[:, offp[E]:] == 0) and np.all(sT[:, offp[E] // 32:] == 0)


@pytest.mark.parametrize("T,E,k,C", [(40, 5, 2, 64), (700, 6, 2, 256), (1000, 64, 4, 128), (300, 16, 8, 192)])
@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("pad", [32, 64, 128])
def test_grouped_token_blocks(T, E, k, C, gather, pad):
    from expert_ffn_layer_top_amd import ops
    rng = np.random.default_rng(T + E + C)
    logits = rng.standard_normal((T, E))
    logits[:, E // 2] -= 100.0                            # an empty expert group
    idx, _, _ = moe.route_topk(logits, k)
    _, off, dest, row_token, offp = moe.route_metadata(idx, E, pad=pad)
    x = to_bf16_bits(rng.standard_normal((T, C)).astype(np.float32))
    xp = moe.permute(x, dest)
    n = T * k
    note(f"mxfp8 grouped T={T} E={E} k={k} C={C} gather={gather} pad={pad}")
    if gather:
        q, s = ops.mxfp8_quantize_grouped(bf16_to_dev(x), i32_to_dev(off), i32_to_dev(offp), n,
                                          row_token=i32_to_dev(row_token))
    else:
        q, s = ops.mxfp8_quantize_grouped(bf16_to_dev(xp), i32_to_dev(off), i32_to_dev(offp), n)
    rq, rs = mxfp8.quantize_grouped(xp, off, offp)
    P = ops.mx_pad_cap(n, E)
    q, s = host(q), host(s)
    assert q.shape == (C, P) and s.shape == (P // 32, C)
    s = s.T                                               # block-major on the device
    assert np.array_equal(q[:, : offp[E]], rq) and np.array_equal(s[:, : offp[E] // 32], rs)
    assert np.all(q[:, offp[E]:] == 0) and np.all(s[:, offp[E] // 32:] == 0)
