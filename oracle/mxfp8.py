"""MXFP8 block quantisation: E4M3 elements with one shared E8M0 scale per 32 elements.

TEST INFRASTRUCTURE ONLY (see the package docstring).

("Ai2 rebuilds Olmo's training stack ..." / "MXFP8 reduces compute and memory costs":
8-bit floats with a separate scale for each small block of values.)  Blocks are 32
consecutive elements along a GEMM's contraction dimension.  Scale rule (the MX
definition's rule; the pages do not give one): for a block v[0..31] of bf16 values

    amax = max |v_i|
    amax == 0:  scale byte 0, every element the signed zero of v_i
    otherwise:  e = floor(log2(amax)) (exact, from the binary exponent),
                shared = clamp(e - 8, -127, 127)      (8 = exponent of 448, E4M3's largest)
                scale byte = shared + 127,  q_i = E4M3_RNE_saturating(v_i / 2^shared)

v_i / 2^shared is exact (a power-of-two scaling of a bf16 value), so the only
rounding is E4M3's own.  Dequantisation is q * 2^(scale - 127), exact in float64.
"""

import numpy as np

from .codecs import bf16_to_f64, e4m3_encode_rne_sat, e4m3_to_f64, e8m0_to_f64

BLOCK = 32


def quantize_blocks(v_bf16, scale_mode=0):
    """Quantise bf16 blocks along the last axis (length a multiple of 32).

    scale_mode 0 is the rule above.  scale_mode 1 takes instead the smallest power of two X with
    amax / X <= 448 (E4M3's largest value), so no element saturates: since 448 = 1.75 * 2^8 this
    is shared = floor(log2 amax) - 8, plus one when amax's significand exceeds 1.75 (the
    rounded-up scale some training recipes use; the MX definition's rule is mode 0).

    Returns (q uint8, same shape; scale uint8, last axis / 32).
    """
    v = bf16_to_f64(v_bf16)
    *lead, C = v.shape
    if C % BLOCK:
        raise ValueError("quantize_blocks: last axis must be a multiple of 32")
    if scale_mode not in (0, 1):
        raise ValueError("quantize_blocks: scale_mode must be 0 or 1")
    vb = v.reshape(*lead, C // BLOCK, BLOCK)
    amax = np.max(np.abs(vb), axis=-1)
    mant, ex = np.frexp(amax)            # amax = mant * 2^ex, mant in [0.5, 1)
    e = ex.astype(np.int64) - 1          # floor(log2(amax)) for amax > 0
    if scale_mode == 1:
        e = e + (2 * mant > 1.75)        # significand 2 * mant in [1, 2)
    shared = np.clip(e - 8, -127, 127)
    shared = np.where(amax == 0, -127, shared)
    scale = (shared + 127).astype(np.uint8)
    w = vb / np.exp2(shared.astype(np.float64))[..., None]
    q = e4m3_encode_rne_sat(w)
    return q.reshape(*lead, C), scale


def dequantize_blocks(q, scale):
    """Inverse of quantize_blocks (blocks along the last axis): float64 values."""
    qv = e4m3_to_f64(q)
    *lead, C = qv.shape
    s = e8m0_to_f64(scale)
    return (qv.reshape(*lead, C // BLOCK, BLOCK) * s[..., None]).reshape(*lead, C)


def quantize_rows(x_bf16, scale_mode=0):
    """Blocks along the contiguous (last) dimension; output in the input's layout."""
    return quantize_blocks(x_bf16, scale_mode)


def quantize_cols(x_bf16, scale_mode=0):
    """Blocks along the strided (first) dimension of a [..., R, C] tensor; the output is
    transposed to [..., C, R] so that each block is contiguous again."""
    x = np.asarray(x_bf16, dtype=np.uint16)
    return quantize_blocks(np.swapaxes(x, -1, -2).copy(), scale_mode)


def quantize_grouped(x_bf16, offsets, offsets_pad, row_token=None):
    """Token-axis blocks restarting at each expert group (the wgrad operands).

    x_bf16 is [n, C] in expert-major row order, or, when row_token is given, the
    token-major source [T, C] read through row_token (row r of the grouped tensor is
    x[row_token[r]]).  Expert e's rows [offsets[e], offsets[e+1]) are placed at padded
    positions [offsets_pad[e], offsets_pad[e] + count_e) of a token axis of length
    offsets_pad[E]; the padding holds zeros (byte 0x00), which change neither a block's
    amax nor any product.  Returns (qT uint8 [C, offsets_pad[E]], scaleT uint8
    [C, offsets_pad[E] / 32]).
    """
    x = np.asarray(x_bf16, dtype=np.uint16)
    off = np.asarray(offsets, dtype=np.int64)
    offp = np.asarray(offsets_pad, dtype=np.int64)
    E = off.shape[0] - 1
    C = x.shape[1]
    npad = int(offp[E])
    grouped = np.zeros((npad, C), dtype=np.uint16)  # bf16 +0.0 padding
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        p0 = offp[e]
        if row_token is None:
            grouped[p0:p0 + (r1 - r0)] = x[r0:r1]
        else:
            grouped[p0:p0 + (r1 - r0)] = x[np.asarray(row_token[r0:r1], dtype=np.int64)]
    return quantize_blocks(grouped.T.copy())


def mx_gemm_nt(qa, sa, qb, sb):
    """C = deq(A) @ deq(B)^T with A [M, K], B [N, K] quantised along K; float64."""
    return dequantize_blocks(qa, sa) @ dequantize_blocks(qb, sb).T
