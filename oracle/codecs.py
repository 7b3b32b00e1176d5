"""Bit codecs for the oracle: bf16, FP8 E4M3 ("fn" variant) and E8M0 scales.

TEST INFRASTRUCTURE ONLY (see the package docstring).

bf16 tensors travel as uint16 bit patterns (the upper half of an IEEE binary32).
E4M3 and E8M0 travel as uint8 codes.  The format facts restated here are those of
the OCP Microscaling (MX) formats definition, which the MXFP8 format named in
"Ai2 rebuilds Olmo's training stack ..." / section "MXFP8 reduces compute and memory
costs" refers to:

  E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 holds
        subnormals m * 2^-9; the largest finite magnitude is 1.75 * 2^8 = 448 (code
        0x7E); codes 0x7F / 0xFF are NaN; there is no infinity.
  E8M0: an unsigned biased exponent, byte s meaning 2^(s - 127); 0xFF is NaN.
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_MAX_CODE = 0x7E


# ---------------------------------------------------------------- bf16

def bf16_to_f64(bits):
    """Decode bf16 bit patterns (uint16 array) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16(x):
    """Round float32 values to bf16 with round-to-nearest-even; returns uint16 bits.

    NaN inputs give a quiet NaN with the input's sign.  Overflow past the largest
    finite bf16 rounds to infinity, as IEEE rounding does.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    qnan = ((u >> 16) | 0x0040).astype(np.uint16)
    return np.where(nan, qnan, r).astype(np.uint16)


def f64_to_bf16(x):
    """float64 -> float32 (RNE) -> bf16 (RNE): how an fp32 accumulator is stored."""
    return f32_to_bf16(np.asarray(x, dtype=np.float64).astype(np.float32))


# ---------------------------------------------------------------- E4M3

def e4m3_to_f64(codes):
    """Decode E4M3 codes (uint8 array) to float64 exactly; NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode_rne_sat(w):
    """Encode finite float64 values to E4M3 with round-to-nearest-even and saturation.

    Magnitudes that round above 448 become +-448 (code 0x7E / 0xFE), never NaN.  The
    sign is kept, including that of -0.0.  Inputs must be finite; the callers only
    pass values v / 2^s of bf16 v, which are exact dyadic rationals, so the scaling
    and the rint below are exact.
    """
    w = np.asarray(w, dtype=np.float64)
    if not np.all(np.isfinite(w)):
        raise ValueError("e4m3_encode_rne_sat: non-finite input")
    neg = np.signbit(w)
    a = np.abs(w)
    code = np.zeros(a.shape, dtype=np.int64)

    # Subnormal range (below the smallest normal 2^-6): spacing 2^-9.
    sub = a < 2.0 ** -6
    m_sub = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)  # 0..8; 8 is the min normal, code 0x08
    code[sub] = m_sub

    # Normal range: a = (m/8) * 2^e with m in [8, 16) before rounding.
    nrm = ~sub
    an = a[nrm]
    e = np.floor(np.log2(an)).astype(np.int64)
    # log2 of a float can be off by one right at powers of two; fix e so 2^e <= a < 2^(e+1).
    e = np.where(np.exp2(e.astype(np.float64)) > an, e - 1, e)
    e = np.where(np.exp2((e + 1).astype(np.float64)) <= an, e + 1, e)
    m = np.rint(an / np.exp2((e - 3).astype(np.float64))).astype(np.int64)  # 8..16
    carry = m == 16
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 8, m)
    c = ((e + 7) << 3) | (m - 8)
    # Saturate: anything above the largest finite code (including 480 = code 0x7F) -> 0x7E.
    c = np.where((e > 8) | ((e == 8) & (m > 14)), E4M3_MAX_CODE, c)
    code[nrm] = c
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


# ---------------------------------------------------------------- E8M0

def e8m0_to_f64(s):
    """Decode E8M0 scale bytes to float64 powers of two; 0xFF gives NaN."""
    s = np.asarray(s, dtype=np.uint8).astype(np.float64)
    return np.where(s == 255, np.nan, np.exp2(s - 127.0))
