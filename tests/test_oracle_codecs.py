"""Pins for the oracle's bit codecs (bf16, E4M3, E8M0) against things other than itself:
the CPU torch casts (an independent library), a brute-force nearest-code search over
every finite E4M3 code, exhaustive enumeration of bf16 inputs, and the landmark table
in tests/golden/e4m3_landmarks.txt (from the format definition)."""

import os

import numpy as np
import pytest
import torch

from oracle import codecs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = codecs.bf16_to_f64(b)
    return b[np.isfinite(v)], v[np.isfinite(v)]


def test_bf16_decode_matches_torch_exhaustive():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bf16_to_f64(b)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[fin], ref[fin])


def test_f32_to_bf16_matches_torch_rne():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    # add exact ties (low half 0x8000) with even and odd upper halves, and near-ties
    hi = rng.integers(0, 2 ** 16, size=20_000, dtype=np.uint64).astype(np.uint32)
    bits = np.concatenate([bits, (hi << 16) | 0x8000, (hi << 16) | 0x7FFF, (hi << 16) | 0x8001])
    x = bits.view(np.float32)
    fin = np.isfinite(x)
    ours = codecs.f32_to_bf16(x[fin])
    ref = torch.from_numpy(x[fin].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f32_to_bf16_nan_stays_nan():
    x = np.array([np.nan, -np.nan], dtype=np.float32)
    assert np.all(np.isnan(codecs.bf16_to_f64(codecs.f32_to_bf16(x))))


def _e4m3_table():
    codes = np.arange(0x7F, dtype=np.uint8)           # 0x00..0x7E: the finite magnitudes
    return codes, codecs.e4m3_to_f64(codes)


def test_e4m3_decode_landmarks_and_monotone():
    codes, vals = _e4m3_table()
    assert vals[0] == 0.0 and vals[0x7E] == 448.0 and vals[0x38] == 1.0 and vals[1] == 2.0 ** -9
    assert np.all(np.diff(vals) > 0)                  # magnitude increases with the code
    assert np.isnan(codecs.e4m3_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def brute_force_e4m3(w):
    """Nearest finite E4M3 magnitude by exhaustive search; ties to the even code."""
    codes, vals = _e4m3_table()
    a = np.abs(w)[:, None]
    dist = np.abs(a - vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among tied candidates prefer an even code (even mantissa LSB)
    even = cand & ((codes[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    return (codes[pick] | np.where(np.signbit(w), 0x80, 0)).astype(np.uint8)


@pytest.mark.parametrize("shift", [-12, -8, -4, 0, 4, 8])
def test_e4m3_encoder_exhaustive_vs_brute_force_and_torch(shift):
    # every finite bf16 value, moved by a power of two so each range of the E4M3 grid
    # (subnormals, normals, saturation) is hit with every bf16 mantissa
    _, v = all_finite_bf16()
    w = np.ldexp(v, shift)
    w = w[np.isfinite(w)]
    ours = codecs.e4m3_encode_rne_sat(w)
    # the brute-force distances are exact in float64 only for moderate magnitudes; above
    # that every finite code is farther than 448, so the answer is plain saturation
    mod = np.abs(w) < 2.0 ** 40
    assert np.array_equal(ours[mod], brute_force_e4m3(w[mod]))
    assert np.all((ours[~mod] & 0x7F) == 0x7E)
    ref = torch.from_numpy(np.clip(w, -448.0, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_golden_landmarks(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "e4m3_landmarks.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            val, code = line.split()
            if "*" in val:
                a, b = val.split("*")
                v = float(a) * 2.0 ** float(b.split("^")[1])
            elif val.lstrip("-").startswith("2^"):
                v = 2.0 ** float(val.lstrip("-").split("^")[1]) * (-1 if val.startswith("-") else 1)
            else:
                v = float(val)
            rows.append((v, int(code, 16)))
    w = np.array([r[0] for r in rows])
    want = np.array([r[1] for r in rows], dtype=np.uint8)
    assert np.array_equal(codecs.e4m3_encode_rne_sat(w), want)


def test_e4m3_roundtrip_of_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(codecs.e4m3_encode_rne_sat(codecs.e4m3_to_f64(codes)), codes)


def test_e8m0_decode():
    s = np.arange(255, dtype=np.uint8)
    assert np.array_equal(codecs.e8m0_to_f64(s), 2.0 ** (np.arange(255) - 127.0))
    assert np.isnan(codecs.e8m0_to_f64(np.array([255], dtype=np.uint8)))[0]
    ref = torch.from_numpy(s.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(codecs.e8m0_to_f64(s), ref)


# ---------------------------------------------------------------- f64 -> bf16 (fp32 storage)

def _bf16_neighbours():
    """Finite positive bf16 values v with an even last mantissa bit and their successors."""
    b = np.arange(0x0080, 0x7F7F, 2, dtype=np.uint32).astype(np.uint16)     # normals, even mantissa
    return b, codecs.bf16_to_f64(b), codecs.bf16_to_f64(b + 1)


def test_f64_to_bf16_equals_f32_rounding_on_f32_values():
    # values representable in fp32 take one rounding, pinned above against torch
    rng = np.random.default_rng(9)
    x = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(codecs.f64_to_bf16(x.astype(np.float64)), codecs.f32_to_bf16(x))


def test_f64_to_bf16_rounds_through_fp32():
    # The helper models an fp32 accumulator stored as bf16: first to fp32 (nearest even), then to
    # bf16 (nearest even).  Just above a bf16 midpoint m (itself an fp32 value), an excess below
    # half an fp32 ulp is lost in the first rounding, so the tie goes to the even neighbour; an
    # excess above it rounds away, as a single rounding would.
    b, v, w = _bf16_neighbours()
    m = (v + w) / 2
    assert np.array_equal(codecs.f64_to_bf16(m), b)                          # exact tie -> even
    assert np.array_equal(codecs.f64_to_bf16(m * (1 + 2.0 ** -30)), b)       # below half an fp32 ulp
    assert np.array_equal(codecs.f64_to_bf16(m * (1 + 2.0 ** -20)), b + 1)   # above it
    assert np.array_equal(codecs.f64_to_bf16(-m * (1 + 2.0 ** -20)), (b + 1) | 0x8000)


def test_f64_to_bf16_error_bound_and_monotone():
    rng = np.random.default_rng(10)
    x = np.sort(rng.standard_normal(100_000) * np.exp2(rng.integers(-60, 60, size=100_000)))
    r = codecs.bf16_to_f64(codecs.f64_to_bf16(x))
    assert np.all(np.abs(r - x) <= (2.0 ** -8 + 2.0 ** -24) * np.abs(x))   # half a bf16 ulp + fp32 step
    assert np.all(np.diff(r) >= 0)
