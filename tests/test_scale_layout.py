"""The host helper that undoes the GEMM scale layout (used by the GPU tests to compare scale bytes
with the oracle's row-major scales), against the layout's definition written out byte by byte."""

import numpy as np
import pytest

from tests.gpu_util import gemm_group, gemm_scales_to_rows


@pytest.mark.parametrize("R,K", [(5, 64), (7, 128), (3, 512), (9, 7168), (4, 2048), (6, 96), (1, 32)])
def test_gemm_scales_to_rows_inverts_the_layout(R, K):
    rng = np.random.default_rng(R * K)
    rows = rng.integers(0, 256, size=(2, R, K // 32), dtype=np.uint8)
    G = gemm_group(K)
    flat = np.zeros((2, R * (K // 32)), np.uint8)
    for m in range(2):
        for r in range(R):
            for b in range(K // 32):
                flat[m, ((b // G) * R + r) * G + b % G] = rows[m, r, b]
    assert np.array_equal(gemm_scales_to_rows(flat.reshape(2, R, K // 32), R, K), rows)
    assert np.array_equal(gemm_scales_to_rows(flat[0], R, K), rows[0])
    assert G in (1, 4, 16) and (K // 32) % G == 0
