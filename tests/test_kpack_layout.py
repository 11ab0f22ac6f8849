"""The test-side k-packed permutation (tests/gpu_util.kpack) against the layout formula
of fp8_quant_row_kpacked, element by element (no GPU)."""
import numpy as np

from tests.gpu_util import kpack


def test_kpack_matches_the_formula():
    for lead, R, C in [((), 32, 192), ((3,), 16, 128)]:
        q = np.arange(int(np.prod(lead, dtype=np.int64)) * R * C, dtype=np.int64).reshape(*lead, R, C)
        p = kpack(q)
        q3 = q.reshape(-1, R, C)
        for b in range(q3.shape[0]):
            for r in range(R):
                for c in range(C):
                    idx = b * R * C + ((r // 16) * (C // 64) + c // 64) * 1024 + (r % 16) * 64 + c % 64
                    assert p[idx] == q3[b, r, c]


def test_one_chunk_is_16_rows_of_64():
    q = np.arange(16 * 64, dtype=np.int64).reshape(16, 64)
    assert np.array_equal(kpack(q), q.reshape(-1))


def test_pair_interleave_matches_the_formula():
    R, C = 6, 128
    q = np.arange(R * C, dtype=np.int64).reshape(R, C)
    p = kpack(q, 2)
    for r in range(R):
        for c in range(C):
            assert p[((r // 2) * (C // 64) + c // 64) * 128 + (r % 2) * 64 + c % 64] == q[r, c]
