"""The FP6 operand-tile model used by the GPU tests (no GPU needed).

The matrix-core GEMM stores INT4 codes as FP6 E2M3 numbers. These tests pin
the host model of that format and layout to the format's definition and to
brute-force bit extraction, so that tile comparisons in the GPU tests rest on
something other than the model itself.
"""
import numpy as np
import pytest

import fp6_layout as F


def test_e2m3_represents_every_symmetric_int4_code():
    # OCP FP6 E2M3: bias 1, max normal 2^2 * 1.875 = 7.5, min subnormal 0.125
    vals = sorted(F.e2m3_value(c) for c in range(64))
    assert max(vals) == 7.5 and min(vals) == -7.5
    assert min(v for v in vals if v > 0) == 0.125
    for q in range(-7, 8):
        assert F.e2m3_value(F.ENC[q]) == q
    assert all(F.e2m3_value(c) != -8 for c in range(64))      # -8 has no E2M3 value


def test_e2m3_codes_of_the_header():
    # magnitudes 0..7 encode as 0, 8, 16, 20, 24, 26, 28, 30; negatives set bit 5
    assert [F.ENC[q] for q in range(8)] == [0, 8, 16, 20, 24, 26, 28, 30]
    assert all(F.ENC[-q] == F.ENC[q] | 32 for q in range(1, 8))


def test_exact_accumulation_bound():
    # |product| <= 49; a K-term sum of integers below 2^24 is exact in fp32
    K = 131072
    assert 49 * K < 2 ** 24
    assert np.float32(49 * K) == 49 * K and np.float32(49 * K - 1) == 49 * K - 1


@pytest.mark.parametrize("R,K", [(1, 64), (33, 128), (300, 192)])
def test_tile_round_trip_and_bit_positions(R, K):
    rng = np.random.default_rng(R + K)
    q = rng.integers(-7, 8, (R, K))
    b = F.tile(q)
    assert len(b) == F.tiles_size(R, K) == F.rows_padded(R) * K * 3 // 4
    np.testing.assert_array_equal(F.untile(b, R, K), q)
    assert np.all(F.untile(b, F.rows_padded(R), K)[R:] == 0)
    KT = K // 64
    for _ in range(300):
        r, k = int(rng.integers(0, R)), int(rng.integers(0, K))
        t = (r // 32) * KT + k // 64
        lane = 32 * ((k % 64) // 32) + r % 32
        e = k % 32
        lane_str = bytes(b[t * 1536 + lane * 16:t * 1536 + lane * 16 + 16]) + \
            bytes(b[t * 1536 + 1024 + lane * 8:t * 1536 + 1024 + lane * 8 + 8])
        bits = int.from_bytes(lane_str, "little")
        assert F.e2m3_value((bits >> (6 * e)) & 63) == q[r, k]
