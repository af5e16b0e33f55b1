"""The staging index arithmetic of the tiled streaming convolutions (CPU).

The kernels divide a flat staging index e by an extent d fixed for the launch as
q = trunc(float32(e) * float32(1/d)), then correct q by one step from the sign and size of the
remainder e - q*d.  This test replays that arithmetic in IEEE float32 (the GPU's v_mul_f32 and
truncating conversion round the same way) for every divisor up to 8192 and checks it against
integer division for dividends below 2^24.
"""
import numpy as np


def fast_divmod(e, d):
    inv = np.float32(1.0) / np.float32(d)
    q = (e.astype(np.float32) * inv).astype(np.uint32)
    r = e.astype(np.int64) - q.astype(np.int64) * d
    q = np.where(r < 0, q - 1, np.where(r >= d, q + 1, q))
    r = np.where(r < 0, r + d, np.where(r >= d, r - d, r))
    return q, r


def test_fast_divmod_matches_integer_division():
    rng = np.random.default_rng(5)
    small = np.arange(0, 20000, dtype=np.uint32)
    for d in range(1, 8193):
        e = np.concatenate([small, rng.integers(0, 1 << 24, 4000, dtype=np.uint32),
                            np.array([(1 << 24) - 1, d * 4000 - 1, d * 4000], dtype=np.uint32)])
        q, r = fast_divmod(e, d)
        np.testing.assert_array_equal(q, e // d)
        np.testing.assert_array_equal(r, e % d)
