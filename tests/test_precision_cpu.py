"""Number-format facts the bf16-storage decode path relies on (CPU only).

The key rebuild converts the stored bf16 coefficients to fp16 before the
fp16 matrix product; the conversion must not change any value in fp16's
normal range, and values beyond fp16's largest finite number must saturate
there (round toward zero), not become infinite.
"""

import numpy as np


def _all_bf16_as_f32():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    return bits.view(np.float32)


def test_bf16_values_in_fp16_normal_range_convert_exactly():
    x = _all_bf16_as_f32()
    m = np.isfinite(x) & (np.abs(x) >= np.float32(2.0 ** -14)) & (np.abs(x) <= np.float32(65504.0))
    # 2 signs x 30 binades (2^-14 .. 2^15) x 128 bf16 significands
    assert m.sum() == 2 * 30 * 128
    y = x[m].astype(np.float16).astype(np.float32)
    np.testing.assert_array_equal(y, x[m])


def test_bf16_beyond_fp16_range_saturates_toward_zero():
    # round toward zero in fp16 of a value above the largest finite fp16
    # number is that number; a round-to-nearest conversion would give inf
    x = _all_bf16_as_f32()
    big = x[np.isfinite(x) & (x > np.float32(65504.0))]
    assert len(big) > 0
    rtz = np.minimum(big, np.float32(65504.0)).astype(np.float16)
    assert np.all(rtz == np.float16(65504.0))
    with np.errstate(over="ignore"):
        assert np.all(np.isinf(big.astype(np.float16)[big >= np.float32(65520.0)]))
