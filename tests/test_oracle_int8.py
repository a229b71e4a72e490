"""Pins of the oracle's int8 cache quantizer (symmetric, one fp32 scale per (token, kv
head) row, round half to even) and of attention over dequantized rows."""
import numpy as np
import pytest

from oracle import oracle


def test_known_values_and_ties_to_even():
    x = np.array([[127.0, -63.5, 0.0, 1.0, 2.5, -0.5]], np.float32)
    q, s = oracle.quantize_rows(x)
    assert s.dtype == np.float32 and s[0] == np.float32(1.0)
    assert q.tolist() == [[127, -64, 0, 1, 2, 0]]          # -63.5 -> -64, 2.5 -> 2, -0.5 -> 0


def test_zero_row_gives_zero_scale_and_codes():
    q, s = oracle.quantize_rows(np.zeros((3, 16), np.float32))
    assert not s.any() and not q.any()


@pytest.mark.parametrize("seed", range(4))
def test_codes_bound_max_and_error(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((50, 128)) * rng.uniform(1e-3, 1e3, (50, 1))).astype(np.float32)
    q, s = oracle.quantize_rows(x)
    assert np.abs(q.astype(int)).max() <= 127
    # the largest |x| of a row maps to +-127
    i = np.argmax(np.abs(x), axis=1)
    assert np.array_equal(np.abs(q[np.arange(50), i]), np.full(50, 127))
    # every element within half a step (plus the fp32 division) of its code
    err = np.abs(x.astype(np.float64) - oracle.dequantize_rows(q, s))
    assert (err <= 0.5 * s[:, None] * (1 + 1e-6) + 1e-30).all()
    # odd symmetry
    qn, sn = oracle.quantize_rows(-x)
    assert np.array_equal(sn, s) and np.array_equal(qn, -q)


def test_bf16_rows_widen_before_quantizing():
    # bf16 1.0 (0x3F80) and -2.0 (0xC000): scale 2/127, codes 64 (63.5 ties to even) and -127
    q, s = oracle.quantize_rows(np.array([[0x3F80, 0xC000]], np.uint16))
    assert s[0] == np.float32(2.0) / np.float32(127.0)
    assert q.tolist() == [[64, -127]]


def test_attention_takes_float64_storage_exactly():
    """The float64 storage path reads the values themselves: a one-key decode returns that
    key's value row exactly."""
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 2, 8))
    k = rng.standard_normal((1, 4, 1, 8))
    v = rng.standard_normal((1, 4, 1, 8))
    out, lse = oracle.paged_attention(q, k, v, np.zeros((1, 1), np.int32), [0, 1], [1], 0.5, False)
    assert np.array_equal(out[0, 0], v[0, 0, 0]) and np.array_equal(out[0, 1], v[0, 0, 0])
    np.testing.assert_allclose(lse[0], 0.5 * (q[0] @ k[0, 0, 0]), rtol=0, atol=1e-15)
