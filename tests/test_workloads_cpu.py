"""CPU checks of the seeded input generator (random draws only, no recurrence arithmetic)."""
import numpy as np

from gated_deltanet_recurrence_rule_amd import workloads as W


def _row_norms(a):
    return np.sqrt(np.sum(a * a, axis=-1)).ravel()


def test_unit_rows_by_default():
    inp = W.random_small(1, [300], 2, 4, 64, 64, dtype="f32")
    for name in ("q", "k"):
        assert np.allclose(_row_norms(inp.as_f64(name)), 1.0, atol=1e-6)


def test_norm_spread_rows():
    """NormSpread gives zero rows, rows below the 1e-12 normalisation floor, and norms spread
    over [1e-2, 1e2], in both element types; v, g and beta are drawn exactly as without it."""
    spread = W.NormSpread(lo=1e-2, hi=1e2, p_zero=0.05, p_tiny=0.02, tiny=1e-13)
    for dtype in ("bf16", "f32"):
        inp = W.random_small(900, [4000], 4, 8, 128, 128, dtype=dtype, qk_spread=spread)
        plain = W.random_small(900, [4000], 4, 8, 128, 128, dtype=dtype)
        for name in ("q", "k"):
            n = _row_norms(inp.as_f64(name))
            assert 0.03 < np.mean(n == 0) < 0.07
            tiny = (n > 0) & (n < 1e-12)
            assert 0.01 < np.mean(tiny) < 0.03
            assert np.allclose(n[tiny], 1e-13, rtol=1e-2)
            big = n[n > 1e-6]
            assert big.min() >= 1e-2 * 0.99 and big.max() <= 1e2 * 1.01
            assert big.min() < 0.012 and big.max() > 80
        for name in ("v", "g", "beta"):
            assert np.array_equal(getattr(inp, name), getattr(plain, name))
