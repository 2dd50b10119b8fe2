"""The property the matrix-core router relies on, checked on the CPU: a
float32 weight w splits exactly into three bf16 terms, hi = bf16(w), mid =
bf16(w - hi), lo = w - hi - mid (each difference exact in float32, lo exact
in bf16), and a bf16 activation times any of the terms is exact in float32,
so the router's products are the float32 products of the unsplit weight."""
import numpy as np


def bf16_rne(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float32."""
    b = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16 << 16
    return (b & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def _weights(n=200_000, seed=7):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 3, n)).astype(np.float32)
    # values at bf16 rounding ties and at the ends of a binade
    ties = (np.float32(1.0) + np.float32(2.0 ** -8) * np.arange(1, 64, 2, dtype=np.float32))
    edge = np.array([1.0, -1.0, np.nextafter(np.float32(2.0), np.float32(0.0)),
                     np.float32(2.0 ** -100), np.float32(3.0e38)], np.float32)
    return np.concatenate([w, ties, -ties, edge])


def test_three_bf16_terms_are_exact():
    w = _weights()
    hi = bf16_rne(w)
    r1 = w - hi                                   # float32 arithmetic
    mid = bf16_rne(r1)
    r2 = r1 - mid
    lo = bf16_rne(r2)
    # every difference is exact, and lo needs no rounding
    assert np.array_equal(r1.astype(np.float64), w.astype(np.float64) - hi.astype(np.float64))
    assert np.array_equal(r2.astype(np.float64), r1.astype(np.float64) - mid.astype(np.float64))
    assert np.array_equal(lo, r2)
    total = hi.astype(np.float64) + mid.astype(np.float64) + lo.astype(np.float64)
    assert np.array_equal(total, w.astype(np.float64))


def test_products_with_bf16_activations_are_exact_in_float32():
    rng = np.random.default_rng(8)
    w = _weights(50_000, seed=9)
    x = bf16_rne(rng.standard_normal(w.size).astype(np.float32) * 3)
    hi = bf16_rne(w)
    mid = bf16_rne(w - hi)
    lo = (w - hi) - mid
    for t in (hi, mid, lo):
        exact = x.astype(np.float64) * t.astype(np.float64)
        # products in float32's normal range (the router's are far inside it)
        ok = (np.abs(exact) > 2.0 ** -120) & (np.abs(exact) < 2.0 ** 127)
        with np.errstate(over="ignore"):
            got = (x * t).astype(np.float64)
        assert np.array_equal(got[ok], exact[ok])
