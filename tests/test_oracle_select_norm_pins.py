"""Pins of the oracle's robust normalisations ("SpecPrefill - Implementation
Guide", Limitations item 5: percentile-based or z-score normalisation as the
remedy for min-max's sensitivity to outliers). The readings (percentile clip to
two order statistics, then min-max between them; z-score clipped at +-c
standard deviations, mapped onto [0, 1], with its statistics taken exactly on a
2^-16 grid of the min-max values) are fixed here by closed forms and special
cases that a dropped term, a wrong index or a wrong sign would break."""
import math

import numpy as np
import pytest

import oracle


def v_of(x, norm, lo=0.0, hi=0.0, **kw):
    x = np.asarray(x, np.float32)
    args = dict(chunk=1, pool_k=1, mode="topk", keep_rate=0.5)
    args.update(kw)
    _, _, dbg = oracle.select(x, norm=norm, norm_lo=lo, norm_hi=hi, debug=True, **args)
    return dbg["v"]


def test_percentile_zero_one_is_minmax():
    rng = np.random.default_rng(1)
    x = rng.random(3000).astype(np.float32) ** 3
    for kw in (dict(mode="topk", keep_rate=0.2), dict(mode="mass", mass=0.7)):
        a = oracle.select(x, 32, 5, norm="minmax", debug=True, **kw)
        b = oracle.select(x, 32, 5, norm="percentile", norm_lo=0.0, norm_hi=1.0, debug=True, **kw)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[2]["v"], b[2]["v"])


def test_percentile_clip_closed_form():
    """x = 0, 1, ..., 98 and one outlier 1000 (M = 100). p_hi = 0.9 picks the
    order statistic at index ceil(0.9 * 99) = 90, i.e. 90; p_lo = 0.1 the one at
    floor(0.1 * 99) = 9. Then v = clamp((x - 9) / 81, 0, 1): the outlier and
    everything from 90 up is 1, everything up to 9 is 0."""
    x = np.arange(100, dtype=np.float32)
    x[99] = 1000.0
    v = v_of(x, "percentile", 0.1, 0.9)
    want = np.clip((x - np.float32(9)) / np.float32(81), 0, 1).astype(np.float32)
    assert np.array_equal(v, want)
    assert v[99] == 1.0 and v[90] == 1.0 and v[9] == 0.0 and v[0] == 0.0
    # min-max on the same scores squeezes the 99 ordinary tokens below 0.1
    assert np.max(v_of(x, "minmax")[:99]) < 0.1


def test_percentile_degenerate_range():
    """lo == hi (a plateau spans both quantiles): v = 1 for x >= hi, else 0."""
    x = np.array([0.0] * 10 + [1.0] * 80 + [2.0] * 10, np.float32)
    v = v_of(x, "percentile", 0.2, 0.8)  # indices 19 and 80: both 1.0
    assert np.array_equal(v, (x >= 1.0).astype(np.float32))


def test_zscore_two_points():
    """Half the scores at one value, half at another: y in {0, 65536}, the mean
    is midway and the standard deviation is half the gap, so z = +-1 exactly
    and v = (+-1 + c) / (2c); c = 0.5 clips to 0 and 1."""
    x = np.array([0.25, 0.75] * 500, np.float32)
    v = v_of(x, "zscore", 0.0, 2.0)
    assert np.array_equal(v[0::2], np.full(500, 0.25, np.float32))
    assert np.array_equal(v[1::2], np.full(500, 0.75, np.float32))
    v = v_of(x, "zscore", 0.0, 0.5)
    assert np.array_equal(v, np.array([0.0, 1.0] * 500, np.float32))


def test_zscore_three_points():
    """Scores 0, 1, 2 in equal numbers: y in {0, 32768, 65536}, variance
    (2/3) 2^30, z = -sqrt(3/2), 0, sqrt(3/2); with c = 3, v = (z + 3) / 6."""
    x = np.array([0.0, 1.0, 2.0] * 300, np.float32)
    v = v_of(x, "zscore", 0.0, 3.0)
    z = math.sqrt(1.5)
    np.testing.assert_allclose(v[0::3], (3 - z) / 6, rtol=1e-7)
    assert np.all(v[1::3] == np.float32(0.5))
    np.testing.assert_allclose(v[2::3], (3 + z) / 6, rtol=1e-7)


def test_zscore_outlier_is_clipped():
    """999 zeros and one 1: y = 0 (999 times) and 65536; the outlier's z is
    sqrt(999) > c = 3, so it is clipped to v = 1; each zero has
    z = -1/sqrt(999) and v = (3 - 1/sqrt(999)) / 6."""
    x = np.zeros(1000, np.float32)
    x[500] = 1.0
    v = v_of(x, "zscore", 0.0, 3.0)
    assert v[500] == 1.0
    others = np.delete(v, 500)
    np.testing.assert_allclose(others, (3 - 1 / math.sqrt(999)) / 6, rtol=1e-7)
    assert np.all(others == others[0])


def test_zscore_constant_scores():
    assert np.all(v_of(np.full(77, 0.3, np.float32), "zscore", 0.0, 3.0) == 1.0)
    assert np.all(v_of(np.full(1, 0.3, np.float32), "zscore", 0.0, 3.0) == 1.0)


def test_robust_norms_spread_the_ordinary_scores_under_an_outlier():
    """One extreme token: min-max leaves every other token below 0.011; the
    percentile clip (at the 1st and 99th percentiles) and the clipped z-score
    spread the ordinary tokens over most of [0, 1], and the outlier is 1."""
    rng = np.random.default_rng(7)
    x = (0.01 + 0.01 * rng.random(4096)).astype(np.float32)
    x[1000] = 1.0
    ordinary = np.ones(4096, bool)
    ordinary[1000] = False
    v_mm = v_of(x, "minmax")
    assert v_mm[1000] == 1.0 and v_mm[ordinary].max() < 0.011
    for v in (v_of(x, "percentile", 0.01, 0.99), v_of(x, "zscore", 0.0, 0.02)):
        assert v[1000] == 1.0
        assert v[ordinary].max() - v[ordinary].min() > 0.9


@pytest.mark.parametrize("norm,lo,hi", [("percentile", 0.5, 0.5), ("percentile", -0.1, 0.9),
                                        ("percentile", 0.1, 1.5), ("zscore", 0.0, 0.0),
                                        ("zscore", 0.1, 3.0), ("zscore", 0.0, -1.0),
                                        (7, 0.0, 1.0)])
def test_norm_parameters_rejected(norm, lo, hi):
    with pytest.raises(ValueError):
        oracle.select(np.ones(10, np.float32), 2, 1, "topk", keep_rate=0.5, norm=norm,
                      norm_lo=lo, norm_hi=hi)
