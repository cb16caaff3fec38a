"""Pins of the oracle's output metrics and of its weighted combine.

The tolerance on GEMM outputs is max relative error 1e-2 and RMS relative error
2e-3, both normwise over one output tensor (max|y - r| / max|r| and
||y - r|| / ||r||).  The vectors below are built from powers of two so that every
expected figure is exact; each case is chosen so that a plausible slip in the
metric (dividing by max|y| instead of max|r|, an element-wise relative error,
a mean of ratios in place of the norm ratio) gives a different number.

The combine is pinned from its definition, y[t] = sum over slots j of
w[t, j] * o[inv[t*k + j]]: with one-hot rows o[s] = e_s every output entry is a
single weight, so any mis-pairing of slot, weight or token moves a value."""

import math

import numpy as np
import pytest

import oracle
from oracle.moe import combine


def test_normwise_single_perturbation():
    ref = np.array([1.0, -2.0, 4.0, 0.0])
    y = ref.copy()
    y[0] += 0.5                      # error at the smallest non-zero element
    mx, rms = oracle.normwise_errors(y, ref)
    assert mx == 0.5 / 4.0           # normwise: over max|ref| = 4, not over |ref_0| = 1
    assert rms == 0.5 / math.sqrt(21.0)
    assert mx != 0.5                 # an element-wise relative error would give 0.5
    # the error on the largest element: dividing by max|y| (4.5) would differ
    y = ref.copy()
    y[2] += 0.5
    mx, rms = oracle.normwise_errors(y, ref)
    assert mx == 0.125 and mx != 0.5 / 4.5
    assert rms == 0.5 / math.sqrt(21.0)


def test_normwise_two_errors_norm_ratio():
    ref = np.array([3.0, 4.0])
    y = np.array([3.0 - 0.25, 4.0 + 0.5])
    mx, rms = oracle.normwise_errors(y, ref)
    assert mx == 0.5 / 4.0
    assert rms == math.sqrt(0.25 ** 2 + 0.5 ** 2) / 5.0
    mean_of_ratios = np.mean(np.abs(y - ref) / np.abs(ref))
    assert rms != mean_of_ratios


def test_normwise_scale_invariant_and_shape_free():
    rng = np.random.default_rng(7)
    ref = rng.standard_normal((5, 7))
    y = ref + rng.standard_normal((5, 7)) * 1e-3
    base = oracle.normwise_errors(y, ref)
    for e in (-40, -3, 17, 60):
        s = 2.0 ** e                  # exact scaling: identical figures
        assert oracle.normwise_errors(y * s, ref * s) == base
    assert oracle.normwise_errors(y.ravel(), ref.ravel()) == base


def test_normwise_zero_reference_is_absolute():
    ref = np.zeros(3)
    y = np.array([0.0, -0.5, 0.25])
    mx, rms = oracle.normwise_errors(y, ref)
    assert mx == 0.5
    assert rms == math.sqrt(0.25 + 0.0625)
    assert oracle.normwise_errors(ref, ref) == (0.0, 0.0)


def test_within_tolerance_boundaries():
    ref = np.array([3.0, 4.0] + [0.0] * 6)
    # max_rel exactly 2^-7 < 1e-2, rms_rel = 2^-5 / 5 = 6.25e-3 > 2e-3: fails on rms
    y = ref.copy()
    y[1] += 2.0 ** -5
    ok, mx, rms = oracle.within_tolerance(y, ref)
    assert (mx, rms) == (2.0 ** -7, 2.0 ** -5 / 5.0) and not ok
    # a larger reference norm with the same error passes both
    ref2 = np.full(400, 4.0)
    y2 = ref2.copy()
    y2[0] += 2.0 ** -5
    ok2, mx2, rms2 = oracle.within_tolerance(y2, ref2)
    assert mx2 == 2.0 ** -7 and rms2 == 2.0 ** -5 / 80.0 and ok2
    # max_rel just above 1e-2 fails even with a tiny rms
    y3 = ref2.copy()
    y3[0] += 4.0 * 0.0101
    ok3, mx3, _ = oracle.within_tolerance(y3, ref2)
    assert mx3 > oracle.MAX_REL_TOL and not ok3
    # the bounds themselves are the stated ones
    assert oracle.MAX_REL_TOL == 1e-2 and oracle.RMS_REL_TOL == 2e-3


def test_normwise_rejects_shape_mismatch():
    with pytest.raises(AssertionError):
        oracle.normwise_errors(np.zeros(3), np.zeros(4))


@pytest.mark.parametrize("T,k", [(3, 2), (5, 3), (4, 8)])
def test_combine_one_hot_pairing(T, k):
    rng = np.random.default_rng(100 + 10 * T + k)
    R = T * k
    inv = rng.permutation(R).astype(np.int32)           # routed row -> sorted position
    o = np.eye(R)                                       # sorted position s -> e_s
    # distinct powers of two: exact, and no weight equals another
    w = np.exp2(-np.arange(1, R + 1, dtype=np.float64)).reshape(T, k)
    w = w[:, rng.permutation(k)]
    y = combine(o, inv, w)
    expect = np.zeros((T, R))
    for t in range(T):
        for j in range(k):
            expect[t, inv[t * k + j]] = w[t, j]
    assert np.array_equal(y, expect)
    # the slips a combine can make change the result: weights paired with the
    # next slot, or the rows of another token
    assert not np.array_equal(combine(o, inv, np.roll(w, 1, axis=1)), expect)
    assert not np.array_equal(combine(o, np.roll(inv, k), w), expect)


def test_combine_sums_in_slot_order():
    # three slots whose fp64 sum depends on the order: 2^53 + 1 rounds to 2^53
    big = 2.0 ** 53
    o = np.array([[big], [-big], [1.0]])
    w = np.ones((1, 3))
    assert combine(o, np.array([0, 1, 2]), w)[0, 0] == 1.0      # (big - big) + 1
    assert combine(o, np.array([0, 2, 1]), w)[0, 0] == 0.0      # (big + 1) - big
