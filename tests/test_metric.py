"""The parity metric itself: max|x - ref| / RMS(ref) over a whole tensor (fp64), and its
streamed form.  Checked on arrays whose value is known in closed form."""
import math

import numpy as np
import pytest

import workloads as W


def test_known_value():
    ref = np.array([3.0, -4.0, 0.0, 0.0])              # RMS = sqrt(25 / 4) = 2.5
    x = ref + np.array([0.0, 0.5, -1.0, 0.25])         # max |diff| = 1.0
    assert W.rel_max_err(x, ref) == pytest.approx(1.0 / 2.5, rel=1e-15)


def test_max_is_over_every_element_and_rms_is_of_ref():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((7, 5, 3))
    x = ref.copy()
    x[6, 4, 2] += 1e-3                                  # the last element carries the error
    rms = math.sqrt(float(np.mean(ref ** 2)))
    assert W.rel_max_err(x, ref) == pytest.approx(1e-3 / rms, rel=1e-9)
    # the metric is not symmetric: it divides by the RMS of the reference only
    assert W.rel_max_err(ref, 10 * x) != W.rel_max_err(10 * x, ref)


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_result_is_infinite_error(bad):
    ref = np.ones(10)
    x = ref.copy()
    x[3] = bad
    assert W.rel_max_err(x, ref) == math.inf


def test_empty_and_zero_references():
    assert W.rel_max_err(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0
    assert W.rel_max_err(np.zeros(5), np.zeros(5)) == 0.0
    assert W.rel_max_err(np.full(5, 1e-30), np.zeros(5)) == math.inf


def test_shapes_must_match():
    with pytest.raises(ValueError):
        W.rel_max_err(np.zeros((4, 1, 3)), np.zeros((4, 2, 3)))   # would broadcast silently
    with pytest.raises(ValueError):
        W.ErrAccum().add(np.zeros(3), np.zeros(4))


def test_streamed_equals_whole():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((64, 6, 8))
    x = ref + 1e-4 * rng.standard_normal(ref.shape)
    acc = W.ErrAccum()
    for a in range(0, 64, 10):                         # ragged pieces along the token axis
        for h in range(0, 6, 4):
            acc.add(x[a:a + 10, h:h + 4], ref[a:a + 10, h:h + 4])
    assert acc.value() == pytest.approx(W.rel_max_err(x, ref), rel=1e-12)
    acc.add(np.array([np.nan]), np.array([1.0]))
    assert acc.value() == math.inf
    assert W.ErrAccum().value() == 0.0


def test_identity_bar_closed_form():
    from parity_helpers import identity_bar
    n = 400
    a, b = np.ones(n), np.full(n, 2.0)                  # RMS(a) = 1, |b| = 2 sqrt(n) = 40
    assert identity_bar([(a, b, 0.1)]) == pytest.approx(6 * 0.1 * 40.0, rel=1e-12)
    assert identity_bar([(a, b, 0.1), (np.zeros(0), np.zeros(0), 1.0)], sigmas=1) == pytest.approx(4.0)
    torch = pytest.importorskip("torch")
    assert identity_bar([(torch.ones(n), torch.full((n,), 2.0), 0.1)]) == pytest.approx(24.0, rel=1e-12)


def test_identity_bar_covers_independent_errors_and_not_a_wrong_block():
    """Independent errors of the stated size stay far inside the bar; replacing one block of a
    by a vector of the same norm and random direction lands far outside it."""
    from parity_helpers import identity_bar
    rng = np.random.default_rng(5)
    n = 200_000
    a, b = rng.standard_normal(n), rng.standard_normal(n)
    e = 1e-3
    a_err = a + e * rng.uniform(-1, 1, n)
    bar = identity_bar([(a, b, e)])
    assert abs(a_err @ b - a @ b) < bar / 2
    a_bad = a.copy()
    a_bad[:n // 96] = rng.standard_normal(n // 96)      # one "head" of 96 wrong
    assert abs(a_bad @ b - a @ b) > 3 * bar
