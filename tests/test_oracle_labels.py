"""Pins for the label-distribution oracle (oracle/labels.py): the closed cases
the tutorial states for confidence, the logistic function for two labels,
scipy's softmax and entropy, shift invariance and stability."""
import math

import numpy as np
import pytest
from scipy.special import expit, softmax
from scipy.stats import entropy

from oracle import labels as L


def test_uniform_logits_give_zero_confidence_and_middle_score():
    # tutorial, "interpret confidence carefully": equal probabilities -> confidence 0
    for n in (2, 5, 64):
        row = np.full(100, 3.25)
        p = L.distribution(row, range(n))
        assert np.allclose(p, 1.0 / n, rtol=0, atol=1e-15)
        assert abs(L.confidence(p)) < 1e-12
        assert abs(L.expected_index(p) - (n - 1) / 2) < 1e-12
        assert L.choice(row, range(n)) == 0  # all tied: the first label


def test_point_mass_gives_confidence_one():
    # same passage: a point mass -> confidence 1
    row = np.zeros(70)
    row[33] = 2000.0
    ids = list(range(20, 60))
    p = L.distribution(row, ids)
    assert L.choice(row, ids) == 13 and p[13] == 1.0
    assert L.confidence(p) == 1.0
    assert L.expected_index(p) == 13.0


def test_two_labels_are_the_logistic_of_the_difference():
    # Bool: p(yes) = 1 / (1 + exp(l_no - l_yes))
    g = np.random.default_rng(0)
    for _ in range(50):
        row = g.normal(0, 4, 10)
        p = L.distribution(row, [7, 2])
        assert abs(p[0] - expit(row[7] - row[2])) < 1e-14


@pytest.mark.parametrize("n", [1, 3, 17, 64])
def test_matches_scipy_softmax_and_entropy(n):
    g = np.random.default_rng(n)
    row = g.normal(0, 3, 300)
    ids = g.choice(300, n, replace=False)
    p = L.distribution(row, ids)
    assert np.allclose(p, softmax(row[ids]), rtol=1e-13, atol=1e-15)
    want = 1.0 if n == 1 else 1.0 - entropy(softmax(row[ids])) / math.log(n)
    assert abs(L.confidence(p) - want) < 1e-12
    assert L.choice(row, ids) == int(np.argmax(row[ids]))


def test_shift_invariant_and_stable_for_huge_logits():
    g = np.random.default_rng(3)
    row = g.normal(0, 2, 64)
    ids = list(range(64))
    p0 = L.distribution(row, ids)
    p1 = L.distribution(row + 1e5, ids)  # exp(1e5) overflows: only a stable softmax survives
    assert np.all(np.isfinite(p1)) and np.allclose(p0, p1, rtol=1e-9)


def test_rows_with_fewer_options_use_the_first_labels():
    g = np.random.default_rng(4)
    logits = g.normal(0, 3, (3, 500))
    ids = list(g.choice(500, 8, replace=False))
    probs, ch, ex, cf = L.classify(logits, ids, counts=[8, 2, 1])
    assert np.allclose(probs.sum(1), 1.0)
    assert np.all(probs[1, 2:] == 0) and np.all(probs[2, 1:] == 0) and probs[2, 0] == 1.0
    assert abs(probs[1, 0] - expit(logits[1, ids[0]] - logits[1, ids[1]])) < 1e-14
    assert cf[2] == 1.0 and ch[2] == 0 and ex[2] == 0.0
