"""Pins for the oracle's entropy, max-over-decoded, decision and unmask choice.

Closed forms: uniform row -> log V; one-hot row -> 0; a two-level row, whose
entropy has the closed form log Z - a c e^c / Z (the identity H = LSE(z) - E_p[z],
not the -sum p log p the oracle evaluates).  Library routine: scipy's
entropy of scipy's softmax.  Invariants: shift and permutation invariance and
0 <= H <= log V.  Decision rule: strict ">" (EntropyCache (pt) §2 and (zh) §2.2
both send E <= tau to the partial pass).
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle.entropy import choose, decide, entropy_max, max_entropy, row_stats, softmax_entropy


@pytest.mark.parametrize("V", [1, 2, 7, 1024, 126464])
def test_uniform_row_has_entropy_log_v(V):
    H, a, p1 = softmax_entropy(np.full(V, 3.25))
    assert abs(H - math.log(V)) <= 1e-12 * max(1.0, math.log(V))
    assert a == 0
    assert abs(p1 - 1.0 / V) <= 1e-15


@pytest.mark.parametrize("V,hot", [(2, 0), (1024, 517), (152064, 152063)])
def test_one_hot_row_has_zero_entropy(V, hot):
    z = np.full(V, -1e4)
    z[hot] = 0.0
    H, a, p1 = softmax_entropy(z)
    assert H == 0.0 and a == hot and p1 == 1.0


@pytest.mark.parametrize("V,a,c", [(10, 3, 1.7), (1024, 1, 12.0), (126464, 40, -2.5), (5, 5, 0.3)])
def test_two_level_row_closed_form(V, a, c):
    z = np.zeros(V)
    z[:a] = c
    perm = np.random.default_rng(V).permutation(V)
    z = z[perm]
    Z = a * math.exp(c) + (V - a)
    H_closed = math.log(Z) - a * c * math.exp(c) / Z
    H, _, p1 = softmax_entropy(z)
    assert abs(H - H_closed) <= 1e-11
    assert abs(p1 - max(math.exp(c), 1.0) / Z) <= 1e-14


def test_matches_scipy_entropy_of_softmax():
    g = np.random.default_rng(1)
    for V in (3, 100, 5000):
        for s in (0.01, 1.0, 30.0):
            z = g.standard_normal(V) * s
            H, a, p1 = softmax_entropy(z)
            p = scipy.special.softmax(z)
            assert abs(H - scipy.stats.entropy(p)) <= 1e-10
            assert a == int(np.argmax(z))
            assert abs(p1 - p.max()) <= 1e-14


def test_invariants_shift_permutation_bounds():
    g = np.random.default_rng(2)
    z = g.standard_normal(777) * 4
    H0, a0, _ = softmax_entropy(z)
    H1, _, _ = softmax_entropy(z + 123.5)
    perm = g.permutation(777)
    H2, a2, _ = softmax_entropy(z[perm])
    assert abs(H0 - H1) < 1e-11 and abs(H0 - H2) < 1e-11
    assert perm[a2] == a0
    assert 0.0 <= H0 <= math.log(777)


def test_non_finite_logits():
    H, a, p1 = softmax_entropy([0.0, 0.0, -np.inf, -np.inf])
    assert abs(H - math.log(2)) < 1e-15 and a == 0 and p1 == 0.5
    H, a, p1 = softmax_entropy([np.nan, 1.0, 3.0, 3.0])
    assert math.isnan(H) and math.isnan(p1) and a == 2
    H, a, p1 = softmax_entropy([1.0, np.inf, 2.0])
    assert math.isnan(H) and a == 1
    H, a, p1 = softmax_entropy([-np.inf, -np.inf])
    assert math.isnan(H) and a == 0


def test_argmax_takes_the_lowest_index_on_ties():
    assert softmax_entropy([1.0, 3.0, 3.0, -2.0])[1] == 1
    assert softmax_entropy([5.0, 5.0])[1] == 0


def test_max_entropy_and_decision():
    H = np.array([0.5, 2.0, 1.0, np.nan])
    assert max_entropy(H, []) == -math.inf
    assert max_entropy(H, [0, 2]) == 1.0
    assert math.isnan(max_entropy(H, [1, 3]))
    assert decide(2.0, 2.0) == 0                       # E == tau -> partial
    assert decide(np.nextafter(2.0, 3.0), 2.0) == 1
    assert decide(math.nan, 2.0) == 1
    assert decide(-math.inf, -math.inf) == 0          # nothing decoded -> partial
    assert decide(0.0, -math.inf) == 1 and decide(50.0, math.inf) == 0


def test_entropy_max_over_all_rows():
    g = np.random.default_rng(3)
    z = g.standard_normal((6, 50)) * np.array([0.1, 1, 3, 10, 30, 100])[:, None]
    r = entropy_max(z, None, 2.0)
    H, _, _ = row_stats(z)
    assert r["E"] == H.max()
    assert r["flag"] == int(H.max() > 2.0)


def test_choose_top_p1_with_position_ties():
    pos = [10, 11, 12, 13]
    assert list(choose(pos, [0.5, 0.9, 0.9, 0.1], 1)) == [11]
    assert list(choose(pos, [0.5, 0.9, 0.9, 0.1], 2)) == [11, 12]
    assert list(choose(pos, [0.5, 0.9, 0.9, 0.1], 3)) == [10, 11, 12]
    assert list(choose([3, 1, 2], [0.9, 0.5, 0.9], 1)) == [2]     # tie -> lower position
    assert list(choose([4, 5], [np.nan, 0.2], 1)) == [5]
    assert list(choose([4, 5], [0.2, 0.3], 7)) == [4, 5]
    assert list(choose([], [], 2)) == []


def test_choose_matches_argsort_for_distinct_values():
    g = np.random.default_rng(4)
    for n in range(1, 10):
        p1 = g.random(20)
        pos = np.sort(g.choice(1000, 20, replace=False))
        want = np.sort(pos[np.argsort(-p1, kind="stable")[:n]])
        np.testing.assert_array_equal(choose(pos, p1, n), want)
