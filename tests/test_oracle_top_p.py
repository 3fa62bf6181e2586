"""Pins for the score-mass (top-p) page selection oracle (CPU only).

Checked against what the rule must give independently of how the oracle
walks the pages: hand-worked cases, exhaustive search for the smallest page
set reaching the mass on tiny inputs, the Top-B selection when the cap binds,
and monotonicity in p.
"""
import itertools

import numpy as np
import pytest

import oracle as O
from oracle import top_p as TP


def test_equal_scores_hand_worked():
    # ten equal scores: every mass 1, total 10, target 5.5 -> six pages; ties to the lower index
    got = TP.select_pages_top_p(np.zeros(10), 0.55, 1.0, cap=100)
    assert got.tolist() == [0, 1, 2, 3, 4, 9]


def test_full_mass_keeps_every_page():
    got = TP.select_pages_top_p(np.arange(12, dtype=float), 1.0, 0.0, cap=100)   # c = 0: all masses 1
    assert got.tolist() == list(range(12))


def test_one_dominant_page():
    s = np.zeros(20)
    s[7] = 100.0
    for p in (0.1, 0.5, 0.99):
        assert TP.select_pages_top_p(s, p, 1.0, cap=100).tolist() == [0, 7, 19]


def test_short_lists_keep_everything():
    assert TP.select_pages_top_p(np.array([3.0]), 0.1, 1.0, cap=8).tolist() == [0]
    assert TP.select_pages_top_p(np.array([3.0, -1.0]), 0.1, 1.0, cap=8).tolist() == [0, 1]


@pytest.mark.parametrize("seed", range(40))
def test_smallest_set_by_exhaustive_search(seed):
    r = np.random.default_rng(seed)
    P = int(r.integers(3, 9))
    s = np.round(r.normal(0, 2, P), 1)          # rounded: some exact ties
    c = float(r.uniform(0.2, 2.0))
    p = float(r.uniform(0.05, 0.999))
    got = TP.select_pages_top_p(s, p, c, cap=100)
    w = np.exp(c * (s - s.max()))
    target = p * w.sum()
    middle = list(range(1, P - 1))
    # smallest number of middle pages whose best choice reaches the target
    best = None
    for k in range(len(middle) + 1):
        reach = [sub for sub in itertools.combinations(middle, k) if w[0] + w[P - 1] + w[list(sub)].sum() >= target * (1 - 1e-12)]
        if reach:
            best = k
            break
    assert best is not None
    assert len(got) == best + 2
    # the kept middle pages carry the largest masses available for that count
    kept = [i for i in got.tolist() if 0 < i < P - 1]
    assert np.isclose(w[kept].sum(), np.sort(w[middle])[::-1][:best].sum(), rtol=1e-12, atol=0)


@pytest.mark.parametrize("cap", [2, 3, 5, 9])
def test_cap_gives_top_b(cap):
    r = np.random.default_rng(cap)
    s = r.normal(0, 1, 30)
    got = TP.select_pages_top_p(s, 0.999, 0.05, cap=cap)      # flat masses: the cap binds
    assert got.tolist() == O.select_pages(s, cap).tolist()


def test_monotone_in_p():
    r = np.random.default_rng(3)
    s = r.normal(0, 3, 200)
    sizes = [len(TP.select_pages_top_p(s, p, 0.7, cap=1000)) for p in np.linspace(0.01, 1.0, 60)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))
    prev = set()
    for p in np.linspace(0.01, 1.0, 60):
        cur = set(TP.select_pages_top_p(s, p, 0.7, cap=1000).tolist())
        assert prev <= cur
        prev = cur
