"""Pins of the CPU oracle to facts other than itself (CPU only).

Each group ties one oracle function to something a reader can check without
trusting the oracle: hand-worked closed forms (tests/golden), invariants that
characterise the result, brute force on tiny inputs, or a library routine
(torch SDPA in float64, scipy, numpy.percentile).
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O

RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------- storage ---

def test_decode_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0000, 0x8000, 0x7F7F, 0x0001], dtype=np.uint16)
    v = O.decode_bf16(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 3.140625
    assert v[3] == 0.0 and v[4] == 0.0 and np.signbit(v[4])
    assert v[5] == (2 - 2 ** -7) * 2.0 ** 127          # largest finite bf16
    assert v[6] == 2.0 ** -133                         # smallest subnormal bf16


# --------------------------------------------------------------- metadata ---

def test_golden_page_minmax(golden):
    c = golden["scores_and_selection"]
    K = np.array(c["keys"], dtype=np.float64)
    kmin, kmax = O.page_minmax(K, c["page_size"])
    assert np.array_equal(kmin, np.array(c["kmin"], dtype=np.float64))
    assert np.array_equal(kmax, np.array(c["kmax"], dtype=np.float64))


@pytest.mark.parametrize("L,ps", [(1, 8), (7, 8), (8, 8), (33, 16), (100, 16), (129, 64)])
def test_page_minmax_characterisation(L, ps):
    # kmin <= k <= kmax for every token of the page, and both bounds are attained.
    K = RNG.standard_normal((L, 5))
    kmin, kmax = O.page_minmax(K, ps)
    assert kmin.shape[0] == O.page_count(L, ps) == math.ceil(L / ps)
    for p in range(kmin.shape[0]):
        blk = K[p * ps:min(L, (p + 1) * ps)]
        assert np.all(blk >= kmin[p]) and np.all(blk <= kmax[p])
        assert np.all(np.any(blk == kmin[p], axis=0)) and np.all(np.any(blk == kmax[p], axis=0))


def test_partial_page_ignores_unwritten_slots():
    # A pool whose unwritten slots hold a poison value: the gathered page summary never sees it.
    ps, D, L = 8, 4, 13
    pool = np.full((3, 1, ps, D), 1000.0)
    pt = np.array([2, 0, 1])
    K = RNG.standard_normal((L, D))
    for t in range(L):
        pool[pt[t // ps], 0, t % ps] = K[t]
    Kg = O.gather_tokens(pool, pt, L, 0, ps)
    assert np.array_equal(Kg, K)
    kmin, kmax = O.page_minmax(Kg, ps)
    assert kmax.max() < 1000.0


def test_append_one_by_one_equals_bulk():
    ps, L, D = 16, 77, 6
    K = RNG.standard_normal((L, D))
    kmin_b, kmax_b = O.page_minmax(K, ps)
    P = O.page_count(L, ps)
    kmin = np.zeros((P, D))
    kmax = np.zeros((P, D))
    for t in range(L):
        p, slot = divmod(t, ps)
        kmin[p], kmax[p] = O.append_minmax(kmin[p], kmax[p], K[t], slot)
    assert np.array_equal(kmin, kmin_b) and np.array_equal(kmax, kmax_b)


def test_gather_is_permutation_invariant():
    ps, D, L = 4, 3, 18
    K = RNG.standard_normal((L, D))
    outs = []
    for seed in range(3):
        perm = np.random.default_rng(seed).permutation(6)
        pool = np.zeros((6, 1, ps, D))
        for t in range(L):
            pool[perm[t // ps], 0, t % ps] = K[t]
        outs.append(O.gather_tokens(pool, perm, L, 0, ps))
    for o in outs:
        assert np.array_equal(o, K)


# ---------------------------------------------------------------- scoring ---

def test_golden_scores(golden):
    c = golden["scores_and_selection"]
    q = np.array(c["group_queries"], dtype=np.float64)
    s = O.page_scores(q, np.array(c["kmin"], float), np.array(c["kmax"], float))
    assert np.array_equal(s, np.array(c["scores"]))


def _rand_pages(P, ps, D, G):
    K = RNG.standard_normal((P * ps, D))
    q = RNG.standard_normal((G, D))
    return K, q


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_score_is_upper_bound(G):
    ps, P, D = 16, 12, 32
    K, q = _rand_pages(P, ps, D, G)
    kmin, kmax = O.page_minmax(K, ps)
    s = O.page_scores(q, kmin, kmax)
    for p in range(P):
        logits = K[p * ps:(p + 1) * ps] @ q.T          # [tokens][G]
        per_head_max = logits.max(axis=0).sum()       # sum_h max_t q_h.k_t
        joint_max = logits.sum(axis=1).max()          # max_t sum_h q_h.k_t
        assert s[p] >= per_head_max - 1e-12 >= joint_max - 2e-12


def test_score_tight_for_single_token_pages():
    K, q = _rand_pages(9, 1, 16, 4)
    kmin, kmax = O.page_minmax(K, 1)
    s = O.page_scores(q, kmin, kmax)
    np.testing.assert_allclose(s, (K @ q.T).sum(axis=1), rtol=0, atol=1e-12)


def test_score_sign_split_identity():
    # sum_h max(q*kmax, q*kmin) == kmax*sum_h max(q,0) + kmin*sum_h min(q,0) because kmax >= kmin.
    K, q = _rand_pages(20, 16, 64, 4)
    kmin, kmax = O.page_minmax(K, 16)
    s = O.page_scores(q, kmin, kmax)
    alt = kmax @ np.maximum(q, 0).sum(axis=0) + kmin @ np.minimum(q, 0).sum(axis=0)
    np.testing.assert_allclose(s, alt, rtol=1e-13, atol=1e-12)


def test_score_scales_exactly_with_power_of_two_queries():
    K, q = _rand_pages(10, 8, 16, 2)
    kmin, kmax = O.page_minmax(K, 8)
    s1 = O.page_scores(q, kmin, kmax)
    s4 = O.page_scores(4.0 * q, kmin, kmax)
    assert np.array_equal(4.0 * s1, s4)


# -------------------------------------------------------------- selection ---

def test_golden_selection(golden):
    for key in ("scores_and_selection", "selection_ties"):
        c = golden[key]
        for budget, want in c["selection"].items():
            got = O.select_pages(np.array(c["scores"]), int(budget))
            assert got.tolist() == want, (key, budget)


def _beats(s, i, j):
    return s[i] > s[j] or (s[i] == s[j] and i < j)


@pytest.mark.parametrize("trial", range(40))
def test_selection_brute_force(trial):
    r = np.random.default_rng(1000 + trial)
    P = int(r.integers(3, 11))
    s = r.integers(-3, 4, size=P).astype(np.float64)  # small range: many ties
    K = int(r.integers(2, P))
    got = O.select_pages(s, K)
    middle = range(1, P - 1)
    valid = []
    for sub in itertools.combinations(middle, K - 2):
        rest = [j for j in middle if j not in sub]
        if all(_beats(s, i, j) for i in sub for j in rest):
            valid.append(sorted([0, P - 1, *sub]))
    assert len(valid) == 1
    assert got.tolist() == valid[0]


def test_selection_edge_cases():
    assert O.select_pages(np.array([3.0]), 16).tolist() == [0]
    assert O.select_pages(np.array([3.0, -1.0]), 16).tolist() == [0, 1]
    s = np.array([-9.0, 5.0, 4.0, 3.0, -9.0])
    assert O.select_pages(s, 2).tolist() == [0, 4]          # forced pages despite lowest scores
    assert O.select_pages(s, 0).tolist() == [0, 4]          # budget below 2 still keeps sink + local
    assert O.select_pages(s, 5).tolist() == [0, 1, 2, 3, 4]
    assert O.select_pages(s, 100).tolist() == [0, 1, 2, 3, 4]


# -------------------------------------------------------------- attention ---

def _sdpa(q, K, V, scale, mask=None):
    qt = torch.from_numpy(q)[None, None, None, :]
    kt = torch.from_numpy(K)[None, None]
    vt = torch.from_numpy(V)[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)[0, 0, 0].numpy()


@pytest.mark.parametrize("L,D", [(1, 8), (37, 64), (300, 128)])
def test_attention_matches_torch_sdpa(L, D):
    q = RNG.standard_normal(D)
    K = RNG.standard_normal((L, D))
    V = RNG.standard_normal((L, D))
    scale = 1.0 / math.sqrt(D)
    o, lse = O.attention(q, K, V, scale)
    np.testing.assert_allclose(o, _sdpa(q, K, V, scale), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(scale * (K @ q)), rtol=1e-13)


def test_sparse_decode_matches_masked_sdpa():
    ps, L, D, G = 16, 200, 32, 2
    K = RNG.standard_normal((L, D))
    V = RNG.standard_normal((L, D))
    q = RNG.standard_normal((G, D))
    o, lse, pages = O.sparse_decode_unit(q, K, V, ps, 5, 1 / math.sqrt(D))
    mask = np.zeros(L, dtype=bool)
    mask[O.tokens_of_pages(pages, L, ps)] = True
    assert pages[0] == 0 and pages[-1] == O.page_count(L, ps) - 1 and len(pages) == 5
    for h in range(G):
        np.testing.assert_allclose(o[h], _sdpa(q[h], K, V, 1 / math.sqrt(D), mask), rtol=1e-12, atol=1e-12)


def test_golden_attention(golden):
    c = golden["attention_two_tokens"]
    o, lse = O.attention(np.array(c["q"]), np.array(c["keys"]), np.array(c["values"]), math.log(3))
    np.testing.assert_allclose(o, c["out"], rtol=0, atol=1e-14)
    assert abs(lse - math.log(4)) < 1e-14


def test_attention_closed_forms():
    D = 16
    V = RNG.standard_normal((5, D))
    q = RNG.standard_normal(D)
    o, lse = O.attention(q, V[:1] * 0 + 1.0, V[:1], 0.25)           # one token: o = v0
    assert np.array_equal(o, V[0]) and abs(lse - 0.25 * q.sum()) < 1e-14
    Kid = np.tile(RNG.standard_normal(D), (5, 1))                  # identical keys: mean of V
    o, lse = O.attention(q, Kid, V, 0.3)
    np.testing.assert_allclose(o, V.mean(axis=0), rtol=1e-13, atol=1e-14)
    Vc = np.full((5, D), 2.5)                                     # constant V: that constant
    o, _ = O.attention(q, RNG.standard_normal((5, D)), Vc, 0.3)
    np.testing.assert_allclose(o, Vc[0], rtol=1e-14)


def test_empty_sequence_conventions():
    # no token: the sum of weights is empty (0), so lse = ln 0 and the output is taken as zeros;
    # the empty sequence keeps no page and scores none
    D = 8
    o, lse = O.attention(RNG.standard_normal(D), np.zeros((0, D)), np.zeros((0, D)), 0.5)
    assert np.array_equal(o, np.zeros(D)) and lse == -np.inf
    kmin, kmax = O.page_minmax(np.zeros((0, D)), 16)
    assert kmin.shape == (0, D) and O.select_pages(O.page_scores(np.ones((2, D)), kmin, kmax), 5).size == 0
    o, lse = O.dense_decode_unit(np.ones((2, D)), np.zeros((0, D)), np.zeros((0, D)), 16, 0.5)
    assert np.array_equal(o, np.zeros((2, D))) and np.all(lse == -np.inf)
    # the convention is the identity of the log-sum-exp merge: adding the empty set changes nothing
    K, V = RNG.standard_normal((5, D)), RNG.standard_normal((5, D))
    q = RNG.standard_normal(D)
    full = O.attention(q, K, V, 0.5)
    o, lse = O.lse_merge([full, O.attention(q, K[:0], V[:0], 0.5)])
    assert np.array_equal(o, full[0]) and lse == full[1]


def test_lse_merge_of_splits_equals_unsplit():
    L, D = 97, 32
    q = RNG.standard_normal(D)
    K = RNG.standard_normal((L, D)) * 3
    V = RNG.standard_normal((L, D))
    full = O.attention(q, K, V, 0.2)
    cuts = [0, 10, 11, 50, 97]
    parts = [O.attention(q, K[a:b], V[a:b], 0.2) for a, b in zip(cuts, cuts[1:])]
    o, lse = O.lse_merge(parts)
    np.testing.assert_allclose(o, full[0], rtol=1e-12, atol=1e-12)
    assert abs(lse - full[1]) < 1e-12


def test_full_budget_sparse_equals_dense():
    ps, L, D, G = 16, 150, 64, 4
    K = RNG.standard_normal((L, D))
    V = RNG.standard_normal((L, D))
    q = RNG.standard_normal((G, D))
    o_s, lse_s, pages = O.sparse_decode_unit(q, K, V, ps, O.page_count(L, ps), 0.125)
    o_d, lse_d = O.dense_decode_unit(q, K, V, ps, 0.125)
    assert np.array_equal(o_s, o_d) and np.array_equal(lse_s, lse_d)


# ------------------------------------------------------------- acceptance ---

def test_golden_acceptance(golden):
    a = np.array([math.log(3), 0.0])
    b = np.array(golden["acceptance_two_outcomes"]["b"])
    assert abs(O.acceptance(a, b, 1.0) - 0.75) < 1e-15
    assert abs(O.acceptance(a, b, 2.0) - (0.5 + 1 / (math.sqrt(3) + 1))) < 1e-15


def test_acceptance_invariants():
    a = RNG.standard_normal(1000) * 3
    b = a + RNG.standard_normal(1000) * 0.3
    assert abs(O.acceptance(a, a) - 1.0) < 1e-14                   # identical rows
    assert abs(O.acceptance(a, a + 17.25) - 1.0) < 1e-12         # shift invariance
    x, y = O.acceptance(a, b, 1.3), O.acceptance(b, a, 1.3)
    assert abs(x - y) < 1e-15                                      # symmetry
    assert 0.0 <= x <= 1.0
    assert abs(x - (1 - O.total_variation(a, b, 1.3))) < 1e-12     # alpha = 1 - TV
    assert O.acceptance(a, b, 1e6) > 1 - 1e-4                      # T -> inf: both uniform
    p = scipy.special.softmax(a / 1.3)
    q = scipy.special.softmax(b / 1.3)
    assert abs(x - np.minimum(p, q).sum()) < 1e-12


@pytest.mark.parametrize("s,r", [(0.1, 0.7), (0.5, 0.5), (0.99, 0.01)])
def test_acceptance_two_outcome_closed_form(s, r):
    a = np.log([s, 1 - s])
    b = np.log([r, 1 - r]) + 3.0
    assert abs(O.acceptance(a, b) - (1 - abs(s - r))) < 1e-14


def test_acceptance_disjoint_support_is_small():
    a = np.array([50.0, 0.0, 0.0])
    b = np.array([0.0, 0.0, 50.0])
    assert O.acceptance(a, b) < 1e-20


def test_golden_tail_stats(golden):
    c = golden["percentile"]
    mean, p5 = O.tail_stats(c["values"])
    assert abs(p5 - c["p5"]) < 1e-15 and abs(mean - c["mean"]) < 1e-15


@pytest.mark.parametrize("n", [1, 2, 3, 64, 1000])
def test_tail_stats_matches_numpy(n):
    x = RNG.random(n)
    mean, p5 = O.tail_stats(x)
    assert abs(p5 - np.percentile(x, 5)) < 1e-15
    assert abs(mean - np.mean(x)) < 1e-15


def test_monitor_window_hand_worked():
    """A window of 5 after appending [0.9, 0.8] then [0.7, 0.95, 0.99, 0.5]: the last five values
    0.8, 0.7, 0.95, 0.99, 0.5; sorted 0.5, 0.7, 0.8, 0.95, 0.99; rank 0.05 * 4 = 0.2 gives
    0.5 + 0.2 * (0.7 - 0.5) = 0.54; mean 3.94 / 5 = 0.788."""
    w = O.monitor_window([np.array([0.9, 0.8]), np.array([0.7, 0.95, 0.99, 0.5])], 5)
    assert w.tolist() == [0.8, 0.7, 0.95, 0.99, 0.5]
    mean, p5 = O.tail_stats(w)
    assert abs(mean - 0.788) < 1e-15 and abs(p5 - 0.54) < 1e-15
    # fewer values than the window holds: all of them; a batch longer than the window: its tail
    assert O.monitor_window([np.array([0.3])], 5).tolist() == [0.3]
    assert O.monitor_window([np.arange(10.0)], 3).tolist() == [7.0, 8.0, 9.0]
    assert O.monitor_window([], 3).shape == (0,)
