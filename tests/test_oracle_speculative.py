"""Pins for the verification / speculative-sampling oracle (CPU only).

Each check ties the oracle to something other than itself: torch's
scaled-dot-product attention (fp64, explicit causal mask) for the multi-query
verification, numpy's searchsorted for the inverse-CDF draw, and the defining
property of exact speculative sampling (the emitted token follows the
verifier's distribution) by exhaustive enumeration on a tiny vocabulary.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------ verify attention ---

@pytest.mark.parametrize("T,G,L,D", [(1, 2, 37, 16), (7, 4, 50, 32), (3, 1, 3, 8), (8, 8, 200, 64)])
def test_verify_matches_torch_sdpa_with_causal_mask(T, G, L, D):
    r = _rng(T * 100 + L)
    q = r.standard_normal((T, G, D))
    K = r.standard_normal((L, D))
    V = r.standard_normal((L, D))
    scale = 1.0 / math.sqrt(D)
    out, lse = O.verify_decode_unit(q, K, V, scale)
    # torch reference: rows (t, h) against all L tokens with a boolean mask that
    # lets position t see tokens 0 .. L - T + t
    qt = torch.from_numpy(q.reshape(T * G, D))[None, None]
    Kt = torch.from_numpy(K)[None, None]
    Vt = torch.from_numpy(V)[None, None]
    vis = np.zeros((T * G, L), dtype=bool)
    for t in range(T):
        vis[t * G:(t + 1) * G, :L - T + t + 1] = True
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=torch.from_numpy(vis)[None, None],
                                                           scale=scale)[0, 0].numpy().reshape(T, G, D)
    assert np.abs(out - ref).max() < 1e-12
    # lse against a direct log-sum-exp of the visible logits (scipy-free)
    z = scale * (q.reshape(T * G, D) @ K.T)
    z = np.where(vis, z, -np.inf)
    zmax = z.max(axis=1, keepdims=True)
    lse_ref = (zmax[:, 0] + np.log(np.exp(z - zmax).sum(axis=1))).reshape(T, G)
    assert np.abs(lse - lse_ref).max() < 1e-12


def test_verify_is_causal_and_last_row_is_dense():
    r = _rng(5)
    T, G, L, D = 5, 2, 40, 16
    q = r.standard_normal((T, G, D))
    K = r.standard_normal((L, D))
    V = r.standard_normal((L, D))
    out, _ = O.verify_decode_unit(q, K, V, 0.25)
    # perturb the token right after row 1's last visible position (L - T + 1)
    K2, V2 = K.copy(), V.copy()
    K2[L - T + 2] += 3.0
    V2[L - T + 2] -= 2.0
    out2, _ = O.verify_decode_unit(q, K2, V2, 0.25)
    assert np.array_equal(out[:2], out2[:2])           # rows 0, 1 do not see it
    assert np.abs(out[2:] - out2[2:]).min() > 0.0      # rows 2.. do
    # the last row sees every token: equal to dense decode (pages of 8)
    dense, _ = O.dense_decode_unit(q[T - 1], K, V, 8, 0.25)
    assert np.abs(out[T - 1] - dense).max() < 1e-12


# ------------------------------------------------------- inverse CDF draw ---

def test_inverse_cdf_matches_searchsorted():
    r = _rng(7)
    for trial in range(200):
        V = int(r.integers(1, 40))
        w = r.random(V) * (r.random(V) < 0.7)
        if w.sum() == 0:
            w[int(r.integers(V))] = 1.0
        u = float(r.random())
        v = O.inverse_cdf_draw(w, u)
        ref = int(np.searchsorted(np.cumsum(w), u * w.sum(), side="right"))
        assert v == ref and w[v] > 0, (trial, v, ref)


def test_inverse_cdf_edges():
    w = np.array([0.0, 0.0, 2.0, 0.0, 1.0, 0.0])
    assert O.inverse_cdf_draw(w, 0.0) == 2           # first token with weight
    assert O.inverse_cdf_draw(w, 0.6666) == 2
    assert O.inverse_cdf_draw(w, 0.6667) == 4
    assert O.inverse_cdf_draw(w, 0.999999) == 4      # never a zero-weight token


# --------------------------------------------------- speculative sampling ---

def _grid(n):
    return (np.arange(n) + 0.5) / n  # midpoints of n equal cells of [0, 1)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_emitted_token_follows_verifier_distribution(seed):
    """k = 1: P(emit v) = sum_x q(x) [P(keep | x) 1{v = x} + P(reject | x) r(v)] must equal p(v).

    P(keep | x) integrates the oracle's accept test over a fine grid of
    u_accept, and the token after a rejection integrates the oracle's draw over
    a fine grid of u_sample; no formula of the method is retyped here.
    """
    r = _rng(seed)
    Vs = 6
    a = r.standard_normal((2, Vs)) * 1.5
    b = r.standard_normal((1, Vs)) * 1.5
    p = O.softmax_t(a[0], 1.0)
    q = O.softmax_t(b[0], 1.0)
    n = 4000
    emit = np.zeros(Vs)
    for x in range(Vs):
        kept = 0
        rejected_tokens = np.zeros(Vs)
        for ua in _grid(n):
            m, tok = O.speculative_accept(a, b, [x], [ua], 0.5)
            if m == 1:
                kept += 1
        emit[x] += q[x] * kept / n
        # the token drawn after a rejection at position 0 (u_accept = 1 - tiny forces the rejection
        # whenever rejection is possible at all)
        if kept < n:
            for us in _grid(n):
                m, tok = O.speculative_accept(a, b, [x], [1.0 - 1e-12], us)
                assert m == 0
                rejected_tokens[tok] += 1.0 / n
            emit += q[x] * (1 - kept / n) * rejected_tokens
    assert np.abs(emit - p).max() < 2e-3, (emit, p)


def test_identical_distributions_keep_every_draft():
    r = _rng(11)
    k, Vs = 6, 50
    logits = r.standard_normal((k + 1, Vs)) * 2
    draft = [int(r.integers(Vs)) for _ in range(k)]
    u = r.random(k) * 0.999999
    us = float(r.random())
    m, tok = O.speculative_accept(logits, logits[:k].copy(), draft, u, us)
    assert m == k
    pk = O.softmax_t(logits[k], 1.0)
    assert tok == int(np.searchsorted(np.cumsum(pk), us * pk.sum(), side="right"))


def test_rejection_draws_from_positive_residual_only():
    # drafter puts almost all mass on token 0, verifier almost none: position 0 is rejected and
    # the replacement is never token 0 (its residual max(0, p - q) is zero)
    Vs = 8
    a = np.zeros((3, Vs))
    a[0, 0] = -20.0
    b = np.zeros((2, Vs))
    b[0, 0] = 20.0
    for us in _grid(97):
        m, tok = O.speculative_accept(a, b, [0, 3], [0.5, 0.5], us)
        assert m == 0 and tok != 0


def test_rejection_with_no_residual_mass_draws_from_verifier():
    # identical distributions and an accept uniform of 1 (one past the documented range, which forces the
    # rejection): the residual max(0, p - q) is 0 everywhere, so the token is drawn from p itself, exactly as an
    # inverse-CDF draw over p (searchsorted on its cumulative sums) gives it
    r = _rng(11)
    a = r.standard_normal((2, 12))
    p = np.exp(a[0] - a[0].max())
    p /= p.sum()
    cdf = np.cumsum(p)
    for us in _grid(61):
        m, tok = O.speculative_accept(a, a[:1].copy(), [5], [1.0], us)
        assert m == 0
        assert tok == int(np.searchsorted(cdf, us * cdf[-1], side="right"))


def test_temperature_divides_logits():
    r = _rng(3)
    a = r.standard_normal((2, 10))
    b = r.standard_normal((1, 10))
    got = [O.speculative_accept(a, b, [4], [ua], 0.37, temperature=2.0) for ua in _grid(50)]
    ref = [O.speculative_accept(a / 2.0, b / 2.0, [4], [ua], 0.37) for ua in _grid(50)]
    assert got == ref
