"""GPU parity of exact speculative sampling (spdec_spec_accept) against the oracle.

The kept-draft count and the emitted token are integers decided by floating
point: they must equal the oracle's except where the oracle's own fp64 margin
is within fp32 rounding (an accept test u*q(x) vs p(x) closer than 1e-4
relative, or a draw whose target lies within 2e-5 of the total of a token
boundary); such sequences are counted and must stay rare, and a draw inside
the band must still land on a token adjacent to the boundary with positive
weight.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_decode_page_amd import spdec

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

ACCEPT_BAND = 1e-4
DRAW_BAND = 2e-5


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(spdec.LIB_PATH):
        from sparse_attention_decode_page_amd import build
        build.build()
    spdec.lib()
    assert torch.cuda.is_available()


def _inputs(B, k, V, seed, sigma=2.0, noise=0.5, same=False, temperature=1.0):
    r = np.random.default_rng(seed)
    p = (sigma * r.standard_normal((B, k + 1, V))).astype(np.float32)
    q = p[:, :k] if same else (p[:, :k] + noise * r.standard_normal((B, k, V))).astype(np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    draft = np.zeros((B, k), dtype=np.int32)
    for b in range(B):
        for i in range(k):  # drafts drawn from the drafter's distribution (test-side input generation)
            draft[b, i] = r.choice(V, p=O.softmax_t(q[b, i], temperature))
    ua = r.random((B, k)).astype(np.float32)
    us = r.random(B).astype(np.float32)
    return p, q, draft, ua, us


def _draw_weights(p, q, n, k, temperature):
    """The weights the emitted token is drawn from after n kept drafts (the oracle's reading: a residual with no
    mass draws from p_n)."""
    pp = O.softmax_t(p[n], temperature)
    if n == k:
        return pp
    w = np.maximum(pp - O.softmax_t(q[n], temperature), 0.0)
    return w if w.sum() > 0.0 else pp


def _band_consistent(p, q, draft, ua, temperature, n_gpu, tok_gpu, i_band):
    """The GPU took an accept decision inside the fp32/fp64 band at position i_band: every decision outside the
    band must still match, and the token must carry weight in the row the GPU's count implies."""
    k = draft.shape[0]
    assert i_band <= n_gpu <= k, (i_band, n_gpu)
    for j in range(k):
        if j == i_band or j > n_gpu:
            continue
        pp = O.softmax_t(p[j], temperature)
        qq = O.softmax_t(q[j], temperature)
        x = int(draft[j])
        lhs, rhs = float(ua[j]) * qq[x], pp[x]
        if abs(lhs - rhs) <= ACCEPT_BAND * max(lhs, rhs, 1e-30):
            continue
        assert (lhs < rhs) == (j < n_gpu), (j, n_gpu, lhs, rhs)
    w = _draw_weights(p, q, n_gpu, k, temperature)
    assert 0 <= tok_gpu < w.shape[0] and w[tok_gpu] > 0.0, (n_gpu, tok_gpu)


def _oracle_checked(p, q, draft, ua, us, temperature, n_gpu, tok_gpu):
    """Compare one sequence; returns 'exact', 'band' or raises."""
    k = draft.shape[0]
    # the oracle's accept chain, with margins
    n_or = k
    for i in range(k):
        pp = O.softmax_t(p[i], temperature)
        qq = O.softmax_t(q[i], temperature)
        x = int(draft[i])
        lhs, rhs = float(ua[i]) * qq[x], pp[x]
        if abs(lhs - rhs) <= ACCEPT_BAND * max(lhs, rhs, 1e-30):
            _band_consistent(p, q, draft, ua, temperature, n_gpu, tok_gpu, i)
            return "band"
        if not lhs < rhs:
            n_or = i
            break
    n_ref, tok_ref = O.speculative_accept(p, q, draft, ua.astype(np.float64), float(us), temperature)
    assert n_ref == n_or
    assert n_gpu == n_ref, (n_gpu, n_ref)
    if tok_gpu == tok_ref:
        return "exact"
    # a different token is allowed only when the draw target sits on a boundary within the band
    w = _draw_weights(p, q, n_ref, k, temperature)
    cdf = np.cumsum(w)
    Z = cdf[-1]
    target = float(us) * Z
    lo = cdf[tok_gpu - 1] if tok_gpu > 0 else 0.0
    assert w[tok_gpu] > 0.0, (tok_gpu, tok_ref)
    assert lo - DRAW_BAND * Z <= target < cdf[tok_gpu] + DRAW_BAND * Z, (tok_gpu, tok_ref, target, lo, cdf[tok_gpu])
    return "band"


def _run(p, q, draft, ua, us, temperature=1.0, stride=None):
    B, k1, V = p.shape
    k = k1 - 1
    dev = "cuda"
    if stride is None:
        pt = torch.from_numpy(p).to(dev)
        qt = torch.from_numpy(q).to(dev) if k > 0 else None
    else:  # rows padded to `stride` elements
        pp = np.zeros((B, k1, stride), dtype=np.float32)
        pp[:, :, :V] = p
        pt = torch.from_numpy(pp).to(dev)[:, :, :V]
        qt = None
        if k > 0:
            qq = np.zeros((B, k, stride), dtype=np.float32)
            qq[:, :, :V] = q
            qt = torch.from_numpy(qq).to(dev)[:, :, :V]
    n, tok = spdec.spec_accept(pt, qt, torch.from_numpy(draft).to(dev) if k > 0 else None,
                               torch.from_numpy(ua).to(dev) if k > 0 else None, torch.from_numpy(us).to(dev),
                               temperature)
    torch.cuda.synchronize()
    return n.cpu().numpy(), tok.cpu().numpy()


def _check_all(p, q, draft, ua, us, temperature=1.0, stride=None, max_band=2):
    n, tok = _run(p, q, draft, ua, us, temperature, stride)
    kinds = [_oracle_checked(p[b], q[b], draft[b], ua[b], us[b], temperature, int(n[b]), int(tok[b]))
             for b in range(p.shape[0])]
    band = kinds.count("band")
    print(f"  B={p.shape[0]} k={p.shape[1] - 1} V={p.shape[2]}: exact {kinds.count('exact')}, band {band}, "
          f"kept {np.bincount(n, minlength=p.shape[1]).tolist()}", flush=True)
    assert band <= max_band
    return n, tok


@pytest.mark.parametrize("B,k,V,seed", [(16, 6, 5000, 0), (8, 6, 151936, 1), (32, 3, 20000, 2), (12, 1, 8193, 3)])
def test_spec_accept_matches_oracle(B, k, V, seed):
    print(f"spec_accept B={B} k={k} V={V}", flush=True)
    _check_all(*_inputs(B, k, V, seed))


def test_no_drafts_draws_from_the_verifier():
    p, q, draft, ua, us = _inputs(10, 0, 3000, 5)
    n, tok = _check_all(p, q, draft, ua, us)
    assert np.all(n == 0)


def test_identical_distributions_keep_every_draft():
    p, q, draft, ua, us = _inputs(12, 6, 4000, 6, same=True)
    ua = np.minimum(ua, np.float32(0.999))
    n, tok = _check_all(p, q, draft, ua, us)
    assert np.all(n == 6)


def test_rejection_with_no_residual_mass_draws_from_verifier():
    """Identical verifier and drafter logits with an accept uniform of 1 (one past the documented range, which
    forces a rejection at the first position): the residual has no mass anywhere, and the token is drawn from
    the verifier's own distribution, as in the oracle."""
    p, q, draft, ua, us = _inputs(12, 3, 20000, 8, same=True)
    ua = np.ones_like(ua)
    # every accept test sits exactly on its boundary (1 * q(x) == p(x)), so all are in the band by construction
    n, tok = _check_all(p, q, draft, ua, us, max_band=12)
    assert np.all(n == 0)
    for b in range(12):
        n_ref, tok_ref = O.speculative_accept(p[b], q[b], draft[b], ua[b].astype(np.float64), float(us[b]))
        assert n_ref == 0
        if int(tok[b]) != tok_ref:  # only a draw target on a token boundary (fp32 vs fp64) may differ
            cdf = np.cumsum(O.softmax_t(p[b, 0], 1.0))
            target = float(us[b]) * cdf[-1]
            assert abs(target - cdf[min(int(tok[b]), tok_ref)]) <= DRAW_BAND * cdf[-1], (b, int(tok[b]), tok_ref)


def test_temperature_and_padded_unaligned_rows():
    p, q, draft, ua, us = _inputs(8, 4, 6001, 7, temperature=0.7)
    _check_all(p, q, draft, ua, us, temperature=0.7, stride=6003)   # stride % 4 != 0: scalar loads
    _check_all(p, q, draft, ua, us, temperature=0.7, stride=6004)


def test_spec_accept_is_deterministic():
    p, q, draft, ua, us = _inputs(16, 6, 30000, 8)
    a = _run(p, q, draft, ua, us)
    b = _run(p, q, draft, ua, us)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_spec_accept_reused_workspace():
    """One workspace across calls of different batch, draft length, vocabulary and temperature: each result
    equals the same call on a fresh workspace."""
    shapes = [(16, 6, 30000, 1.0), (3, 2, 1000, 0.7), (16, 6, 30000, 1.2), (4, 0, 5000, 1.0)]
    nbytes = max(spdec.spec_accept_workspace_bytes(B, k, V) for B, k, V, _ in shapes)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for i, (B, k, V, T) in enumerate(shapes):
        p, q, draft, ua, us = _inputs(B, k, V, 40 + i, temperature=T)
        args = [torch.from_numpy(p).cuda(), torch.from_numpy(q).cuda() if k > 0 else None,
                torch.from_numpy(draft).cuda() if k > 0 else None, torch.from_numpy(ua).cuda() if k > 0 else None,
                torch.from_numpy(us).cuda()]
        n1, t1 = spdec.spec_accept(*args, temperature=T, workspace=ws)
        n2, t2 = spdec.spec_accept(*args, temperature=T)
        torch.cuda.synchronize()
        assert torch.equal(n1, n2) and torch.equal(t1, t2), (B, k, V, T)
