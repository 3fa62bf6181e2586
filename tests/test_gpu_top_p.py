"""GPU parity of score-mass (top-p) page selection (spdec_select_pages_top_p).

The kept count is an integer decided by floating point (fp64 sums in the
oracle, 2^-48 fixed-point sums on the GPU): it must equal the oracle's except
where the oracle's kept mass lies within 1e-6 (relative) of the target on
either side of its last page (then it may differ by one). The
kept set must be the Top-K set of the oracle's fp64 scores for the kept count,
outside the 1e-6 score tie band at the cut.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

from oracle import top_p as TP
from sparse_attention_decode_page_amd import spdec
from sparse_attention_decode_page_amd import synth as S

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gpu_support as GS  # noqa: E402

pytestmark = pytest.mark.gpu
MASS_BAND = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(spdec.LIB_PATH):
        from sparse_attention_decode_page_amd import build
        build.build()
    spdec.lib()
    assert torch.cuda.is_available()


def _oracle_count_and_band(s32, top_p, c, kcap):
    """Oracle kept count on the fp32-rounded scores, and whether its decision lies in the mass band."""
    P = s32.shape[0]
    got = TP.select_pages_top_p(s32, top_p, c, kcap)
    K = len(got)
    w = TP.page_mass(s32, c)
    target = top_p * w.sum()
    order = sorted(range(1, P - 1), key=lambda i: (-s32[i], i))
    acc = [w[0] + w[P - 1]]
    for p in order:
        acc.append(acc[-1] + w[p])
    near = any(abs(acc[j] - target) <= MASS_BAND * target for j in (K - 3, K - 2) if 0 <= j < len(acc))
    return K, near


def _check(wl, top_p, units, use_budget=True, c=None, expect_all=False):
    spec = wl.spec
    dw = GS.DeviceWorkload(wl)
    cache = dw.cache
    spdec.build_meta(cache)
    G = spec.group
    c = 1.0 / (G * math.sqrt(spec.head_dim)) if c is None else c
    c32 = float(np.float32(c))
    cap = dw.max_budget if use_budget else int(wl.page_table.shape[1])
    budget = dw.budget if use_budget else None
    scores = torch.zeros((spec.batch, spec.num_kv_heads, cache.max_pages), dtype=torch.float32, device="cuda")
    idx, cnt = spdec.select_pages_top_p(cache, dw.q, top_p, cap, score_scale=c32, budget_pages=budget,
                                        scores_out=scores)
    idx2, cnt2 = spdec.select_pages_top_p(cache, dw.q, top_p, cap, score_scale=c32, budget_pages=budget)
    # the kept sets have the form the sparse decode takes (ascending pages below the page count, at most cap)
    pre = spdec.check_inputs(cache, q=dw.q, sel_idx=idx, sel_cnt=cnt, max_budget_pages=cap)
    assert pre["first_bad_sequence"] == cache.batch, pre
    torch.cuda.synchronize()
    assert torch.equal(cnt, cnt2)
    idx_h, cnt_h, idx2_h = idx.cpu().numpy(), cnt.cpu().numpy(), idx2.cpu().numpy()
    banded = 0
    sizes = []
    for (b, g) in units:
        K64, _ = GS.unit_kv_f64(wl, b, g)
        s64 = GS.oracle_scores(wl, b, g, K64)
        s32 = s64.astype(np.float32).astype(np.float64)
        P = s64.shape[0]
        kcap = min(max(int(wl.budget_pages[b]), 2), cap, P) if use_budget else min(cap, P)
        K_o, near = _oracle_count_and_band(s32, top_p, c32, kcap)
        k = int(cnt_h[b, g])
        assert np.array_equal(idx_h[b, g, :k], idx2_h[b, g, :k])
        if expect_all:   # the whole mass: the last page meets the target by construction
            assert k == P and idx_h[b, g, :k].tolist() == list(range(P)), (b, g, k, P)
            sizes.append(k)
            continue
        if near:
            banded += 1
            assert abs(k - K_o) <= 1, (b, g, k, K_o)
        else:
            assert k == K_o, (b, g, k, K_o)
        GS.check_selection(idx_h[b, g], k, s64, k, k)   # the Top-k set of the oracle's scores
        sizes.append(k)
    print(f"  top_p {top_p}: {len(units)} units, kept {min(sizes)}..{max(sizes)} pages, {banded} in the mass band",
          flush=True)
    assert banded <= max(1, len(units) // 10)


CASES = [
    # (batch, Hq, Hkv, D, ps, lens, budget tokens)
    (3, 8, 2, 128, 16, ("uniform", 300, 3000), 1024),
    (2, 4, 2, 64, 8, ("uniform", 40, 900), 256),
    (2, 16, 2, 128, 32, ("uniform", 500, 4000), 2048),
    (4, 4, 4, 128, 64, ("uniform", 3, 5000), 4096),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("top_p", [0.3, 0.9, 0.99])
def test_top_p_small_all_units(case, top_p):
    B, Hq, Hkv, D, ps, lens, bt = CASES[case]
    spec = S.custom_spec(f"topp{case}", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                         dtype="bf16", lens=lens, budget=("tokens", bt), outlier_channels=2)
    wl = S.make_workload(spec, seed=40 + case)
    print(f"top-p case {case}: G={spec.group} D={D} ps={ps}", flush=True)
    _check(wl, top_p, [(b, g) for b in range(B) for g in range(Hkv)])


@pytest.mark.parametrize("seed", range(6))
def test_top_p_random_shapes(seed):
    """Seeded random shapes, p and score scale, with and without the per-sequence cap."""
    r = np.random.default_rng(5000 + seed)
    G = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.choice([1, 2]))
    D = int(r.choice([64, 128]))
    ps = int(r.choice([8, 16, 32, 64]))
    B = int(r.integers(1, 4))
    spec = S.custom_spec(f"topp-rand{seed}", batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                         page_size=ps, dtype="bf16", lens=("uniform", 1, 200 * ps),
                         budget=("tokens", int(r.integers(2, 60)) * ps), outlier_channels=2)
    wl = S.make_workload(spec, seed=seed)
    top_p = float(r.uniform(0.05, 0.995))
    c = float(r.uniform(0.2, 3.0)) / (G * math.sqrt(D))
    _check(wl, top_p, [(b, g) for b in range(B) for g in range(Hkv)], use_budget=bool(r.random() < 0.5), c=c)


def test_top_p_without_cap_and_full_mass():
    spec = S.custom_spec("topp-nocap", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                         dtype="bf16", lens=("uniform", 100, 2500), budget=("tokens", 64), outlier_channels=2)
    wl = S.make_workload(spec, seed=51)
    units = [(b, g) for b in range(3) for g in range(2)]
    _check(wl, 0.8, units, use_budget=False)
    _check(wl, 1.0, units, use_budget=False, c=0.0, expect_all=True)   # flat masses, all of them: every page


@pytest.mark.parametrize("tokens", [65600, 96000, 140000])
def test_top_p_long_tables(tokens):
    # 8200, 12000 and 17500 pages: 1024-thread workgroups with 8, 16 and 32 keys per thread
    spec = S.custom_spec(f"topp-long{tokens}", batch=1, num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=8,
                         dtype="bf16", lens=("fixed", tokens), budget=("tokens", 64), outlier_channels=2)
    wl = S.make_workload(spec, seed=3)
    _check(wl, 0.7, [(0, 0), (0, 1)], use_budget=False)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_top_p_qwen3_8b_ragged_sampled():
    wl = S.make_workload("qwen3-8b-ragged", seed=0)
    _check(wl, 0.9, GS.sample_units(wl, 8, seed=9))


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_top_p_long_context_8190_middle_pages():
    wl = S.make_workload("long-131k-ps16", seed=0)
    _check(wl, 0.95, GS.sample_units(wl, 3, seed=2), use_budget=False)


@pytest.mark.parametrize("use_budget", [True, False])
def test_top_p_one_kernel_form(use_budget):
    """A batch of at least one (sequence, KV head) per compute unit takes the one-kernel form (scores in LDS, the
    same cut): kept pages, counts and scores bit for bit as the scoring and top-p kernels give them on the first
    sequences as a batch of their own, and sampled units against the oracle."""
    spec = S.custom_spec("topp-one", batch=40, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                         dtype="bf16", lens=("uniform", 1, 6000), budget=("tokens", 1024), outlier_channels=2)
    wl = S.make_workload(spec, seed=61)
    dw = GS.DeviceWorkload(wl)
    cache = dw.cache
    spdec.build_meta(cache)
    assert spdec.select_pages_form(cache, dw.max_budget) == "one kernel"
    c32 = float(np.float32(1.0 / (spec.group * math.sqrt(spec.head_dim))))
    cap = dw.max_budget if use_budget else int(wl.page_table.shape[1])
    budget = dw.budget if use_budget else None
    shape = (spec.batch, spec.num_kv_heads, cache.max_pages)
    sc_a = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    idx_a, cnt_a = spdec.select_pages_top_p(cache, dw.q, 0.9, cap, score_scale=c32, budget_pages=budget,
                                            scores_out=sc_a)
    n = 12   # 96 units: the scoring and top-p kernels
    sub = spdec.PagedCache(cache.k_pool, cache.v_pool, cache.kminmax, cache.page_table[:n], cache.seq_lens[:n],
                           cache.num_q_heads)
    assert spdec.select_pages_form(sub, dw.max_budget) != "one kernel"
    sc_b = torch.full((n,) + shape[1:], float("nan"), dtype=torch.float32, device="cuda")
    idx_b, cnt_b = spdec.select_pages_top_p(sub, dw.q[:n], 0.9, cap, score_scale=c32,
                                            budget_pages=budget[:n] if budget is not None else None, scores_out=sc_b)
    torch.cuda.synchronize()
    ca, cb = cnt_a.cpu().numpy(), cnt_b.cpu().numpy()
    ia, ib = idx_a.cpu().numpy(), idx_b.cpu().numpy()
    sa, sb = sc_a.cpu().numpy(), sc_b.cpu().numpy()
    assert np.array_equal(ca[:n], cb)
    for b in range(n):
        P = wl.pages(b)
        assert np.array_equal(sa[b, :, :P].view(np.uint32), sb[b, :, :P].view(np.uint32)), b
        for g in range(spec.num_kv_heads):
            k = int(ca[b, g])
            assert np.array_equal(ia[b, g, :k], ib[b, g, :k]), (b, g)
    print(f"  top-p one kernel (budget {use_budget}): {n} of {spec.batch} sequences equal to the two kernels",
          flush=True)
    _check(wl, 0.9, GS.sample_units(wl, 10, seed=62), use_budget=use_budget)
