"""GPU parity of the shared-prefix page selection (spdec_select_pages_shared).

Groups of N consecutive sequences share their prompt pages. The shared pages'
bounds come from one read per (group, KV head), the rest from each sequence's
own pages; every score is the same fp64 sum in the same order as the
per-sequence selection, so scores must be bit-identical to spdec_select_pages
and the selection equal. Sampled units are also checked against the fp64
oracle under the tie band.
"""
import os
import sys

import numpy as np
import pytest
import torch

from sparse_attention_decode_page_amd import spdec
from sparse_attention_decode_page_amd import synth as S

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gpu_support as GS  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(spdec.LIB_PATH):
        from sparse_attention_decode_page_amd import build
        build.build()
    spdec.lib()
    assert torch.cuda.is_available()


def _check(wl, shared, N, units):
    spec = wl.spec
    print(f"select shared {spec.name}: B={spec.batch} N={N} G={spec.group} D={spec.head_dim} ps={spec.page_size} "
          f"shared pages {shared.tolist()[:4]}", flush=True)
    dw = GS.DeviceWorkload(wl)
    c = dw.cache
    spdec.build_meta(c)
    sh = torch.from_numpy(shared.astype(np.int32)).cuda()
    ref_idx, ref_cnt, ref_scores = GS.run_select(dw)
    scores = torch.full((c.batch, c.num_kv_heads, c.max_pages), float("nan"), dtype=torch.float32, device="cuda")
    idx, cnt = spdec.select_pages_shared(c, dw.q, N, sh, dw.budget, dw.max_budget, scores_out=scores)
    # the same call through the workspace (no scores out)
    idx2, cnt2 = spdec.select_pages_shared(c, dw.q, N, sh, dw.budget, dw.max_budget)
    # inputs meet the documented preconditions and the selection is of the form the decode takes
    pre = spdec.check_inputs(c, q=dw.q, sel_idx=idx, sel_cnt=cnt, max_budget_pages=dw.max_budget, group_size=N,
                             shared_pages=sh)
    assert pre["first_bad_sequence"] == spec.batch, pre
    torch.cuda.synchronize()
    P = np.minimum((wl.lens + spec.page_size - 1) // spec.page_size, c.max_pages)
    s_h, r_h = scores.cpu().numpy(), ref_scores.cpu().numpy()
    for b in range(spec.batch):
        assert np.array_equal(s_h[b, :, :P[b]].view(np.uint32), r_h[b, :, :P[b]].view(np.uint32)), b
    assert torch.equal(cnt, ref_cnt) and torch.equal(cnt2, ref_cnt)
    cnt_h, idx_h, idx2_h, ref_h = cnt.cpu().numpy(), idx.cpu().numpy(), idx2.cpu().numpy(), ref_idx.cpu().numpy()
    for b in range(spec.batch):
        for g in range(spec.num_kv_heads):
            k = cnt_h[b, g]
            assert np.array_equal(idx_h[b, g, :k], ref_h[b, g, :k]), (b, g)
            assert np.array_equal(idx2_h[b, g, :k], ref_h[b, g, :k]), (b, g)
    for (b, g) in units:
        K64, _ = GS.unit_kv_f64(wl, b, g)
        s64 = GS.oracle_scores(wl, b, g, K64)
        GS.check_selection(idx_h[b, g], int(cnt_h[b, g]), s64, int(wl.budget_pages[b]), dw.max_budget)
    print(f"  scores bit-identical, selection equal; {len(units)} units checked against the oracle", flush=True)


CASES = [
    # (batch, Hq, Hkv, D, ps, gen lens, N, prompt tokens, budget)
    (8, 8, 2, 128, 16, ("uniform", 10, 300), 4, 200, ("tokens", 64)),    # prompt ends mid-page
    (6, 4, 2, 64, 8, ("uniform", 1, 90), 3, 96, ("tokens", 48)),         # page size 8, prompt on a page boundary
    (8, 16, 2, 128, 32, ("uniform", 40, 400), 8, 1500, ("tokens", 256)),  # group 8, eight members
    (4, 4, 4, 128, 64, ("uniform", 5, 200), 2, 4000, ("tokens", 512)),   # one query head per KV head
    (4, 8, 2, 128, 16, ("uniform", 50, 60), 1, 320, ("tokens", 64)),     # groups of one
    (16, 8, 2, 128, 16, ("uniform", 100, 3000), 8, 9000, ("tokens", 1024)),  # long shared prompt
    (6, 4, 2, 64, 8, ("list", [0, 0, 0, 0, 5, 1]), 3, 96, ("tokens", 48)),  # members holding only the prompt
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_select_shared_matches_select(case):
    B, Hq, Hkv, D, ps, gen, N, prompt, budget = CASES[case]
    spec = S.custom_spec(f"selshared{case}", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                         dtype="bf16", lens=gen, budget=budget, outlier_channels=2, prompt=("shared", N, prompt))
    wl = S.make_workload(spec, seed=20 + case)
    _check(wl, wl.shared_pages, N, GS.sample_units(wl, 6, seed=case))


@pytest.mark.parametrize("seed", range(6))
def test_select_shared_random_shapes(seed):
    """Seeded random groups (1-8 members, any group size, page size, prompt and generated lengths, budgets)."""
    r = np.random.default_rng(4000 + seed)
    N = int(r.integers(1, 9))
    groups = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.choice([1, 2]))
    D = int(r.choice([64, 128]))
    ps = int(r.choice([8, 16, 32, 64]))
    prompt = int(r.integers(1, 60 * ps))
    spec = S.custom_spec(f"selshared-rand{seed}", batch=N * groups, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                         head_dim=D, page_size=ps, dtype="bf16", lens=("uniform", 1, 30 * ps),
                         budget=("tokens", int(r.integers(2, 40)) * ps), outlier_channels=2,
                         prompt=("shared", N, prompt))
    wl = S.make_workload(spec, seed=seed)
    _check(wl, wl.shared_pages, N, [(b, g) for b in range(N * groups) for g in range(Hkv)])


def test_select_shared_fewer_shared_pages_and_none():
    spec = S.custom_spec("selshared-partial", batch=8, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                         dtype="bf16", lens=("uniform", 30, 200), budget=("tokens", 128), prompt=("shared", 4, 400))
    wl = S.make_workload(spec, seed=31)
    _check(wl, np.array([7, 0], dtype=np.int32), 4, [(0, 0), (5, 1)])
    _check(wl, np.zeros(2, dtype=np.int32), 4, [(3, 1)])


def test_select_shared_rejects_unsupported():
    spec = S.custom_spec("selshared-f32", batch=4, num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                         dtype="f32", lens=("fixed", 64), budget=("tokens", 64))
    dw = GS.DeviceWorkload(S.make_workload(spec, seed=0))
    sh = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):
        spdec.select_pages_shared(dw.cache, dw.q, 2, sh, dw.budget, dw.max_budget)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_select_shared_qwen3_8b_grouped():
    wl = S.make_workload("qwen3-8b-grouped", seed=0)
    _check(wl, wl.shared_pages, wl.spec.prompt[1], GS.sample_units(wl, 6, seed=7))
