"""GPU: spdec_sparse_path (one decode step: page selection, then attention over the kept pages) against the two
calls it stands for and against the CPU oracle.

Batches with at least one (sequence, KV head) per compute unit run the step as one kernel, batches of at most half
as many in the sliced form (each unit's pages cut over several workgroups); in both the selection (sel_idx,
sel_cnt, scores) must equal spdec_select_pages' bit for bit, and out / lse must agree with spdec_sparse_decode over
that selection to fp32 rounding of a different summation order (3e-6 max-abs; both are within the oracle's bf16
bar of 1e-2, checked per unit). Other shapes run the two calls, so every output is bitwise equal.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_decode_page_amd import spdec
from sparse_attention_decode_page_amd import synth as S

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gpu_support as GS  # noqa: E402

pytestmark = pytest.mark.gpu

# Bar between the one-kernel step and the two calls: both accumulate the same fp32 terms (p_t v_t, e^{z_t}) per
# token; only the grouping of the per-chunk sums differs. Outputs are convex combinations of bf16 values ~N(0,1)
# (|v| < 6), so a few ulps of 6 plus the relative error of the normaliser bound the difference.
TOL_SPLIT = 3e-6


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(spdec.LIB_PATH):
        from sparse_attention_decode_page_amd import build
        build.build()
    spdec.lib()
    assert torch.cuda.is_available()


def _form(dw) -> str:
    """The documented rule for the form spdec_sparse_path takes, checked against the library's own answer."""
    c = dw.cache
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = c.batch * c.num_kv_heads
    cap = dw.max_budget
    base = c.dtype == torch.bfloat16 and c.num_q_heads // c.num_kv_heads <= 4
    form = "two calls"
    if base and c.max_pages <= 4096 and cap <= 4096 and c.batch <= 512 and units >= cus:
        form = "one kernel"
    elif base and units <= 128 and cap <= 4096:
        S = min(16, cus // units)
        while 2 <= S <= 16 and -(-c.max_pages // S) > 4096:
            S += 1
        if 2 <= S <= 16 and S * (cap - 2) <= 4096:
            form = "sliced"
    assert spdec.sparse_path_form(c, cap) == form, (form, spdec.sparse_path_form(c, cap))
    return form


def _run(wl, units, max_budget=None, expect_form=None):
    spec = wl.spec
    dw = GS.DeviceWorkload(wl)
    if max_budget is not None:
        dw.max_budget = max_budget
    c = dw.cache
    spdec.build_meta(c)
    form = _form(dw)
    if expect_form is not None:
        assert form == expect_form, form
    # the two calls
    scores_a = torch.zeros((c.batch, c.num_kv_heads, c.max_pages), dtype=torch.float32, device=c.device)
    idx_a, cnt_a = spdec.select_pages(c, dw.q, dw.budget, dw.max_budget, scores_out=scores_a)
    out_a, lse_a = spdec.sparse_decode(c, dw.q, idx_a, cnt_a, dw.max_budget)
    # the step; output buffers poisoned so that a missed write shows
    scores_b = torch.full_like(scores_a, float("nan"))
    idx_b = torch.full_like(idx_a, -7)
    cnt_b = torch.full_like(cnt_a, -7)
    out_b = torch.full_like(out_a, float("nan"))
    lse_b = torch.full_like(lse_a, float("nan"))
    spdec.sparse_path(c, dw.q, dw.budget, dw.max_budget, sel_idx=idx_b, sel_cnt=cnt_b, scores_out=scores_b,
                      out=out_b, lse=lse_b)
    torch.cuda.synchronize()
    cnt_a_h, cnt_b_h = cnt_a.cpu().numpy(), cnt_b.cpu().numpy()
    idx_a_h, idx_b_h = idx_a.cpu().numpy(), idx_b.cpu().numpy()
    sa, sb = scores_a.cpu().numpy(), scores_b.cpu().numpy()
    assert np.array_equal(cnt_a_h, cnt_b_h)
    for b in range(spec.batch):
        P = wl.pages(b)
        assert np.array_equal(sa[b, :, :P].view(np.uint32), sb[b, :, :P].view(np.uint32)), b
        for g in range(spec.num_kv_heads):
            k = int(cnt_a_h[b, g])
            assert np.array_equal(idx_a_h[b, g, :k], idx_b_h[b, g, :k]), (b, g)
    oa, ob = out_a.cpu().numpy(), out_b.cpu().numpy()
    la, lb = lse_a.cpu().numpy(), lse_b.cpu().numpy()
    assert np.all(np.isfinite(ob))
    live = wl.lens > 0
    assert np.array_equal(np.isneginf(la), np.isneginf(lb))
    assert np.all(np.isneginf(lb[~live])) and np.all(ob[~live] == 0)
    d_out = float(np.abs(oa - ob).max())
    d_lse = float(np.abs(la[live] - lb[live]).max()) if live.any() else 0.0
    if form != "two calls":
        assert d_out <= TOL_SPLIT and d_lse <= TOL_SPLIT, (d_out, d_lse)
    else:
        assert d_out == 0.0 and d_lse == 0.0, (d_out, d_lse)
    # the oracle, unit by unit, over the step's own selection
    tol = GS.TOL_OUT[spec.dtype]
    scale = GS.default_scale(wl)
    G = spec.group
    worst = 0.0
    for (b, g) in units:
        P = wl.pages(b)
        K64, V64 = GS.unit_kv_f64(wl, b, g)
        s64 = GS.oracle_scores(wl, b, g, K64)
        k = int(cnt_b_h[b, g])
        GS.check_selection(idx_b_h[b, g], k, s64, int(wl.budget_pages[b]), dw.max_budget)
        o, lse = O.decode_unit(GS.q_group_f64(wl, b, g), K64, V64, idx_b_h[b, g, :k], spec.page_size, scale)
        e = float(np.abs(ob[b, g * G:(g + 1) * G] - o).max())
        el = float(np.abs(lb[b, g * G:(g + 1) * G] - lse).max()) if P else 0.0
        assert e <= tol and el <= tol, (b, g, e, el)
        worst = max(worst, e, el)
    say(f"  {spec.name}: {form}: step vs calls out {d_out:.2e} lse {d_lse:.2e}; "
        f"{len(units)} units vs oracle, worst {worst:.2e}")
    return dw


def _lens(seed, n, lo, hi, zeros=0):
    r = np.random.default_rng(seed)
    lens = [int(x) for x in r.integers(lo, hi + 1, n)]
    for i in range(zeros):
        lens[(7 * i + 3) % n] = 0
    return lens


# dtype D, Hq, Hkv, ps, batch, (lo, hi) tokens, budget pages (lo, hi), zero-length sequences
CASES = [
    ("D128 G4 ps16", 128, 32, 8, 16, 40, (1, 6000), (0, 90), 3),
    ("D128 G2 ps32", 128, 16, 8, 32, 32, (1, 9000), (0, 60), 2),   # 256 units: no ordering by size
    ("D64 G1 ps8", 64, 8, 8, 8, 34, (1, 16384), (0, 300), 2),
    ("D64 G4 ps64", 64, 16, 4, 64, 70, (1, 20000), (0, 40), 4),
    ("D128 G1 ps16", 128, 8, 8, 16, 33, (2000, 32768), (100, 400), 0),
    # 512 sequences of one KV head (the most the form takes): ranks of 512 sequences, one comparison loop each
    ("D64 G4 ps16 B512", 64, 4, 1, 16, 512, (1, 3000), (0, 60), 5),
    # equal lengths and budgets: every unit reads the same bytes, the order falls back to the sequence index
    ("D128 G2 ps16 equal", 128, 2, 1, 16, 300, (1000, 1000), (20, 20), 0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_step_matches_calls_and_oracle(case):
    name, D, Hq, Hkv, ps, B, (lo, hi), (blo, bhi), zeros = CASES[case]
    lens = _lens(case, B, lo, hi, zeros)
    bud = [int(x) for x in np.random.default_rng(100 + case).integers(blo, bhi + 1, B)]
    say(f"case path {name}: batch {B}, lens {lo}..{hi} ({zeros} empty), budget pages {blo}..{bhi}")
    spec = S.custom_spec(f"path-{case}", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                         dtype="bf16", lens=("list", lens), budget=("pages", bud), outlier_channels=4)
    wl = S.make_workload(spec, seed=case)
    _run(wl, GS.sample_units(wl, 40, seed=case), expect_form="one kernel")


@pytest.mark.parametrize("pages", [2050, 4096])
def test_step_longest_lists(pages):
    """The widest page tables of the one-kernel form's two sizes (2050 pages: 2048 middle pages, four keys per
    thread; 4096: eight), on two long sequences among short ones: budgets that keep every page, all but one (the
    Top-B over every middle page), two (sink and local only) and a list capacity of `pages`."""
    B = 32
    r = np.random.default_rng(pages)
    lens = [pages * 16, pages * 16 - 5] + [int(x) for x in r.integers(1, 2000, B - 2)]
    bud = [pages, pages - 1] + [2, 40] * ((B - 2) // 2)
    bud[5] = pages  # a short sequence with a budget above its page count
    say(f"case path longest lists: page table of {pages} pages, capacity {pages}")
    spec = S.custom_spec(f"path-longest{pages}", batch=B, num_q_heads=32, num_kv_heads=8, head_dim=128,
                         page_size=16, dtype="bf16", lens=("list", lens), budget=("pages", bud), outlier_channels=4)
    wl = S.make_workload(spec, seed=21)
    assert wl.page_table.shape[1] == pages
    _run(wl, [(0, 0), (0, 5), (1, 3), (1, 7), (2, 1), (5, 6), (31, 2)], expect_form="one kernel")


def test_step_capacity_two():
    """A list capacity of 2: every unit keeps its sink and local pages only (no select)."""
    B = 40
    say("case path capacity 2")
    spec = S.custom_spec("path-cap2", batch=B, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                         dtype="bf16", lens=("list", _lens(9, B, 1, 3000, 2)), budget=("pages", [50] * B),
                         outlier_channels=4)
    wl = S.make_workload(spec, seed=9)
    _run(wl, GS.sample_units(wl, 20, seed=9), max_budget=2, expect_form="one kernel")


@pytest.mark.parametrize("what", ["between the forms", "f32", "G8", "long tables"])
def test_step_runs_the_two_calls_elsewhere(what):
    """Shapes outside both fused forms: the step is the two calls, bit for bit."""
    kw = dict(batch=20, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, dtype="bf16",
              lens=("uniform", 100, 5000), budget=("pages", [3, 20, 40, 80] * 5), outlier_channels=4)
    if what == "f32":
        kw.update(batch=40, dtype="f32", outlier_channels=0, budget=("pages", [20] * 40))
    elif what == "G8":
        kw.update(batch=40, num_q_heads=64, budget=("pages", [20] * 40))
    elif what == "long tables":
        kw.update(batch=40, lens=("list", [70000] + [300] * 39), budget=("pages", [100] * 40))
    elif what == "between the forms":
        assert 128 < 20 * 8 < 256
    say(f"case path fallback: {what}")
    wl = S.make_workload(S.custom_spec(f"path-fb-{what}", **kw), seed=5)
    _run(wl, GS.sample_units(wl, 8, seed=5), expect_form="two calls")


# The sliced form: dtype D, Hq, Hkv, ps, batch, (lo, hi) tokens, budget pages, empty sequences
SLICED = [
    ("D128 G4 ps16", 128, 32, 8, 16, 4, (20000, 40000), [3, 40, 200, 400], 0),
    ("D128 G2 ps32", 128, 16, 8, 32, 6, (1, 60000), [2, 100, 800, 120, 0, 60], 1),
    ("D64 G1 ps8", 64, 4, 4, 8, 8, (30000, 70000), [500, 2, 7, 256, 511, 100, 300, 1], 0),
    ("D64 G4 ps64", 64, 16, 4, 64, 3, (100, 200000), [30, 10, 60], 0),
    ("D128 G4 ps16 one unit", 128, 4, 1, 16, 1, (65536, 65536), [250], 0),
    # 128 units, the most the form takes: two slices per unit
    ("D128 G4 ps16 128 units", 128, 32, 8, 16, 16, (1, 30000), [2, 9, 64, 300, 130, 0, 45, 1000, 17, 250, 80,
                                                                    3, 500, 120, 33, 700], 1),
]


@pytest.mark.parametrize("case", range(len(SLICED)))
def test_sliced_step_matches_calls_and_oracle(case):
    """Few units (at most half the compute units): each unit's pages cut into slices scored by separate
    workgroups, the unit's Top-B taken from the slices' candidates, the kept pages streamed by the slices and
    merged: selection bit for bit as the two calls, outputs within fp32 reordering, sampled units against the
    oracle. Budgets below 2, equal to and above the page count, empty sequences."""
    name, D, Hq, Hkv, ps, B, (lo, hi), bud, zeros = SLICED[case]
    lens = _lens(500 + case, B, lo, hi, zeros)
    say(f"case sliced {name}: batch {B}, lens {lens}, budget pages {bud}")
    spec = S.custom_spec(f"sliced-{case}", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                         dtype="bf16", lens=("list", lens), budget=("pages", bud), outlier_channels=4)
    wl = S.make_workload(spec, seed=500 + case)
    _run(wl, GS.sample_units(wl, 12, seed=case), expect_form="sliced")


def test_sliced_workspace_shared_across_calls_and_shapes():
    """One workspace (never cleared between calls) through sliced calls of two shapes, a one-kernel call and a
    two-call shape: every result equals a fresh workspace's bit for bit."""
    def wl_of(name, B, Hkv, lens, bud, seed):
        spec = S.custom_spec(name, batch=B, num_q_heads=4 * Hkv, num_kv_heads=Hkv, head_dim=128, page_size=16,
                             dtype="bf16", lens=("list", lens), budget=("pages", bud), outlier_channels=4)
        return S.make_workload(spec, seed=seed)
    shapes = [wl_of("ws-a", 4, 8, [20000, 9000, 30000, 100], [300, 40, 200, 2], 1),
              wl_of("ws-b", 2, 4, [50000, 7000], [120, 60], 2),
              wl_of("ws-c", 40, 8, _lens(3, 40, 1, 3000, 1), [30] * 40, 3),
              wl_of("ws-d", 20, 8, _lens(4, 20, 1, 3000, 1), [30] * 20, 4)]
    devs = [GS.DeviceWorkload(w) for w in shapes]
    for dw in devs:
        spdec.build_meta(dw.cache)
    need = max(spdec.sparse_path_workspace_bytes(dw.cache, dw.max_budget) for dw in devs)
    shared = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")  # not cleared: nothing may rely on zeros
    say("case sliced workspace shared: forms " + ", ".join(spdec.sparse_path_form(dw.cache, dw.max_budget)
                                                           for dw in devs))
    for rep in range(2):
        for dw in devs:
            got = spdec.sparse_path(dw.cache, dw.q, dw.budget, dw.max_budget, workspace=shared)
            want = spdec.sparse_path(dw.cache, dw.q, dw.budget, dw.max_budget)
            torch.cuda.synchronize()
            for x, y in zip(got, want):
                if x.dtype == torch.float32:
                    x, y = x.view(torch.int32), y.view(torch.int32)
                assert torch.equal(x, y), (rep, dw.wl.spec.name)


def _sub_cache(c, n):
    """The first n sequences of a cache as a batch of their own (leading rows of the page table and lengths)."""
    return spdec.PagedCache(c.k_pool, c.v_pool, c.kminmax, c.page_table[:n], c.seq_lens[:n], c.num_q_heads)


def _check_select_forms(wl, units, n_sub):
    """spdec_select_pages in the form its shape takes (the step's rule, full workspace) against the two kernels
    (scores to scores_out, no workspace: a scoring and a Top-k kernel for every shape the one-kernel form does not
    take; for one-kernel shapes, the first n_sub sequences as a batch of their own): sel_cnt, sel_idx and scores
    bit for bit; sampled units against the oracle's scores and the Top-B rule."""
    dw = GS.DeviceWorkload(wl)
    c = dw.cache
    spdec.build_meta(c)
    form = _form(dw)
    assert spdec.select_pages_form(c, dw.max_budget) == form
    ws = torch.full((spdec.select_workspace_bytes(c, dw.max_budget),), 0xA5, dtype=torch.uint8, device=c.device)
    shape = (c.batch, c.num_kv_heads, c.max_pages)
    sc_a = torch.full(shape, float("nan"), dtype=torch.float32, device=c.device)
    idx_a, cnt_a = spdec.select_pages(c, dw.q, dw.budget, dw.max_budget, scores_out=sc_a, workspace=ws)
    idx_b, cnt_b = spdec.select_pages(c, dw.q, dw.budget, dw.max_budget, workspace=ws)
    sc_c = torch.full(shape, float("nan"), dtype=torch.float32, device=c.device)
    if form == "one kernel":
        sub = _sub_cache(c, n_sub)
        assert spdec.select_pages_form(sub, dw.max_budget) != "one kernel"
        idx_c, cnt_c = spdec.select_pages(sub, dw.q[:n_sub], dw.budget[:n_sub], dw.max_budget,
                                          scores_out=sc_c[:n_sub])
        nb = n_sub
    else:
        idx_c, cnt_c = spdec.select_pages(c, dw.q, dw.budget, dw.max_budget, scores_out=sc_c)
        nb = c.batch
    torch.cuda.synchronize()
    ca, cb, cc = cnt_a.cpu().numpy(), cnt_b.cpu().numpy(), cnt_c.cpu().numpy()
    ia, ib, ic = idx_a.cpu().numpy(), idx_b.cpu().numpy(), idx_c.cpu().numpy()
    sa, scc = sc_a.cpu().numpy(), sc_c.cpu().numpy()
    assert np.array_equal(ca, cb) and np.array_equal(ca[:nb], cc)
    for b in range(c.batch):
        P = wl.pages(b)
        if b < nb:
            assert np.array_equal(sa[b, :, :P].view(np.uint32), scc[b, :, :P].view(np.uint32)), b
        for g in range(c.num_kv_heads):
            k = int(ca[b, g])
            assert np.array_equal(ia[b, g, :k], ib[b, g, :k]), (b, g)
            if b < nb:
                assert np.array_equal(ia[b, g, :k], ic[b, g, :k]), (b, g)
    for (b, g) in units:
        K64, _ = GS.unit_kv_f64(wl, b, g)
        s64 = GS.oracle_scores(wl, b, g, K64)
        GS.check_selection(ia[b, g], int(ca[b, g]), s64, int(wl.budget_pages[b]), dw.max_budget)
    say(f"  {wl.spec.name}: select {form}: equal to the two kernels on {nb} of {c.batch} sequences; "
        f"{len(units)} units vs oracle")


@pytest.mark.parametrize("case", [("one kernel", i) for i in range(len(CASES))] +
                         [("sliced", i) for i in range(len(SLICED))])
def test_select_forms_match_two_kernels_and_oracle(case):
    """spdec_select_pages in its fused forms (one kernel for batches of at least one unit per compute unit,
    sliced for few units) selects and scores exactly as its scoring and Top-k kernels do."""
    kind, i = case
    if kind == "one kernel":
        name, D, Hq, Hkv, ps, B, (lo, hi), (blo, bhi), zeros = CASES[i]
        lens = _lens(i, B, lo, hi, zeros)
        bud = [int(x) for x in np.random.default_rng(100 + i).integers(blo, bhi + 1, B)]
        seed = i
    else:
        name, D, Hq, Hkv, ps, B, (lo, hi), bud, zeros = SLICED[i]
        lens = _lens(500 + i, B, lo, hi, zeros)
        seed = 500 + i
    say(f"case select forms {kind} {name}: batch {B}")
    spec = S.custom_spec(f"select-{kind[0]}{i}", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                         page_size=ps, dtype="bf16", lens=("list", lens), budget=("pages", bud), outlier_channels=4)
    wl = S.make_workload(spec, seed=seed)
    # a sub-batch of at most 128 units runs the two kernels when its scores go to scores_out
    _check_select_forms(wl, GS.sample_units(wl, 12, seed=seed), n_sub=max(1, min(B, 120 // Hkv)))


LONG = ["long-131k-ps8", "long-131k-ps16", "long-131k-ps32", "long-131k-ps64"]


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", LONG)
def test_sliced_step_full_size(name):
    """The 131K-token cache at every page size (4 sequences, 32 units): the sliced form, every unit against the
    two calls, sampled units against the oracle, and the planted block kept."""
    say(f"case sliced full-size {name}: generating")
    wl = S.make_workload(name, seed=0, build_pool=True)
    dw = _run(wl, GS.sample_units(wl, 6, seed=4), expect_form="sliced")
    sel_idx, sel_cnt = spdec.select_pages(dw.cache, dw.q, dw.budget, dw.max_budget)
    si, sc = sel_idx.cpu().numpy(), sel_cnt.cpu().numpy()
    ps = wl.spec.page_size
    for b in range(wl.spec.batch):
        for g in range(wl.spec.num_kv_heads):
            s0 = int(wl.plant_start[b, g])
            pages = set(range(s0 // ps, (s0 + wl.spec.planted_block - 1) // ps + 1))
            assert pages <= set(si[b, g, :sc[b, g]].tolist()), (b, g)
    torch.cuda.empty_cache()


FULL = ["qwen3-8b-ragged", "qwen3-1.7b-L16k", "qwen3-8b-L32k-acceptance"]


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL)
def test_step_full_size(name):
    """The full-size workloads that take the one-kernel form: every unit against the two calls, sampled units
    against the oracle."""
    say(f"case path full-size {name}: generating")
    wl = S.make_workload(name, seed=0, build_pool=True)
    _run(wl, GS.sample_units(wl, 24, seed=3), expect_form="one kernel")
    torch.cuda.empty_cache()


def test_step_repeat_is_bitwise():
    """Two steps on the same inputs write the same bits (no atomics, fixed orders)."""
    B = 40
    spec = S.custom_spec("path-repeat", batch=B, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                         dtype="bf16", lens=("list", _lens(31, B, 1, 8000, 1)),
                         budget=("pages", [int(x) for x in np.random.default_rng(32).integers(0, 200, B)]),
                         outlier_channels=4)
    wl = S.make_workload(spec, seed=31)
    dw = GS.DeviceWorkload(wl)
    spdec.build_meta(dw.cache)
    say("case path repeat")
    r1 = [t.clone() for t in spdec.sparse_path(dw.cache, dw.q, dw.budget, dw.max_budget)]
    r2 = spdec.sparse_path(dw.cache, dw.q, dw.budget, dw.max_budget)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b)
