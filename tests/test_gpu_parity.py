"""GPU parity: every ABI call against the CPU oracle, element by element.

Small and edge-case shapes are checked on every (sequence, KV head); the
full-size workloads on sampled units (the oracle computes them one by one)
plus properties checked on every unit. Bars: metadata bit-exact; page sets
exact outside the 1e-6 score band around the cut; outputs within 1e-5 (fp32)
or 1e-2 (bf16) max-abs; acceptance within 1e-5.
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


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(spdec.LIB_PATH):
        from sparse_attention_decode_page_amd import build
        build.build()
    spdec.lib()
    assert torch.cuda.is_available()


# Host-side state of the case being checked, read by _unit_errors in this process or in forked workers.
_CTX = {}
# Forked numpy-only workers for the oracle side of the full-size cases: children of this process hold its
# device file open, so parent and workers stay within the GPU machine's 16 processes per GPU.
MAX_WORKERS = 12


def _unit_errors(bg):
    """Oracle comparison of one (sequence, KV head): metadata bit-exact, scores within 1.2e-7 relative, page set
    valid under the tie band, sparse and dense attention within the dtype's bar. Returns the unit's errors."""
    b, g = bg
    wl, meta, dw_max_budget = _CTX["wl"], _CTX["meta"], _CTX["max_budget"]
    sel_idx_h, sel_cnt_h, scores_h = _CTX["sel_idx"], _CTX["sel_cnt"], _CTX["scores"]
    out_s_h, lse_s_h, out_d_h, lse_d_h = _CTX["out_s"], _CTX["lse_s"], _CTX["out_d"], _CTX["lse_d"]
    spec = wl.spec
    ps, G = spec.page_size, spec.group
    tol = GS.TOL_OUT[spec.dtype]
    scale = GS.default_scale(wl)
    K64, V64 = GS.unit_kv_f64(wl, b, g)
    P = wl.pages(b)
    # metadata: bit-exact (compared as decoded values)
    kmin, kmax = O.page_minmax(K64, ps)
    phys = wl.page_table[b, :P]
    gmin = O.to_f64(meta[phys, g, 0], spec.dtype)
    gmax = O.to_f64(meta[phys, g, 1], spec.dtype)
    assert np.array_equal(gmin, kmin) and np.array_equal(gmax, kmax), (b, g)
    # scores within the fp32 band, page set valid under the tie rule
    qg = GS.q_group_f64(wl, b, g)
    s64 = O.page_scores(qg, kmin, kmax)
    # fp32 scores are the fp64-accumulated bound rounded once: within 2^-23 of each page's own score
    err = float((np.abs(scores_h[b, g, :P] - s64) / np.maximum(np.abs(s64), 1e-30)).max()) if P else 0.0
    assert err <= 1.2e-7, (b, g, err)
    cnt = int(sel_cnt_h[b, g])
    GS.check_selection(sel_idx_h[b, g], cnt, s64, int(wl.budget_pages[b]), dw_max_budget)
    # attention over the GPU's page set, and over all pages
    o, lse = O.decode_unit(qg, K64, V64, sel_idx_h[b, g, :cnt], ps, scale)
    es = float(np.abs(out_s_h[b, g * G:(g + 1) * G] - o).max())
    els = float(np.abs(lse_s_h[b, g * G:(g + 1) * G] - lse).max()) if P else 0.0
    assert es <= tol and els <= tol, (b, g, es, els)
    o, lse = O.dense_decode_unit(qg, K64, V64, ps, scale)
    ed = float(np.abs(out_d_h[b, g * G:(g + 1) * G] - o).max())
    eld = float(np.abs(lse_d_h[b, g * G:(g + 1) * G] - lse).max()) if P else 0.0
    assert ed <= tol and eld <= tol, (b, g, ed, eld)
    return {"score": err, "sparse": es, "dense": ed, "lse": max(els, eld)}


def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _check_units(units, workers):
    if workers <= 1 or len(units) < 16:
        return [_unit_errors(u) for u in units]
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    with ProcessPoolExecutor(workers, mp_context=mp.get_context("fork"), initializer=_one_blas_thread) as ex:
        return list(ex.map(_unit_errors, units, chunksize=max(1, len(units) // (4 * workers))))


def _check_path(wl, units, full_units_props=True, workers=1):
    """Run build_meta -> select -> sparse -> dense on the GPU and check `units` against the oracle."""
    spec = wl.spec
    dw = GS.DeviceWorkload(wl)
    c = dw.cache
    spdec.build_meta(c)
    sel_idx, sel_cnt, scores = GS.run_select(dw)
    # the inputs meet the documented preconditions and the selection has the form the decode takes
    pre = spdec.check_inputs(c, q=dw.q, sel_idx=sel_idx, sel_cnt=sel_cnt, max_budget_pages=dw.max_budget)
    assert pre["first_bad_sequence"] == spec.batch, pre
    out_s, lse_s = spdec.sparse_decode(c, dw.q, sel_idx, sel_cnt, dw.max_budget)
    out_d, lse_d = spdec.dense_decode(c, dw.q)
    torch.cuda.synchronize()
    meta = GS.from_device_storage(dw.kminmax, spec.dtype)
    sel_idx_h, sel_cnt_h = sel_idx.cpu().numpy(), sel_cnt.cpu().numpy()
    out_s_h, lse_s_h = out_s.cpu().numpy(), lse_s.cpu().numpy()
    out_d_h, lse_d_h = out_d.cpu().numpy(), lse_d.cpu().numpy()
    assert np.all(np.isfinite(out_s_h)) and np.all(np.isfinite(out_d_h))
    live = wl.lens > 0  # a sequence with no token has lse = -inf
    assert np.all(np.isfinite(lse_s_h[live])) and np.all(np.isfinite(lse_d_h[live]))
    if full_units_props:
        for b in range(spec.batch):
            P = wl.pages(b)
            for g in range(spec.num_kv_heads):
                K = GS.expected_count(P, int(wl.budget_pages[b]), dw.max_budget)
                assert sel_cnt_h[b, g] == K
                row = sel_idx_h[b, g, :K]
                assert np.all(np.diff(row) > 0) and row[0] == 0 and row[-1] == P - 1
    _CTX.clear()
    _CTX.update(wl=wl, meta=meta, max_budget=dw.max_budget, sel_idx=sel_idx_h, sel_cnt=sel_cnt_h,
                scores=scores.cpu().numpy(), out_s=out_s_h, lse_s=lse_s_h, out_d=out_d_h, lse_d=lse_d_h)
    try:
        errs = _check_units(list(units), workers)
    finally:
        _CTX.clear()
    worst = {k: max((e[k] for e in errs), default=0.0) for k in ("score", "sparse", "dense", "lse")}
    say(f"  {spec.name}: {len(units)} units checked, worst {worst}")
    return dw, sel_idx_h, sel_cnt_h


# ------------------------------------------------------------- small cases ---

def test_tiny_all_units():
    say("case tiny (fp32, D 64, G 2, 1024 tokens, page size 16, budget 16 pages)")
    wl = S.make_workload("tiny", seed=0)
    _check_path(wl, GS.sample_units(wl, 10 ** 9))


EDGE = [
    # dtype, D, Hq, Hkv, ps, lens, budget pages
    ("f32", 64, 2, 2, 16, [1, 2, 15, 16, 17, 33], [16, 16, 16, 2, 3, 2]),
    ("f32", 128, 8, 1, 8, [100, 257, 64], [5, 9, 8]),
    ("bf16", 128, 4, 4, 16, [1, 16, 17, 300, 511, 1000], [2, 2, 2, 7, 12, 40]),
    ("bf16", 64, 16, 2, 32, [33, 64, 65, 2000], [2, 3, 4, 20]),
    ("bf16", 128, 16, 2, 64, [64, 65, 129, 4100], [2, 2, 3, 30]),
    ("bf16", 128, 8, 1, 8, [9, 800, 4095], [2, 50, 300]),
    ("bf16", 128, 32, 8, 16, [5000, 7777], [1, 600]),
    # many short sequences: 640 units (15 partial slots per unit) and 300 units (30 slots) take the
    # merge's 64- and 128-thread forms
    ("bf16", 128, 32, 8, 16, [int(x) for x in np.random.default_rng(77).integers(1, 1200, 80)],
     [int(x) for x in np.random.default_rng(78).integers(0, 40, 80)]),
    ("bf16", 128, 16, 4, 16, [int(x) for x in np.random.default_rng(79).integers(1, 1200, 75)],
     [int(x) for x in np.random.default_rng(80).integers(0, 40, 75)]),
]


@pytest.mark.parametrize("case", range(len(EDGE)))
@pytest.mark.parametrize("seed", [0, 1])
def test_edge_shapes_all_units(case, seed):
    dt, D, Hq, Hkv, ps, lens, bud = EDGE[case]
    say(f"case edge {case} seed {seed}: {dt} D{D} Hq{Hq}/Hkv{Hkv} ps{ps} lens {lens} budget {bud}")
    spec = S.custom_spec(f"edge{case}", batch=len(lens), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                         page_size=ps, dtype=dt, lens=("list", lens), budget=("pages", bud),
                         outlier_channels=4 if dt == "bf16" else 0)
    wl = S.make_workload(spec, seed=seed, headroom=ps)
    _check_path(wl, GS.sample_units(wl, 10 ** 9))


def _random_shape(seed):
    r = np.random.default_rng(1000 + seed)
    dt = "f32" if r.random() < 0.3 else "bf16"
    D = int(r.choice([64, 128]))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 8]))
    ps = int(r.choice([8, 16, 32, 64]))
    B = int(r.integers(1, 6))
    # lengths anywhere up to 60 pages, half of them on or next to a page boundary
    lens = [int(r.integers(1, 60 * ps)) if r.random() < 0.5 else max(1, int(r.integers(0, 40)) * ps + int(r.integers(-1, 2)))
            for _ in range(B)]
    budget = [int(r.integers(0, 40)) for _ in range(B)]
    return dt, D, Hkv * G, Hkv, ps, lens, budget


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_all_units(seed):
    """Seeded random shapes (dtype, head dim, group, page size, ragged lengths on and off page boundaries,
    budgets from 0 to 39 pages), every unit against the oracle."""
    dt, D, Hq, Hkv, ps, lens, bud = _random_shape(seed)
    say(f"case random {seed}: {dt} D{D} Hq{Hq}/Hkv{Hkv} ps{ps} lens {lens} budget {bud}")
    spec = S.custom_spec(f"rand{seed}", batch=len(lens), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                         page_size=ps, dtype=dt, lens=("list", lens), budget=("pages", bud),
                         outlier_channels=4 if dt == "bf16" else 0)
    wl = S.make_workload(spec, seed=seed, headroom=int(np.random.default_rng(seed).integers(0, 3 * ps)))
    _check_path(wl, GS.sample_units(wl, 10 ** 9))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_empty_sequences(dt):
    """Sequences holding no token: no page is kept, the outputs are zeros and lse is -inf (an empty softmax
    sum), and the other sequences of the batch are unaffected."""
    say(f"case empty sequences ({dt})")
    spec = S.custom_spec(f"empty-{dt}", batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, dtype=dt,
                         lens=("list", [0, 40, 0, 300]), budget=("pages", [4, 4, 4, 6]),
                         outlier_channels=4 if dt == "bf16" else 0)
    wl = S.make_workload(spec, seed=12, headroom=16)
    dw, sel_idx_h, sel_cnt_h = _check_path(wl, [(1, 0), (1, 1), (3, 0), (3, 1)], full_units_props=False)
    assert np.all(sel_cnt_h[[0, 2]] == 0)
    out_s, lse_s = spdec.sparse_decode(dw.cache, dw.q, torch.from_numpy(sel_idx_h).cuda(),
                                       torch.from_numpy(sel_cnt_h).cuda(), dw.max_budget)
    out_d, lse_d = spdec.dense_decode(dw.cache, dw.q)
    torch.cuda.synchronize()
    for o, l in ((out_s, lse_s), (out_d, lse_d)):
        assert torch.all(o[[0, 2]] == 0) and torch.all(torch.isneginf(l[[0, 2]]))
        assert torch.all(torch.isfinite(l[[1, 3]]))


def test_more_units_than_the_stream_grid_holds():
    """More (sequence, KV head) units than the persistent grids' unit table holds (8192): scoring falls back to
    one workgroup per (unit, page block) and the decode to fixed splits; both must still match the oracle."""
    spec = S.custom_spec("many-units", batch=1040, num_q_heads=8, num_kv_heads=8, head_dim=64, page_size=16,
                         dtype="bf16", lens=("uniform", 1, 160), budget=("tokens", 48), outlier_channels=2)
    wl = S.make_workload(spec, seed=4)
    assert spec.batch * spec.num_kv_heads > 8192
    say("case many-units: 1040 x 8 units")
    _check_path(wl, GS.sample_units(wl, 48, seed=4))


def test_eight_query_heads_per_kv_head_many_chunks():
    """G = 8 (64 query / 8 KV heads, D 128: the two-set MFMA form of the stream decode) on lists long enough
    that every unit is split over several waves and merged."""
    spec = S.custom_spec("g8", batch=6, num_q_heads=64, num_kv_heads=8, head_dim=128, page_size=16, dtype="bf16",
                         lens=("uniform", 3000, 20000), budget=("tokens", 2048), outlier_channels=4)
    wl = S.make_workload(spec, seed=8)
    say("case G8: 6 x 8 units, 64/8 heads")
    _check_path(wl, GS.sample_units(wl, 12, seed=8))



@pytest.mark.parametrize("tokens", [131100, 262144])
def test_longest_page_tables(tokens):
    """Page tables of 16388 pages and of 32768, the largest the interface takes (page size 8): the Top-B cut
    with 32 keys per thread in 1024-thread workgroups, scoring and both decodes over the longest lists."""
    spec = S.custom_spec(f"longest{tokens}", batch=1, num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=8,
                         dtype="bf16", lens=("fixed", tokens), budget=("tokens", 2048), outlier_channels=2)
    wl = S.make_workload(spec, seed=12)
    assert wl.page_table.shape[1] in (16388, 32768)
    say(f"case longest page table: {wl.page_table.shape[1]} pages")
    _check_path(wl, [(0, 0), (0, 1)])

def test_exact_ties_go_to_lower_index():
    """Pages with identical keys tie exactly in fp32 and fp64; the lower index must win."""
    say("case exact ties")
    spec = S.custom_spec("ties", batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, dtype="bf16",
                         lens=("list", [16 * 40, 16 * 33 + 5]), budget=("pages", [10, 7]))
    wl = S.make_workload(spec, seed=3, headroom=0)
    ps = 16
    rng = np.random.default_rng(9)
    for b in range(2):
        P = wl.pages(b)
        templ = rng.integers(0, 4, size=P)  # page p copies template page templ[p]
        for g in range(2):
            for p in range(1, P - 1):
                src = wl.page_table[b, 1 + templ[p]]
                dst = wl.page_table[b, p]
                if dst != src:
                    wl.k_pool[dst, g] = wl.k_pool[src, g]
    dw, sel_idx_h, sel_cnt_h = _check_path(wl, GS.sample_units(wl, 10 ** 9))
    for b in range(2):
        for g in range(2):
            K64, _ = GS.unit_kv_f64(wl, b, g)
            s64 = GS.oracle_scores(wl, b, g, K64)
            want = O.select_pages(s64, int(wl.budget_pages[b]))
            got = sel_idx_h[b, g, :sel_cnt_h[b, g]]
            assert got.tolist() == want.tolist(), (b, g)


def test_full_budget_sparse_equals_dense_bitwise():
    say("case full budget == dense")
    spec = S.custom_spec("full", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, dtype="bf16",
                         lens=("list", [1000, 1024, 37]), budget=("pages", [64, 64, 64]))
    wl = S.make_workload(spec, seed=1)
    dw = GS.DeviceWorkload(wl)
    c = dw.cache
    spdec.build_meta(c)
    cap = c.max_pages
    sel_idx, sel_cnt = spdec.select_pages(c, dw.q, dw.budget, cap)
    o_s, l_s = spdec.sparse_decode(c, dw.q, sel_idx, sel_cnt, cap)
    o_d, l_d = spdec.dense_decode(c, dw.q)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_d) and torch.equal(l_s, l_d)


def test_determinism_bitwise():
    say("case determinism")
    wl = S.make_workload(S.custom_spec("det", batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                                       dtype="bf16", lens=("list", [3000, 9000, 17, 12345]),
                                       budget=("pages", [64, 100, 4, 256]), outlier_channels=4), seed=2)
    dw = GS.DeviceWorkload(wl)
    c = dw.cache
    spdec.build_meta(c)
    runs = []
    for _ in range(3):
        si, sc, scores = GS.run_select(dw)
        o, l = spdec.sparse_decode(c, dw.q, si, sc, dw.max_budget)
        od, ld = spdec.dense_decode(c, dw.q)
        torch.cuda.synchronize()
        runs.append([t.clone() for t in (si, sc, scores, o, l, od, ld)])
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)



def test_reused_decode_workspace_across_calls():
    """One decode workspace across calls whose units have many, few and no chunks (selections of the full
    budget, of two pages, and counts cut to zero on some units), then a dense call: every result equals the same
    call on a fresh workspace bit for bit (no chunk count or partial survives from an earlier call)."""
    say("case reused decode workspace")
    spec = S.custom_spec("reuse", batch=5, num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=16, dtype="bf16",
                         lens=("list", [4000, 700, 2500, 33, 1800]), budget=("pages", [120, 30, 90, 4, 60]),
                         outlier_channels=2)
    wl = S.make_workload(spec, seed=14)
    dw = GS.DeviceWorkload(wl)
    c = dw.cache
    spdec.build_meta(c)
    cap = dw.max_budget
    nbytes = max(spdec.decode_workspace_bytes(c, cap), spdec.decode_workspace_bytes(c, 0))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    calls = []
    for budget in (dw.budget, torch.full_like(dw.budget, 2), dw.budget):
        si, sc = spdec.select_pages(c, dw.q, budget, cap)
        calls.append((si, sc))
    si, sc = calls[0]
    sc_cut = sc.clone()
    sc_cut[1] = 0
    sc_cut[3, :2] = 0
    calls.append((si, sc_cut))
    for k, (si, sc) in enumerate(calls):
        o1, l1 = spdec.sparse_decode(c, dw.q, si, sc, cap, workspace=ws)
        o2, l2 = spdec.sparse_decode(c, dw.q, si, sc, cap)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), k
    od1, ld1 = spdec.dense_decode(c, dw.q, workspace=ws)
    od2, ld2 = spdec.dense_decode(c, dw.q)
    torch.cuda.synchronize()
    assert torch.equal(od1, od2) and torch.equal(ld1, ld2)
    # units whose count was cut to zero attend over nothing: zeros and lse = -inf
    o, l = spdec.sparse_decode(c, dw.q, si, sc_cut, cap, workspace=ws)
    torch.cuda.synchronize()
    G = spec.group
    assert torch.all(o[1] == 0) and torch.all(torch.isneginf(l[1]))
    assert torch.all(o[3, :2 * G] == 0) and torch.all(torch.isneginf(l[3, :2 * G]))
    assert torch.all(torch.isfinite(l[3, 2 * G:]))

def test_physical_placement_invariance():
    say("case physical permutation")
    spec = S.custom_spec("perm", batch=3, num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=16, dtype="bf16",
                         lens=("list", [500, 2048, 1111]), budget=("pages", [8, 30, 20]))
    wl = S.make_workload(spec, seed=4)
    outs = []
    for variant in range(2):
        if variant == 1:
            perm = np.random.default_rng(77).permutation(wl.num_phys)
            kp, vp = np.empty_like(wl.k_pool), np.empty_like(wl.v_pool)
            kp[perm] = wl.k_pool
            vp[perm] = wl.v_pool
            pt = np.where(wl.page_table >= 0, perm[np.maximum(wl.page_table, 0)], -1).astype(np.int32)
            wl.k_pool, wl.v_pool, wl.page_table = kp, vp, pt
        dw = GS.DeviceWorkload(wl)
        spdec.build_meta(dw.cache)
        si, sc, scores = GS.run_select(dw)
        o, l = spdec.sparse_decode(dw.cache, dw.q, si, sc, dw.max_budget)
        od, ld = spdec.dense_decode(dw.cache, dw.q)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (si, sc, o, l, od, ld)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)



@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_pools_past_four_gib(dt):
    """The same pages placed past 2^31 pool elements (byte offsets past 4 GiB, as a 288 GB device allows):
    build, append, selection, both decodes and the verification give the bits they give on a compact pool."""
    say(f"case pools past 2^31 elements, {dt}")
    spec = S.custom_spec("far", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, dtype=dt,
                         lens=("list", [700, 1500, 33]), budget=("pages", [8, 20, 64]), outlier_channels=2)
    wl = S.make_workload(spec, seed=6, headroom=16)
    off = (1 << 31) // (spec.num_kv_heads * spec.page_size * spec.head_dim) + 7
    n = wl.num_phys
    rng = np.random.default_rng(6)
    k_new32 = rng.standard_normal((spec.batch, spec.num_kv_heads, spec.head_dim), dtype=np.float32)
    v_new32 = rng.standard_normal((spec.batch, spec.num_kv_heads, spec.head_dim), dtype=np.float32)
    conv = (lambda x: S.f32_to_bf16_bits(x)) if dt == "bf16" else (lambda x: x)
    k_new, v_new = GS.to_device_storage(conv(k_new32), dt), GS.to_device_storage(conv(v_new32), dt)
    vq = None
    if dt == "bf16":
        vq = GS.to_device_storage(S.f32_to_bf16_bits(
            rng.standard_normal((spec.batch, 3, spec.num_q_heads, spec.head_dim), dtype=np.float32)), dt)

    def run(dw, far):
        c = dw.cache
        spdec.build_meta(c)
        res = list(GS.run_select(dw))
        res += list(spdec.sparse_decode(c, dw.q, res[0], res[1], dw.max_budget))
        res += list(spdec.dense_decode(c, dw.q))
        if vq is not None:
            res += list(spdec.verify_decode(c, vq))
        spdec.append_kv(c, k_new, v_new)
        res += list(spdec.dense_decode(c, dw.q))
        base = off if far else 0
        res += [dw.k_pool[base:base + n].clone(), dw.v_pool[base:base + n].clone(), dw.kminmax[base:base + n].clone()]
        torch.cuda.synchronize()
        return [t.cpu() for t in res]

    near = run(GS.DeviceWorkload(wl), False)
    dw = GS.DeviceWorkload(wl)
    tdt = dw.k_pool.dtype
    shape = (off + n,) + tuple(dw.k_pool.shape[1:])
    print(f"  far pools: {2 * shape[0] * np.prod(shape[1:]) * dw.k_pool.element_size() / 2**30:.1f} GiB", flush=True)
    kb = torch.zeros(shape, dtype=tdt, device="cuda")
    vb = torch.zeros(shape, dtype=tdt, device="cuda")
    kb[off:] = dw.k_pool
    vb[off:] = dw.v_pool
    mb = torch.zeros((off + n,) + tuple(dw.kminmax.shape[1:]), dtype=tdt, device="cuda")
    pt = torch.where(dw.page_table >= 0, dw.page_table + off, dw.page_table)
    dw.k_pool, dw.v_pool, dw.kminmax, dw.page_table = kb, vb, mb, pt
    dw.seq_lens = torch.from_numpy(wl.lens.astype(np.int32)).cuda()
    dw.cache = spdec.PagedCache(kb, vb, mb, pt, dw.seq_lens, spec.num_q_heads)
    far = run(dw, True)
    for i, (a, b) in enumerate(zip(near, far)):
        assert torch.equal(a, b), i
    del dw, kb, vb, mb
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ append ---

@pytest.mark.parametrize("dt,D,ps", [("f32", 64, 16), ("bf16", 128, 16), ("bf16", 128, 8), ("bf16", 64, 64)])
def test_append_kv_matches_oracle_and_bulk_build(dt, D, ps):
    say(f"case append {dt} D{D} ps{ps}")
    spec = S.custom_spec("append", batch=3, num_q_heads=4, num_kv_heads=2, head_dim=D, page_size=ps, dtype=dt,
                         lens=("list", [ps - 3, 2 * ps, 5 * ps + 1]), budget=("pages", [3, 3, 4]))
    steps = 2 * ps + 5
    wl = S.make_workload(spec, seed=5, headroom=steps)
    dw = GS.DeviceWorkload(wl)
    c = dw.cache
    spdec.build_meta(c)
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    lens = wl.lens.copy()
    for step in range(steps):
        kn, vn = S.append_tokens(wl, step)
        spdec.append_kv(c, GS.to_device_storage(kn, dt), GS.to_device_storage(vn, dt))
        for b in range(spec.batch):
            t = int(lens[b])
            phys = wl.page_table[b, t // ps]
            kp[phys, :, t % ps] = kn[b]
            vp[phys, :, t % ps] = vn[b]
            lens[b] += 1
    torch.cuda.synchronize()
    assert np.array_equal(dw.seq_lens.cpu().numpy(), lens)
    assert np.array_equal(GS.from_device_storage(dw.k_pool, dt), kp)
    assert np.array_equal(GS.from_device_storage(dw.v_pool, dt), vp)
    meta_inc = dw.kminmax.clone()
    spdec.build_meta(c)
    torch.cuda.synchronize()
    # incremental upkeep == bulk rebuild on the GPU, both == oracle
    assert torch.equal(meta_inc.view(torch.int16) if dt == "bf16" else meta_inc,
                       dw.kminmax.view(torch.int16) if dt == "bf16" else dw.kminmax)
    meta = GS.from_device_storage(dw.kminmax, dt)
    for b in range(spec.batch):
        P = (int(lens[b]) + ps - 1) // ps
        for g in range(spec.num_kv_heads):
            K64 = O.to_f64(O.gather_tokens(kp, wl.page_table[b], int(lens[b]), g, ps), dt)
            kmin, kmax = O.page_minmax(K64, ps)
            phys = wl.page_table[b, :P]
            assert np.array_equal(O.to_f64(meta[phys, g, 0], dt), kmin)
            assert np.array_equal(O.to_f64(meta[phys, g, 1], dt), kmax)


def test_append_skips_full_sequences():
    say("case append past capacity")
    spec = S.custom_spec("cap", batch=2, num_q_heads=2, num_kv_heads=1, head_dim=64, page_size=8, dtype="bf16",
                         lens=("list", [16, 10]), budget=("pages", [2, 2]))
    wl = S.make_workload(spec, seed=0, headroom=0)  # sequence 0 is exactly full
    dw = GS.DeviceWorkload(wl)
    kn, vn = S.append_tokens(wl, 0)
    before = dw.k_pool.clone()
    spdec.append_kv(dw.cache, GS.to_device_storage(kn, "bf16"), GS.to_device_storage(vn, "bf16"))
    torch.cuda.synchronize()
    assert dw.seq_lens.cpu().tolist() == [16, 11]
    changed = (before.view(torch.int16) != dw.k_pool.view(torch.int16)).any(dim=(1, 2, 3)).cpu().numpy()
    assert changed.sum() == 1 and changed[wl.page_table[1, 1]]


# -------------------------------------------------------------- acceptance ---

def _acc_check(a, b, T, tol=GS.TOL_ALPHA, stride=None):
    dev = "cuda"
    R, V = a.shape
    if stride is None:
        ta, tb = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    else:
        ba = torch.zeros((R, stride), dtype=torch.float32, device=dev)
        bb = torch.zeros((R, stride), dtype=torch.float32, device=dev)
        ba[:, :V] = torch.from_numpy(a)
        bb[:, :V] = torch.from_numpy(b)
        ta, tb = ba[:, :V], bb[:, :V]
    alpha = spdec.acceptance(ta, tb, T).cpu().numpy()
    want = np.array([O.acceptance(a[r], b[r], T) for r in range(R)])
    err = np.abs(alpha - want).max()
    assert err <= tol, err
    return alpha, want


def test_acceptance_tiny():
    say("case acceptance tiny")
    spec = S.SPECS["tiny"]
    a, b, _ = S.make_logits(spec, 0)
    _acc_check(a, b, spec.temperature)
    _acc_check(a, b, 0.7)
    alpha, _ = _acc_check(a, a.copy(), 1.0)
    assert np.all(np.abs(alpha - 1.0) <= 1e-6)


@pytest.mark.parametrize("V", [1, 3, 4095, 4097, 10000])
def test_acceptance_ragged_vocab_and_unaligned_rows(V):
    say(f"case acceptance V={V}")
    r = np.random.default_rng(V)
    a = (2 * r.standard_normal((5, V))).astype(np.float32)
    b = (a + r.standard_normal((5, V))).astype(np.float32)
    _acc_check(a, b, 1.0)
    _acc_check(a, b, 2.5, stride=V + 1)



def test_acceptance_reused_workspace():
    """One acceptance workspace across calls of different row counts, vocabularies and temperatures: each
    equals the same call on a fresh workspace bit for bit."""
    say("case acceptance reused workspace")
    r = np.random.default_rng(16)
    shapes = [(8, 50000, 1.0), (3, 1000, 0.7), (8, 50000, 1.3), (64, 4097, 1.0)]
    nbytes = max(spdec.acceptance_workspace_bytes(R, V) for R, V, _ in shapes)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for R, V, T in shapes:
        a = torch.from_numpy(r.normal(0, 3, (R, V)).astype(np.float32)).cuda()
        b = a + torch.from_numpy(r.normal(0, 0.3, (R, V)).astype(np.float32)).cuda()
        x1 = spdec.acceptance(a, b, T, workspace=ws)
        x2 = spdec.acceptance(a, b, T)
        torch.cuda.synchronize()
        assert torch.equal(x1, x2), (R, V, T)

def test_acceptance_full_size():
    say("case acceptance 64 x 151936")
    spec = S.SPECS["qwen3-8b-L32k-acceptance"]
    a, b, heavy = S.make_logits(spec, 0)
    alpha, want = _acc_check(a, b, spec.temperature)
    mean, p5 = O.tail_stats(alpha)
    wmean, wp5 = O.tail_stats(want)
    say(f"  mean {mean:.6f} (oracle {wmean:.6f}), p5 {p5:.6f} (oracle {wp5:.6f}), heavy rows {heavy.tolist()}")
    assert abs(mean - wmean) <= 1e-5 and abs(p5 - wp5) <= 1e-5
    assert np.all(alpha[heavy] < np.delete(alpha, heavy).min())


# --------------------------------------------------------------- full size ---

FULL = ["qwen3-1.7b-L16k", "qwen3-8b-ragged", "long-131k-ps8", "long-131k-ps16", "long-131k-ps32",
        "long-131k-ps64", "qwen3-8b-L32k-acceptance"]


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_every_unit(name):
    """The full-size workloads, every (sequence, KV head) against the oracle (forked host workers)."""
    say(f"case full-size {name}: generating")
    wl = S.make_workload(name, seed=0, build_pool=True)
    units = GS.sample_units(wl, 10 ** 9)
    workers = max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0))))
    say(f"  generated; checking all {len(units)} units with {workers} host workers")
    dw, sel_idx_h, sel_cnt_h = _check_path(wl, units, workers=workers)
    if wl.spec.planted_block:
        ps = wl.spec.page_size
        for (b, g) in units:
            s0 = int(wl.plant_start[b, g])
            pages = set(range(s0 // ps, (s0 + wl.spec.planted_block - 1) // ps + 1))
            got = set(sel_idx_h[b, g, :sel_cnt_h[b, g]].tolist())
            assert pages <= got, (b, g, sorted(pages - got))
    del dw
    torch.cuda.empty_cache()


def test_binding_rejects_bad_arguments():
    wl = S.make_workload("tiny", seed=0)
    dw = GS.DeviceWorkload(wl)
    with pytest.raises(ValueError):
        spdec.dense_decode(dw.cache, dw.q[:, :2])
    with pytest.raises(ValueError):
        spdec.select_pages(dw.cache, dw.q, dw.budget.to(torch.int64), 16)
    with pytest.raises(RuntimeError):
        spdec.dense_decode(dw.cache, dw.q, scale=-1.0)
