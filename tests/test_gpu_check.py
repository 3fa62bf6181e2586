"""GPU tests of the device-side precondition checker (``spdec_check_inputs``).

The expected counts come from a plain NumPy restatement of the documented
preconditions. Planted violations (bad lengths, page-table entries outside the
pool, malformed selections, non-finite queries, groups whose shared pages
differ) go only to the checker, which reads the page table, lengths,
selection, query and shared-page counts inside their declared extents and
never dereferences the values it reads; no other kernel sees them.
"""
import math
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


def expected(lens, pt, num_phys, ps, q_bits=None, dtype="bf16", sel_idx=None, sel_cnt=None, max_budget=0,
             group=1, shared=None):
    batch, maxp = pt.shape
    counts = [0] * 5
    bad = set()
    for b in range(batch):
        L = int(lens[b])
        Lc = min(max(L, 0), maxp * ps)
        if Lc != L:
            counts[0] += 1
            bad.add(b)
        P = -(-Lc // ps)
        nb = int(np.sum((pt[b, :P] < 0) | (pt[b, :P] >= num_phys)))
        counts[1] += nb
        if nb:
            bad.add(b)
        if sel_idx is not None:
            for g in range(sel_cnt.shape[1]):
                cnt = int(sel_cnt[b, g])
                rb = cnt < 0 or cnt > min(P, max_budget)
                s = sel_idx[b, g, :min(max(cnt, 0), max_budget)].astype(np.int64)
                rb = rb or bool(np.any(s < 0) or np.any(s >= P) or np.any(np.diff(s) <= 0))
                if rb:
                    counts[2] += 1
                    bad.add(b)
        if q_bits is not None:
            x = q_bits[b].reshape(-1)
            exp_mask = 0x7F80 if dtype == "bf16" else 0x7F800000
            nf = int(np.sum((x & exp_mask) == exp_mask))
            counts[3] += nf
            if nf:
                bad.add(b)
        if shared is not None and b % group == 0:
            Sn = int(shared[b // group])
            gb = Sn < 0 or Sn > maxp
            Sc = min(max(Sn, 0), maxp)
            for m in range(group):
                Lm = min(max(int(lens[b + m]), 0), maxp * ps)
                gb = gb or Sc * ps > Lm or bool(np.any(pt[b + m, :Sc] != pt[b, :Sc]))
            if gb:
                counts[4] += 1
                bad.add(b)
    return counts + [min(bad) if bad else batch]


def _cache(pt, lens, num_phys, hkv, hq, d, ps, dtype=torch.bfloat16):
    # the checker never reads the pools or summaries: small placeholders of the declared shape
    pool = torch.zeros((num_phys, hkv, ps, d), dtype=dtype, device="cuda")
    kmm = torch.zeros((num_phys, hkv, 2, d), dtype=dtype, device="cuda")
    return spdec.PagedCache(pool, pool.clone(), kmm, torch.from_numpy(pt.astype(np.int32)).cuda(),
                            torch.from_numpy(lens.astype(np.int32)).cuda(), hq)


def _report(cache, **kw):
    r = spdec.check_inputs(cache, **kw)
    return [r[k] for k in spdec.CHECK_FIELDS]


def _valid_selection(rng, lens, ps, hkv, max_budget):
    batch = len(lens)
    idx = np.zeros((batch, hkv, max_budget), dtype=np.int32)
    cnt = np.zeros((batch, hkv), dtype=np.int32)
    for b in range(batch):
        P = -(-int(lens[b]) // ps)
        for g in range(hkv):
            k = int(rng.integers(0, min(P, max_budget) + 1))
            idx[b, g, :k] = np.sort(rng.choice(P, size=k, replace=False))
            cnt[b, g] = k
    return idx, cnt


@pytest.mark.parametrize("seed", range(6))
def test_check_counts_planted_violations(seed):
    rng = np.random.default_rng(700 + seed)
    batch, hkv, G, d = 12, 2, int(rng.choice([1, 4, 8])), int(rng.choice([64, 128]))
    ps, maxp, num_phys, max_budget, group = int(rng.choice([8, 16, 64])), 24, 300, 10, 3
    dtype = "bf16" if seed % 2 == 0 else "f32"
    lens = rng.integers(0, maxp * ps + 1, size=batch)
    pt = rng.integers(0, num_phys, size=(batch, maxp)).astype(np.int64)
    shared = rng.integers(0, 5, size=batch // group)
    for n in range(batch // group):  # members share their group's first shared[n] pages, all full
        b0 = n * group
        for m in range(group):
            lens[b0 + m] = max(int(lens[b0 + m]), int(shared[n]) * ps)
            pt[b0 + m, :shared[n]] = pt[b0, :shared[n]]
    sel_idx, sel_cnt = _valid_selection(rng, lens, ps, hkv, max_budget)
    if dtype == "bf16":
        q_bits = S.f32_to_bf16_bits(rng.standard_normal((batch, G * hkv, d), dtype=np.float32))
        specials = [0x7F80, 0xFF80, 0x7FC0, 0x7F81]
    else:
        q_bits = rng.standard_normal((batch, G * hkv, d), dtype=np.float32).view(np.uint32)
        specials = [0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001]
    assert expected(lens, pt, num_phys, ps, q_bits, dtype, sel_idx, sel_cnt, max_budget, group, shared) == \
        [0, 0, 0, 0, 0, batch]

    # plant one kind of violation per affected sequence, all after the first few sequences
    lens[5], lens[9] = (-3, maxp * ps + 1) if seed % 2 else (-2**31, 2**31 - 1)
    b = 6
    P = -(-int(lens[b]) // ps)
    if P:
        pt[b, int(rng.integers(0, P))] = num_phys
    if P < maxp:
        pt[b, P:] = -7  # pages past the length are not in use: not counted
    sel_cnt[7, 1] = min(-(-int(lens[7]) // ps), max_budget) + 1
    if sel_cnt[8, 0] >= 2:
        sel_idx[8, 0, 1] = sel_idx[8, 0, 0]  # a repeated page
    sel_idx[10, 1, :] = -1
    sel_cnt[10, 1] = 1
    for i, v in enumerate(specials):  # four distinct positions
        q_bits[11, i % (G * hkv), i] = v
    shared[1] = maxp + 1 if seed % 2 else 2**31 - 1
    sel_cnt[4, 0] = -2**31
    pt[batch - 1, 0] = (pt[batch - 1, 0] + 1) % num_phys if shared[-1] > 0 else pt[batch - 1, 0]

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cache = _cache(pt, lens, num_phys, hkv, G * hkv, d, ps, tdt)
    qd = GS.to_device_storage(q_bits.view(np.float32) if dtype == "f32" else q_bits, dtype)
    want = expected(lens, pt, num_phys, ps, q_bits, dtype, sel_idx, sel_cnt, max_budget, group, shared)
    got = _report(cache, q=qd, sel_idx=torch.from_numpy(sel_idx).cuda(), sel_cnt=torch.from_numpy(sel_cnt).cuda(),
                  max_budget_pages=max_budget, group_size=group,
                  shared_pages=torch.from_numpy(shared.astype(np.int32)).cuda())
    print(f"seed {seed} {dtype} G={G} d={d} ps={ps}: want {want} got {got}", flush=True)
    assert got == want
    # group 1 (sequences 3..5) holds the first violation
    assert want[0] == 2 and want[3] == len(specials) and want[4] >= 1 and want[5] == 3
    # each part alone (null pointers skip their checks)
    assert _report(cache) == expected(lens, pt, num_phys, ps)
    assert _report(cache, q=qd) == expected(lens, pt, num_phys, ps, q_bits, dtype)


def test_selection_written_by_select_pages_passes():
    """What spdec_select_pages writes meets the selection precondition on every row, with ragged lengths,
    lengths of zero and budgets at and above the page counts."""
    spec = S.custom_spec("check-sel", batch=9, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                         dtype="bf16", lens=("uniform", 0, 700), budget=("tokens", 160), outlier_channels=2)
    wl = S.make_workload(spec, seed=3)
    wl.lens[2] = 0
    dw = GS.DeviceWorkload(wl)
    spdec.build_meta(dw.cache)
    for cap in (2, 10, 64):
        budget = torch.full((spec.batch,), cap, dtype=torch.int32, device="cuda")
        si, sc = spdec.select_pages(dw.cache, dw.q, budget, cap)
        got = _report(dw.cache, q=dw.q, sel_idx=si, sel_cnt=sc, max_budget_pages=cap)
        assert got == [0, 0, 0, 0, 0, spec.batch], (cap, got)


def test_check_is_repeatable_and_overwrites_the_report():
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 200, size=5)
    pt = rng.integers(0, 50, size=(5, 16))
    pt[3, 0] = 99
    cache = _cache(pt, lens, 50, 2, 4, 64, 16)
    report = torch.full((spdec.SPDEC_CHECK_WORDS,), 12345, dtype=torch.int32, device="cuda")
    for _ in range(3):
        r = spdec.check_inputs(cache, report=report)
        assert [r[k] for k in spdec.CHECK_FIELDS] == [0, 1, 0, 0, 0, 3]
        assert report[6:].cpu().tolist() == [0, 0]


def test_check_replays_from_a_graph():
    """The checker captured into a HIP graph (its report cleared by a kernel, not a memset) gives the eager
    counts on every replay, also after the inputs change between replays."""
    import ctypes
    rng = np.random.default_rng(9)
    lens = rng.integers(1, 300, size=6)
    pt = rng.integers(0, 64, size=(6, 20))
    pt[2, 0] = 64
    cache = _cache(pt, lens, 64, 2, 8, 64, 16)
    report = torch.zeros(spdec.SPDEC_CHECK_WORDS, dtype=torch.int32, device="cuda")
    L = spdec.lib()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        st = L.spdec_check_inputs(ctypes.byref(cache.desc), None, None, None, 0, 1, None,
                                  ctypes.c_void_p(report.data_ptr()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == spdec.SPDEC_OK
    for rep in range(3):
        if rep == 2:  # one more bad length between replays
            cache.seq_lens[4] = -1
            torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = report.cpu().tolist()
        eager = spdec.check_inputs(cache)
        assert got[:6] == [eager[k] for k in spdec.CHECK_FIELDS], (rep, got)
        assert got[:2] == ([0, 1] if rep < 2 else [1, 1]) and got[5] == 2
