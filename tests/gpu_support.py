"""Helpers for the GPU parity tests: upload a synthetic workload, run the HIP
path through the binding, and compare against the CPU oracle unit by unit."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle as O
from sparse_attention_decode_page_amd import spdec
from sparse_attention_decode_page_amd import synth as S

TOL_OUT = {"f32": 1e-5, "bf16": 1e-2}
TOL_ALPHA = 1e-5
SCORE_BAND = 1e-6


def to_device_storage(x: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def from_device_storage(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class DeviceWorkload:
    """A workload resident on the GPU: cache tensors, queries, budgets."""

    def __init__(self, wl: S.Workload, dev="cuda"):
        spec = wl.spec
        self.wl = wl
        self.dtype = spec.dtype
        self.k_pool = to_device_storage(wl.k_pool, spec.dtype, dev)
        self.v_pool = to_device_storage(wl.v_pool, spec.dtype, dev)
        tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
        self.kminmax = torch.zeros((wl.num_phys, spec.num_kv_heads, 2, spec.head_dim), dtype=tdt, device=dev)
        self.page_table = torch.from_numpy(wl.page_table).to(dev)
        self.seq_lens = torch.from_numpy(wl.lens.astype(np.int32)).to(dev)
        self.q = to_device_storage(wl.q, spec.dtype, dev)
        self.budget = torch.from_numpy(wl.budget_pages.astype(np.int32)).to(dev)
        self.cache = spdec.PagedCache(self.k_pool, self.v_pool, self.kminmax, self.page_table, self.seq_lens,
                                      spec.num_q_heads)
        self.max_budget = int(max(2, wl.budget_pages.max()))


def unit_kv_f64(wl: S.Workload, b: int, g: int, k_pool=None, v_pool=None, lens=None, page_table=None):
    """Gather (K, V) of one unit from host pools via the oracle and decode to float64."""
    kp = wl.k_pool if k_pool is None else k_pool
    vp = wl.v_pool if v_pool is None else v_pool
    pt = wl.page_table if page_table is None else page_table
    L = int(wl.lens[b] if lens is None else lens[b])
    ps = wl.spec.page_size
    K = O.to_f64(O.gather_tokens(kp, pt[b], L, g, ps), wl.spec.dtype)
    V = O.to_f64(O.gather_tokens(vp, pt[b], L, g, ps), wl.spec.dtype)
    return K, V


def q_group_f64(wl: S.Workload, b: int, g: int) -> np.ndarray:
    G = wl.spec.group
    return O.to_f64(wl.q[b, g * G:(g + 1) * G], wl.spec.dtype)


def sample_units(wl: S.Workload, n: int, seed: int = 0):
    B, H = wl.spec.batch, wl.spec.num_kv_heads
    total = B * H
    if total <= n:
        return [(b, g) for b in range(B) for g in range(H)]
    r = np.random.default_rng(seed)
    picks = {0, total - 1, *r.choice(total, n - 2, replace=False).tolist()}
    return sorted(divmod(int(u), H) for u in picks)


def expected_count(P: int, budget: int, cap: int) -> int:
    return min(max(budget, 2), cap, P)


def check_selection(sel: np.ndarray, cnt: int, scores64: np.ndarray, budget: int, cap: int):
    """Validate a GPU page set against the oracle under the tie band.

    The set must have exactly K distinct ascending pages including 0 and P-1,
    contain every oracle-kept page whose score is outside the band around the
    cut, and exclude every oracle-dropped page outside that band.
    """
    P = scores64.shape[0]
    K = expected_count(P, budget, cap)
    assert cnt == K, (cnt, K)
    got = sel[:cnt].astype(np.int64)
    assert np.all(np.diff(got) > 0), "pages must be ascending and distinct"
    if K >= P:
        assert got.tolist() == list(range(P))
        return
    assert got[0] == 0 and got[-1] == P - 1
    want = O.select_pages(scores64, K)
    if K == 2:
        assert got.tolist() == want.tolist()
        return
    middle_sorted = sorted(range(1, P - 1), key=lambda p: (-scores64[p], p))
    s_cut = scores64[middle_sorted[K - 3]]
    band = SCORE_BAND * abs(s_cut)
    gs, ws = set(got.tolist()), set(want.tolist())
    for p in range(1, P - 1):
        if abs(scores64[p] - s_cut) <= band:
            continue
        assert (p in gs) == (p in ws), (p, scores64[p], s_cut)


def oracle_scores(wl: S.Workload, b: int, g: int, K64: np.ndarray) -> np.ndarray:
    kmin, kmax = O.page_minmax(K64, wl.spec.page_size)
    return O.page_scores(q_group_f64(wl, b, g), kmin, kmax)


def run_select(dw: DeviceWorkload, want_scores=True):
    c = dw.cache
    scores = torch.zeros((c.batch, c.num_kv_heads, c.max_pages), dtype=torch.float32, device=c.device) \
        if want_scores else None
    sel_idx, sel_cnt = spdec.select_pages(c, dw.q, dw.budget, dw.max_budget, scores_out=scores)
    return sel_idx, sel_cnt, scores


def default_scale(wl: S.Workload) -> float:
    return 1.0 / math.sqrt(wl.spec.head_dim)
