"""GPU parity of the sparsity-schedule controller (spdec_budget_update).

The budgets are integers decided by fp32 arithmetic with one rounding per
operation on both sides, so the new state and every budget must equal the
oracle's bit for bit, for random settings and inputs, for the restart rules,
and when the controller reads the tail statistic straight from
spdec_tail_stats (no host round trip).
"""
import os

import numpy as np
import pytest
import torch

import oracle as O
from oracle import control as C
from sparse_attention_decode_page_amd import spdec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(spdec.LIB_PATH):
        from sparse_attention_decode_page_amd import build
        build.build()
    spdec.lib()
    assert torch.cuda.is_available()


def _both(prm: C.BudgetParams):
    dev = spdec.BudgetParams(target=float(prm.target), gain=float(prm.gain), scale_min=float(prm.scale_min),
                             scale_max=float(prm.scale_max), base_tokens=float(prm.base_tokens),
                             tokens_per_token=float(prm.tokens_per_token), page_size=prm.page_size,
                             max_budget_pages=prm.max_budget_pages)
    return dev


def _run(tail, scale, lens, prm):
    t = torch.tensor(np.asarray(tail, dtype=np.float32), device="cuda")
    s = torch.tensor([scale], dtype=torch.float32, device="cuda")
    L = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    out = spdec.budget_update(t, s, L, _both(prm))
    torch.cuda.synchronize()
    return np.float32(s.item()), out.cpu().numpy()


@pytest.mark.parametrize("seed", range(6))
def test_random_settings_match_oracle(seed):
    r = np.random.default_rng(seed)
    prm = C.BudgetParams(target=r.uniform(0.5, 1.0), gain=r.uniform(0.0, 3.0), scale_min=r.uniform(0.01, 0.5),
                         scale_max=r.uniform(1.0, 16.0), base_tokens=r.uniform(0, 4096),
                         tokens_per_token=r.uniform(0, 0.5), page_size=int(2 ** r.integers(0, 8)),
                         max_budget_pages=int(r.integers(2, 4096)))
    B = int(r.integers(1, 3000))
    lens = r.integers(0, 200000, B)
    lens[:3] = [0, 1, 131072][:min(3, B)]
    tail = (r.uniform(0, 1), r.uniform(0.3, 1.0))
    scale = float(r.uniform(0.01, 16.0))
    s_ref, b_ref = C.budget_update(tail, scale, lens, prm)
    s, b = _run(tail, scale, lens, prm)
    print(f"seed {seed}: B={B} ps={prm.page_size} cap={prm.max_budget_pages} scale {scale:.4f} -> {s:.6f}, "
          f"budgets {b.min()}..{b.max()}", flush=True)
    assert s.view(np.uint32) == np.float32(s_ref).view(np.uint32)
    assert np.array_equal(b, b_ref)


def test_boundary_budgets_match_oracle():
    # lengths whose scheduled tokens land exactly on, and one ulp around, page boundaries
    prm = C.BudgetParams(target=0.86, gain=0.5, scale_min=0.125, scale_max=8.0, base_tokens=1024.0,
                         tokens_per_token=0.125, page_size=16, max_budget_pages=32768)
    lens = np.arange(0, 70000, 7, dtype=np.int64)
    for scale, p5 in ((1.0, 0.86), (1.0, 0.7), (0.37, 0.93), (7.9, 0.1)):
        s_ref, b_ref = C.budget_update((0.9, p5), scale, lens, prm)
        s, b = _run((0.9, p5), scale, lens, prm)
        assert s.view(np.uint32) == np.float32(s_ref).view(np.uint32)
        assert np.array_equal(b, b_ref)


def test_restart_rules_on_device():
    prm = C.BudgetParams(target=0.86, gain=0.5, scale_min=0.25, scale_max=4.0, base_tokens=512.0,
                         tokens_per_token=0.0625, page_size=8, max_budget_pages=1024)
    lens = [0, 100, 5000, 40000]
    for tail, scale in (((0.9, float("nan")), 1.5), ((0.9, 0.86), float("nan")), ((0.9, 0.5), -2.0),
                        ((0.9, 0.0), 0.0), ((0.9, float("inf")), 3.0)):
        s_ref, b_ref = C.budget_update(tail, scale, lens, prm)
        s, b = _run(tail, scale, lens, prm)
        assert s == np.float32(s_ref), (tail, scale)
        assert np.array_equal(b, b_ref), (tail, scale)


def test_reads_the_monitor_without_a_host_round_trip():
    r = np.random.default_rng(7)
    prm = C.BudgetParams(target=0.86, gain=0.8, scale_min=0.1, scale_max=10.0, base_tokens=1024.0,
                         tokens_per_token=0.1, page_size=16, max_budget_pages=2048)
    lens = r.integers(8192, 32768, 64).astype(np.int32)
    L = torch.from_numpy(lens).cuda()
    scale = torch.ones(1, dtype=torch.float32, device="cuda")
    budget = torch.empty(64, dtype=torch.int32, device="cuda")
    alphas = [np.clip(1.0 - r.exponential(0.05 + 0.02 * k, 64), 0, 1).astype(np.float32) for k in range(5)]
    tails = torch.empty((len(alphas), 2), dtype=torch.float32, device="cuda")
    for k, a in enumerate(alphas):   # five steps entirely on the device
        spdec.tail_stats(torch.from_numpy(a).cuda(), out=tails[k])
        spdec.budget_update(tails[k], scale, L, _both(prm), budget_pages=budget)
    torch.cuda.synchronize()
    s_ref = np.float32(1.0)
    for k, a in enumerate(alphas):   # the oracle chain on the oracle's own monitor values
        mean, p5 = O.tail_stats(a)
        t_ref = np.array([mean, p5], dtype=np.float32)   # the fp32 rounding of the exact statistics
        assert np.array_equal(tails[k].cpu().numpy(), t_ref), (k, tails[k].cpu().numpy(), t_ref)
        s_ref, b_ref = C.budget_update(t_ref, s_ref, lens, prm)
    assert scale.item() == float(s_ref)
    assert np.array_equal(budget.cpu().numpy(), b_ref)
