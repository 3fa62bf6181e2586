"""GPU parity of the streaming tail monitor (device ring of per-token acceptance; mean and exact lower 5th
percentile on the device) against the oracle's window and tail statistics, and the controller fed from it.

Sparrow project page, "Control Study 1": the stability signal is the lower 5th percentile of the per-token
mismatch over the rollout's tokens. The percentile must equal the fp32 rounding of the oracle's exact value;
the mean (fp64 sums in another order) is within one fp32 rounding.
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


def _acceptance_like(r, n, ties=False):
    a = np.clip(1.0 - np.abs(r.standard_normal(n)) * 0.03 - (r.random(n) < 0.05) * r.random(n) * 0.5, 0, 1)
    a = a.astype(np.float32)
    if ties and n > 20:
        a[r.choice(n, n // 4, replace=False)] = a[0]
        a[r.choice(n, n // 8, replace=False)] = np.float32(0.9)
    return a


def _check(out, window):
    got = out.cpu().numpy()
    mean, p5 = O.tail_stats(window)
    assert got[1] == np.float32(p5), (got[1], p5, window.shape[0])
    assert abs(float(got[0]) - mean) <= 1.2e-7 * max(1.0, abs(mean)), (got[0], mean)


@pytest.mark.parametrize("capacity,sizes,ties", [
    (1, [1, 3, 1], False),
    (7, [2, 5, 1, 9, 3], True),
    (4096, [64] * 10 + [1000, 4000, 5000], True),
    (100003, [64] * 5 + [30000, 70000, 64, 2], False),
])
def test_monitor_matches_oracle_after_every_append(capacity, sizes, ties):
    print(f"case monitor capacity={capacity} sizes={sizes[:6]}...", flush=True)
    r = np.random.default_rng(capacity)
    mon = spdec.TailMonitor(capacity)
    batches = []
    for n in sizes:
        a = _acceptance_like(r, n, ties)
        batches.append(a)
        mon.append(torch.from_numpy(a).cuda())
        out = mon.stats()
        torch.cuda.synchronize()
        _check(out, O.monitor_window(batches, capacity))
    assert mon.count() == sum(sizes)


def test_monitor_two_million_values():
    """A rollout of 64 sequences x ~32K tokens: 2,097,152 values in steps of 64 and of 65536, window of 2^21 + 5
    (not yet full) and of 2^20 (wrapped)."""
    r = np.random.default_rng(5)
    for capacity in ((1 << 21) + 5, 1 << 20):
        print(f"case monitor 2M values, capacity {capacity}", flush=True)
        mon = spdec.TailMonitor(capacity)
        batches = [_acceptance_like(r, 64, ties=True) for _ in range(1024)]
        batches += [_acceptance_like(r, 65536, ties=True) for _ in range(31)]
        for b in batches[:1024]:
            mon.append(torch.from_numpy(b).cuda())
        mon.append(torch.from_numpy(np.concatenate(batches[1024:])).cuda())
        out = mon.stats()
        torch.cuda.synchronize()
        assert mon.count() == 64 * 1024 + 65536 * 31
        _check(out, O.monitor_window(batches, capacity))


def test_monitor_empty_reset_and_determinism():
    mon = spdec.TailMonitor(1000)
    out = mon.stats()
    torch.cuda.synchronize()
    assert np.all(np.isnan(out.cpu().numpy()))
    r = np.random.default_rng(9)
    a = _acceptance_like(r, 777, ties=True)
    mon.append(torch.from_numpy(a).cuda())
    o1 = mon.stats().clone()
    o2 = mon.stats().clone()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    _check(o1, a.astype(np.float64))
    mon.reset()
    b = _acceptance_like(r, 33)
    mon.append(torch.from_numpy(b).cuda())
    out = mon.stats()
    torch.cuda.synchronize()
    assert mon.count() == 33
    _check(out, b.astype(np.float64))
    # all values equal: both order statistics are that value
    mon.reset()
    mon.append(torch.full((5000,), 0.875, dtype=torch.float32, device="cuda"))
    out = mon.stats()
    torch.cuda.synchronize()
    assert out.cpu().numpy().tolist() == [0.875, 0.875]


def test_controller_reads_the_monitor_on_the_device():
    """Ten decode steps of 64 tokens on the device: append, stats, budget update; the oracle chain (window,
    tail statistics rounded to fp32, controller) gives the same scale and budgets bit for bit."""
    r = np.random.default_rng(11)
    prm = C.BudgetParams(target=0.86, gain=0.8, scale_min=0.1, scale_max=10.0, base_tokens=1024.0,
                         tokens_per_token=0.1, page_size=16, max_budget_pages=2048)
    lens = r.integers(8192, 32768, 64).astype(np.int32)
    L = torch.from_numpy(lens).cuda()
    scale = torch.ones(1, dtype=torch.float32, device="cuda")
    budget = torch.empty(64, dtype=torch.int32, device="cuda")
    mon = spdec.TailMonitor(300)
    tails = torch.empty((10, 2), dtype=torch.float32, device="cuda")
    batches = [np.clip(1.0 - r.exponential(0.05 + 0.01 * k, 64), 0, 1).astype(np.float32) for k in range(10)]
    bp = spdec.BudgetParams(**{f: getattr(prm, f) for f in ("target", "gain", "scale_min", "scale_max",
                                                              "base_tokens", "tokens_per_token", "page_size",
                                                              "max_budget_pages")})
    for k, a in enumerate(batches):
        mon.append(torch.from_numpy(a).cuda())
        mon.stats(out=tails[k])
        spdec.budget_update(tails[k], scale, L, bp, budget_pages=budget)
    torch.cuda.synchronize()
    s_ref = np.float32(1.0)
    for k in range(10):
        mean, p5 = O.tail_stats(O.monitor_window(batches[:k + 1], 300))
        t_ref = np.array([mean, p5], dtype=np.float32)
        assert tails[k].cpu().numpy()[1] == t_ref[1]
        s_ref, b_ref = C.budget_update(t_ref, s_ref, lens, prm)
    assert scale.item() == float(s_ref)
    assert np.array_equal(budget.cpu().numpy(), b_ref)
