"""Pins for the sparsity-schedule controller oracle (CPU only).

The control law is a reading (the pages give none), so these checks tie it to
what that reading must satisfy, not to itself: hand-worked updates on exactly
representable values, the fixed point on target, the direction of every
correction, the clamps, the restart rules, and convergence to the closed-form
operating point of a continuous synthetic plant.
"""
import math

import numpy as np
import pytest

from oracle import control as C


def test_hand_worked_update():
    # target 0.875, p5 0.625: error 0.25, step 1 + 0.5 * 0.25 = 1.125, scale 2 -> 2.25 (all exact in fp32)
    prm = C.BudgetParams(target=0.875, gain=0.5, scale_min=0.25, scale_max=8.0, base_tokens=1024.0,
                         tokens_per_token=0.125, page_size=16, max_budget_pages=512)
    s, pages = C.budget_update((0.9, 0.625), 2.0, [8192, 100, 0], prm)
    assert s == np.float32(2.25)
    # 2.25 * (1024 + 0.125 * 8192) = 4608 tokens = 288 pages; 2.25 * (1024 + 12.5) = 2332.125 -> 145.76 -> 146;
    # 2.25 * 1024 = 2304 -> 144
    assert pages.tolist() == [288, 146, 144]


def test_cap_and_floor():
    prm = C.BudgetParams(target=0.86, gain=0.5, scale_min=0.001, scale_max=8.0, base_tokens=1024.0,
                         tokens_per_token=0.125, page_size=16, max_budget_pages=256)
    assert C.budget_pages(2.25, 8192, prm) == 256             # 288 pages, capped
    assert C.budget_pages(0.001, 0, prm) == 2                 # 1.024 tokens -> floor of two pages
    assert C.budget_pages(1.0, 0, prm) == 64                  # exactly 64 pages: no rounding up


def test_on_target_is_a_fixed_point():
    prm = C.BudgetParams(target=0.86, gain=0.7)
    for s in (0.125, 0.3, 1.0, 2.5, 8.0):
        assert C.next_scale(s, np.float32(0.86), prm) == np.float32(s)


@pytest.mark.parametrize("p5", [0.0, 0.5, 0.8, 0.85])
def test_a_low_tail_raises_the_budget(p5):
    prm = C.BudgetParams(target=0.86, gain=0.5)
    s = C.next_scale(1.0, p5, prm)
    assert s > 1.0
    assert C.budget_pages(s, 5000, prm) >= C.budget_pages(1.0, 5000, prm)


@pytest.mark.parametrize("p5", [0.87, 0.95, 1.0])
def test_a_high_tail_lowers_the_budget(p5):
    prm = C.BudgetParams(target=0.86, gain=0.5)
    assert C.next_scale(1.0, p5, prm) < 1.0


def test_scale_clamps():
    prm = C.BudgetParams(target=0.86, gain=4.0, scale_min=0.5, scale_max=2.0)
    assert C.next_scale(1.9, 0.0, prm) == np.float32(2.0)     # 1.9 * (1 + 3.44) clamped
    assert C.next_scale(0.6, 1.0, prm) == np.float32(0.5)     # 0.6 * (1 - 0.56) clamped


def test_restart_rules():
    prm = C.BudgetParams(target=0.86, gain=0.5, scale_min=0.25, scale_max=4.0)
    assert C.next_scale(1.5, float("nan"), prm) == np.float32(1.5)    # no monitor value: no correction
    assert C.next_scale(float("nan"), 0.86, prm) == np.float32(4.0)   # lost state: most lenient schedule
    assert C.next_scale(-1.0, 0.86, prm) == np.float32(4.0)
    assert C.next_scale(0.0, 0.86, prm) == np.float32(4.0)


def test_budgets_monotone_in_scale_and_length():
    prm = C.BudgetParams(target=0.86, gain=0.5, base_tokens=512.0, tokens_per_token=0.0625, page_size=8,
                         max_budget_pages=1024)
    r = np.random.default_rng(0)
    for _ in range(200):
        s1, s2 = sorted(r.uniform(0.1, 4.0, 2))
        L1, L2 = sorted(r.integers(0, 40000, 2))
        assert C.budget_pages(s1, L1, prm) <= C.budget_pages(s2, L1, prm)
        assert C.budget_pages(s1, L1, prm) <= C.budget_pages(s1, L2, prm)


@pytest.mark.parametrize("c,target,gain", [(0.2, 0.86, 0.5), (0.05, 0.9, 1.0), (0.5, 0.8, 0.3)])
def test_converges_to_the_plants_operating_point(c, target, gain):
    # plant: p5(s) = 1 - c / s, increasing in the budget scale; on target at s* = c / (1 - target)
    prm = C.BudgetParams(target=target, gain=gain, scale_min=0.01, scale_max=100.0)
    s = np.float32(1.0)
    for _ in range(400):
        s = C.next_scale(s, np.float32(1.0 - c / float(s)), prm)
    s_star = c / (1.0 - target)
    assert math.isclose(float(s), s_star, rel_tol=1e-4)
