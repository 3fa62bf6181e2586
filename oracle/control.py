"""CPU oracle for the sparsity-schedule controller (fp32 NumPy scalars).

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with the
HIP path and imports nothing from it.

What is computed, and where the pages state it
-----------------------------------------------
* Sparrow project page, "Control Study 1": under a fixed budget the per-token
  sparse-vs-dense mismatch worsens as generation goes on; sparsity scheduling
  gives a more lenient budget as the sequence grows so that the per-token
  mismatch stays roughly constant, and training stays stable while the lower
  5th percentile of the per-token acceptance stays above a threshold (0.86 in
  its takeaway). The page gives no control law ("more details in the paper").
* Sparrow project page, "Control Study 2": budgets are counted in tokens and
  read in pages of ``page_size`` tokens.

Reading (listed in the design notes): the schedule is linear in the cached
length, ``tokens_b = s * (base + slope * L_b)``, and one scalar s (the state)
is corrected once per step from the monitored 5th percentile p5 by a
multiplicative integral step, ``s' = clamp(s * (1 + gain * (target - p5)),
s_min, s_max)``: a tail below the target raises every budget, a tail above it
lowers them, and a tail on target is a fixed point. Pages are
``clamp(ceil(tokens_b / page_size), 2, cap)``.

Precision: the budgets are integers decided by floating point, so this oracle
takes every step in float32 with one rounding per operation, in the order
written above (the order and precision the kernel uses); nothing is fused.
A non-finite p5 leaves s unchanged; a non-finite or non-positive state
restarts from s_max (the most lenient schedule).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["BudgetParams", "budget_update", "budget_pages"]

f32 = np.float32


class BudgetParams:
    """Controller settings: target p5, gain, scale bounds, linear schedule, page size, cap."""

    def __init__(self, target=0.86, gain=0.5, scale_min=0.125, scale_max=8.0, base_tokens=1024.0,
                 tokens_per_token=0.0, page_size=16, max_budget_pages=256):
        self.target = f32(target)
        self.gain = f32(gain)
        self.scale_min = f32(scale_min)
        self.scale_max = f32(scale_max)
        self.base_tokens = f32(base_tokens)
        self.tokens_per_token = f32(tokens_per_token)
        self.page_size = int(page_size)
        self.max_budget_pages = int(max_budget_pages)


def _clamp(x, lo, hi):
    return lo if x < lo else (hi if x > hi else x)


def next_scale(scale, p5, prm: BudgetParams):
    """The state update (float32, one rounding per operation)."""
    s = f32(scale)
    if not (math.isfinite(float(s)) and s > 0):
        s = prm.scale_max
    p = f32(p5)
    if not math.isfinite(float(p)):
        return _clamp(s, prm.scale_min, prm.scale_max)
    e = f32(prm.target - p)
    step = f32(f32(1.0) + f32(prm.gain * e))
    return _clamp(f32(s * step), prm.scale_min, prm.scale_max)


def budget_pages(scale, length, prm: BudgetParams) -> int:
    """Budget in pages of one sequence of cached length ``length`` under scale s."""
    tok = f32(f32(scale) * f32(prm.base_tokens + f32(prm.tokens_per_token * f32(max(int(length), 0)))))
    pages = f32(tok / f32(prm.page_size))
    if not (pages < prm.max_budget_pages):
        return prm.max_budget_pages
    return int(max(math.ceil(float(pages)), 2))


def budget_update(tail, scale, lengths, prm: BudgetParams):
    """One controller step: tail = (mean, p5) of the acceptance; returns (new scale, budgets)."""
    s = next_scale(scale, tail[1], prm)
    return s, np.array([budget_pages(s, L, prm) for L in lengths], dtype=np.int32)
