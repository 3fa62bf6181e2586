"""CPU oracle for score-mass (top-p) page selection (fp64 NumPy).

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with the
HIP path and imports nothing from it.

What is computed, and where the pages state it
-----------------------------------------------
* The RTPurbo abstract on the first page of the source set (another paper's
  method, not Sparrow's) argues that the useful token budget depends strongly
  on the query, so a dynamic top-p selection suits better than a fixed top-k.
  Nothing more is given; the page-level form below is a reading.
* Page scores, the forced sink and local pages and the tie rule are those of
  the Top-B selection (Sparrow project page, "Control Study 2"; the readings
  in ``page_sparse``).

Reading (listed in the design notes): the page scores act as logits of the
pages' attention mass, w_p = exp(c * (s_p - max_q s_q)) with a score scale c
(1 / (G * sqrt(d)) by default: the bound sums the G query heads of a KV head,
each with the softmax scale 1/sqrt(d)). Pages 0 and P-1 are always kept; the
other pages are taken in the Top-B order (score descending, lower index first
on ties) while the kept mass is below top_p times the total mass of all P
pages and fewer than the cap are kept. With P <= 2 every page is kept.
"""
from __future__ import annotations

import numpy as np

__all__ = ["page_mass", "select_pages_top_p"]


def page_mass(scores, score_scale: float) -> np.ndarray:
    """Unnormalised page masses w_p = exp(c (s_p - max s)) in float64."""
    s = np.asarray(scores, dtype=np.float64)
    return np.exp(float(score_scale) * (s - s.max()))


def select_pages_top_p(scores, top_p: float, score_scale: float, cap: int) -> np.ndarray:
    """Pages kept by the score-mass rule, ascending."""
    s = np.asarray(scores, dtype=np.float64)
    P = s.shape[0]
    if P <= 2:
        return np.arange(P, dtype=np.int64)
    kmax = min(max(int(cap), 2), P)
    w = page_mass(s, score_scale)
    target = float(top_p) * w.sum()
    chosen = [0, P - 1]
    acc = w[0] + w[P - 1]
    for p in sorted(range(1, P - 1), key=lambda i: (-s[i], i)):
        if acc >= target or len(chosen) >= kmax:
            break
        chosen.append(p)
        acc += w[p]
    return np.asarray(sorted(chosen), dtype=np.int64)
