"""CPU model of the sliced selection's argument (the few-unit forms of the sparse step and of the selection): the
middle pages are cut into contiguous slices, each slice keeps its own top `need` pages in the Top-B order (score
descending, lower page first), and the unit's top `need` is then taken from the union of the slices' candidates in
the same order. The claim checked here, on seeded scores with many ties, every slice count and every need: the
union holds the whole-unit top `need`, and the top `need` of the union is exactly it (so the tie rule survives the
cut). A page left out by its slice has `need` pages of that slice ahead of it in the order, hence cannot be among
the unit's top `need`."""
import numpy as np
import pytest


def top_need(pages, scores, need):
    """The `need` first pages in the Top-B order (score descending, lower page first)."""
    order = sorted(pages, key=lambda p: (-scores[p], p))
    return sorted(order[:need])


@pytest.mark.parametrize("seed", range(40))
def test_union_of_slice_candidates_holds_the_top_need(seed):
    r = np.random.default_rng(seed)
    M = int(r.integers(1, 400))                      # middle pages
    levels = int(r.integers(1, 12))                  # few distinct scores: many ties
    scores = r.integers(0, levels, M).astype(np.float64)
    if seed % 3 == 0:                                # a planted block of high scores in one slice
        a = int(r.integers(0, M))
        scores[a:a + int(r.integers(1, 50))] = levels + 1
    pages = list(range(M))
    want_all = {need: top_need(pages, scores, need) for need in range(0, M + 1)}
    for S in range(1, 17):
        per = -(-M // S)
        slices = [pages[s * per:(s + 1) * per] for s in range(S)]
        for need in {0, 1, 2, M // 3, M // 2, M - 1, M} | set(int(x) for x in r.integers(0, M + 1, 5)):
            if need < 0 or need > M:
                continue
            cand = [p for sl in slices for p in top_need(sl, scores, min(need, len(sl)))]
            assert set(want_all[need]) <= set(cand), (seed, S, need)
            assert top_need(cand, scores, need) == want_all[need], (seed, S, need)
