"""CPU oracle for query-aware page-sparse decode attention (fp64 NumPy).

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with the
HIP path and imports nothing from it; it reads plain host arrays (the pool,
page table and lengths that the seeded input generator produces) and computes
every step from its definition, slowly and in float64.

What is computed, and where the pages state it
-----------------------------------------------
Sources are the Sparrow project page ("Sparrow: Sparse Rollout for Stable and
Efficient Long-context RL of Large Language Models"), the S3R page ("S3R: Fast
and Faithful RL Rollouts via Self-Sparse Speculative Decoding"), the Sparrow
citation-map page and the wispaper blog summary of Sparrow.

* Paged KV cache and block-sparse (page) attention with a KV budget B and a
  page size: Sparrow project page, "Insights" (block-sparse attention is the
  studied method) and "Control Study 2" (cost model: KV budget B, page size,
  Top-k page selection, page size 16).
* Page scoring: the pages only cite Quest (query-aware sparsity) by title on
  the citation-map page; the score used here is the Quest-style upper bound
  sum_h sum_d max(q_hd * kmax_d, q_hd * kmin_d) over the query heads h that
  share a KV head (a reading; see ``page_scores``).
* Forced first (sink) and last (local) pages: the pages only cite
  StreamingLLM's attention sinks by title (citation-map page); kept as a
  reading.
* Dense attention over the complete KV: S3R abstract (dense verification needs
  the complete historical KV cache).
* Per-token sparse-vs-dense mismatch as an acceptance rate, and its lower
  5th percentile: Sparrow project page, "Insights" and "Control Study 1";
  blog summary ("acceptance rate", threshold 0.86).

Readings where the pages are silent (each listed in the design notes):
softmax scale 1/sqrt(d); the budget counts the forced pages and is clamped to
at least 2 pages; ties in score go to the lower page index; tokens at or past
the sequence length are masked; acceptance divides logits by the temperature
before the softmax; the percentile is linear interpolation.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "decode_bf16", "to_f64", "page_count", "gather_tokens", "page_minmax", "append_minmax",
    "page_scores", "select_pages", "attention", "tokens_of_pages", "decode_unit",
    "sparse_decode_unit", "dense_decode_unit", "softmax_t", "acceptance", "total_variation",
    "tail_stats", "monitor_window", "lse_merge",
]


# ---------------------------------------------------------------- storage ---

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values (bf16 is the top half of a float32)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    return decode_bf16(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)


# ------------------------------------------------------------------ pages ---

def page_count(L: int, ps: int) -> int:
    """Pages of ps tokens holding L tokens; page p covers [p*ps, min((p+1)*ps, L))."""
    return (L + ps - 1) // ps


def gather_tokens(pool: np.ndarray, page_table_row: np.ndarray, L: int, g: int, ps: int) -> np.ndarray:
    """Logical token rows [L][D] of one (sequence, KV head) from a pool [Nphys][Hkv][ps][D]."""
    rows = []
    for t in range(0, L, ps):
        phys = int(page_table_row[t // ps])
        n = min(ps, L - t)
        rows.append(pool[phys, g, :n])
    return np.concatenate(rows, axis=0) if rows else pool[:0, g, 0]


def page_minmax(K: np.ndarray, ps: int):
    """Per-page, per-channel key minimum and maximum over the page's valid tokens.

    K: float64 [L][D] logical keys. Returns (kmin, kmax), each [P][D]. Only the
    tokens the page actually holds take part (a partial last page covers fewer
    than ps tokens). This is the page summary the Quest-style bound needs.
    """
    L = K.shape[0]
    P = page_count(L, ps)
    kmin = np.empty((P, K.shape[1]))
    kmax = np.empty((P, K.shape[1]))
    for p in range(P):
        blk = K[p * ps:min((p + 1) * ps, L)]
        kmin[p] = blk.min(axis=0)
        kmax[p] = blk.max(axis=0)
    return kmin, kmax


def append_minmax(kmin_p, kmax_p, k, slot: int):
    """Incremental form of ``page_minmax`` for one appended key in slot ``slot`` of its page.

    The first token of a page starts the page's summary; later tokens widen it.
    """
    k = np.asarray(k, dtype=np.float64)
    if slot == 0:
        return k.copy(), k.copy()
    return np.minimum(kmin_p, k), np.maximum(kmax_p, k)


# ---------------------------------------------------------------- scoring ---

def page_scores(q_group: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """Quest-style upper bound of the group's attention logits on every page.

    s_p = sum over query heads h of the group, sum over channels d, of
    max(q_hd * kmax_pd, q_hd * kmin_pd). For every token t of page p and head h,
    q_h . k_t <= sum_d max(q_hd*kmax_pd, q_hd*kmin_pd), so s_p bounds the summed
    logits of the group from above. q_group: [G][D]; kmin, kmax: [P][D].
    """
    q = np.asarray(q_group, dtype=np.float64)
    hi = q[:, None, :] * kmax[None, :, :]     # [G][P][D]
    lo = q[:, None, :] * kmin[None, :, :]
    return np.maximum(hi, lo).sum(axis=2).sum(axis=0)


def select_pages(scores: np.ndarray, budget_pages: int) -> np.ndarray:
    """Top-B page selection with the sink and local pages always kept.

    K = min(max(budget, 2), P). If K >= P every page is kept. Otherwise page 0
    (sink) and page P-1 (local, holds the current token) are kept, plus the K-2
    pages of 1..P-2 with the highest scores; equal scores go to the lower page
    index. Returned ascending.
    """
    s = np.asarray(scores, dtype=np.float64)
    P = s.shape[0]
    K = min(max(int(budget_pages), 2), P)
    if K >= P:
        return np.arange(P, dtype=np.int64)
    middle = list(range(1, P - 1))
    middle.sort(key=lambda p: (-s[p], p))
    chosen = sorted([0, P - 1] + middle[:K - 2])
    return np.asarray(chosen, dtype=np.int64)


# -------------------------------------------------------------- attention ---

def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of one query row over token rows K, V.

    z_t = scale * q . k_t ; o = sum_t e^{z_t - m} v_t / sum_t e^{z_t - m} with
    m = max_t z_t ; lse = m + ln sum_t e^{z_t - m}. Returns (o [D], lse).
    With no token at all the pages say nothing; the output is taken as zeros
    and lse as ln 0 = -inf.
    """
    if K.shape[0] == 0:  # no token in the cache: an empty sum, zeros and ln 0
        return np.zeros(V.shape[1]), -math.inf
    z = scale * (K @ np.asarray(q, dtype=np.float64))
    m = z.max()
    w = np.exp(z - m)
    l = w.sum()
    return (w @ V) / l, m + math.log(l)


def tokens_of_pages(pages, L: int, ps: int) -> np.ndarray:
    """Token indices held by the listed pages (tokens >= L are not in the cache)."""
    idx = [np.arange(p * ps, min((p + 1) * ps, L)) for p in pages]
    return np.concatenate(idx) if idx else np.zeros(0, dtype=np.int64)


def decode_unit(q_group: np.ndarray, K: np.ndarray, V: np.ndarray, pages, ps: int, scale: float):
    """Attention of every query head of a group over the tokens of ``pages``.

    Returns (o [G][D], lse [G]). The page set is shared by the group's heads.
    """
    L = K.shape[0]
    t = tokens_of_pages(pages, L, ps)
    Kt, Vt = K[t], V[t]
    outs, lses = [], []
    for h in range(q_group.shape[0]):
        o, lse = attention(q_group[h], Kt, Vt, scale)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.asarray(lses)


def sparse_decode_unit(q_group, K, V, ps: int, budget_pages: int, scale: float):
    """Score pages, select the budget, attend over the selection (one (sequence, KV head))."""
    kmin, kmax = page_minmax(K, ps)
    pages = select_pages(page_scores(q_group, kmin, kmax), budget_pages)
    o, lse = decode_unit(q_group, K, V, pages, ps, scale)
    return o, lse, pages


def dense_decode_unit(q_group, K, V, ps: int, scale: float):
    """Attention over the complete KV of one (sequence, KV head)."""
    return decode_unit(q_group, K, V, range(page_count(K.shape[0], ps)), ps, scale)


def lse_merge(parts):
    """Combine attention results over disjoint token sets from their (o, lse) pairs.

    o = sum_j e^{lse_j - M} o_j / sum_j e^{lse_j - M}, lse = M + ln sum_j e^{lse_j - M}.
    """
    lses = np.asarray([p[1] for p in parts], dtype=np.float64)
    M = lses.max()
    w = np.exp(lses - M)
    o = sum(wj * np.asarray(p[0], dtype=np.float64) for wj, p in zip(w, parts)) / w.sum()
    return o, M + math.log(w.sum())


# ------------------------------------------------------------- acceptance ---

def softmax_t(logits: np.ndarray, temperature: float) -> np.ndarray:
    """softmax(logits / T), max-subtracted."""
    x = np.asarray(logits, dtype=np.float64) / float(temperature)
    e = np.exp(x - x.max())
    return e / e.sum()


def acceptance(a: np.ndarray, b: np.ndarray, temperature: float = 1.0) -> float:
    """Per-token sparse-vs-dense acceptance: sum_v min(softmax(a/T)_v, softmax(b/T)_v).

    Clamped to [0, 1] (the unclamped value is already there up to rounding).
    """
    p = softmax_t(a, temperature)
    q = softmax_t(b, temperature)
    return float(min(1.0, max(0.0, np.minimum(p, q).sum())))


def total_variation(a: np.ndarray, b: np.ndarray, temperature: float = 1.0) -> float:
    """Total-variation distance 1/2 sum_v |p_v - q_v| of the two tempered softmaxes."""
    return 0.5 * float(np.abs(softmax_t(a, temperature) - softmax_t(b, temperature)).sum())


def monitor_window(batches, capacity: int) -> np.ndarray:
    """The values a rollout's tail monitor holds after appending `batches` (arrays of per-token acceptance, in
    order) to a window of `capacity` values: the most recent min(total, capacity) of them (Sparrow project page,
    "Control Study 1": the statistic is taken over the rollout's tokens; the window bounds its memory)."""
    vals = np.concatenate([np.asarray(b, dtype=np.float64).ravel() for b in batches]) if batches else np.zeros(0)
    return vals[max(0, vals.shape[0] - capacity):]


def tail_stats(alphas) -> tuple:
    """Mean and lower 5th percentile (linear interpolation) of per-token acceptance."""
    x = np.sort(np.asarray(alphas, dtype=np.float64))
    n = x.shape[0]
    pos = 0.05 * (n - 1)
    lo = int(math.floor(pos))
    hi = min(lo + 1, n - 1)
    p5 = x[lo] + (pos - lo) * (x[hi] - x[lo])
    return float(x.mean()), float(p5)
