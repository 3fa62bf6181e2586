"""CPU oracle (fp64 NumPy) for dense verification of a sparse draft.

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with the
HIP path and imports nothing from it.

What is computed, and where the pages state it
-----------------------------------------------
* The S3R page ("S3R: Fast and Faithful RL Rollouts via Self-Sparse
  Speculative Decoding"), abstract and Tables 6-7: sparse attention drafts k
  tokens (k = 6 in its measurements), then one full-attention pass verifies
  the k + 1 positions over the complete KV cache, and exact speculative
  sampling decides which drafted tokens stand, so the emitted tokens follow
  the dense policy.
* Exact speculative sampling is the method of the two papers the citation-map
  page lists by title ("Fast Inference from Transformers via Speculative
  Decoding"; "Accelerating Large Language Model Decoding with Speculative
  Sampling"): draft x_i ~ q_i is kept when a uniform u_i satisfies
  u_i < p_i(x_i) / q_i(x_i); at the first rejected position the token is
  drawn from the normalised residual max(0, p_i - q_i); when every draft is
  kept, one more token is drawn from the verifier's next distribution.

Readings where the pages are silent (listed in the design notes):
* Verification attention: query t of the T = k + 1 verified positions sits at
  cache position L - T + t (the drafted tokens are already in the cache, so L
  counts them) and attends to positions 0 .. L - T + t (causal within the
  draft).
* Random draws are inputs: the uniforms of the accept tests and the uniform of
  the final draw are passed in, never generated here.
* A draw from a discrete distribution r (not necessarily normalised) with a
  uniform u takes the first token v whose running sum of r exceeds u * sum(r)
  (inverse CDF in token order).
* Logits are divided by the temperature before the softmax (as for the
  acceptance measure).
* A rejection whose residual max(0, p_j - q_j) has no mass (p_j <= q_j at
  every token, i.e. p_j = q_j up to rounding, where the residual's
  normalisation is undefined) draws from p_j itself, the distribution the
  emitted token must follow.
"""
from __future__ import annotations

import numpy as np

from .page_sparse import attention, softmax_t

__all__ = ["verify_decode_unit", "inverse_cdf_draw", "speculative_accept"]


def verify_decode_unit(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Causal multi-query attention of one (sequence, KV head) over its complete KV.

    q_rows [T][G][D]: the G query heads of the KV head at each of the T
    verified positions; K, V [L][D]: every cached token (the last T are the
    drafted ones). Query t attends to tokens 0 .. L - T + t. Returns
    (out [T][G][D], lse [T][G]).
    """
    T, G, D = q_rows.shape
    L = K.shape[0]
    out = np.zeros((T, G, D))
    lse = np.zeros((T, G))
    for t in range(T):
        n = L - T + t + 1  # tokens visible to position t
        for h in range(G):
            out[t, h], lse[t, h] = attention(q_rows[t, h], K[:n], V[:n], scale)
    return out, lse


def inverse_cdf_draw(weights: np.ndarray, u: float) -> int:
    """The first token v with sum_{w <= v} weights_w > u * sum(weights) (u in [0, 1))."""
    w = np.asarray(weights, dtype=np.float64)
    total = w.sum()
    target = u * total
    run = 0.0
    last = -1
    for v in range(w.shape[0]):
        if w[v] > 0.0:
            last = v
        run += w[v]
        if run > target and w[v] > 0.0:
            return v
    return last  # rounding left the running sum at or below the target: last token with weight


def speculative_accept(p_logits: np.ndarray, q_logits: np.ndarray, draft, u_accept, u_sample: float,
                       temperature: float = 1.0):
    """Exact speculative sampling for one sequence.

    p_logits [k+1][V]: the verifier's (dense) logits at the k + 1 verified
    positions; q_logits [k][V]: the drafter's (sparse) logits at the k drafted
    positions; draft [k]: the drafted tokens; u_accept [k], u_sample: uniforms
    in [0, 1). Draft i is kept when u_i * q_i(x_i) < p_i(x_i). At the first
    rejected position j the emitted token is drawn from max(0, p_j - q_j);
    when all k are kept it is drawn from p_k. Returns (kept drafts, token).
    """
    k = len(draft)
    for i in range(k):
        p = softmax_t(p_logits[i], temperature)
        q = softmax_t(q_logits[i], temperature)
        x = int(draft[i])
        if not (u_accept[i] * q[x] < p[x]):
            residual = np.maximum(p - q, 0.0)
            return i, inverse_cdf_draw(residual if residual.sum() > 0.0 else p, u_sample)
    return k, inverse_cdf_draw(softmax_t(p_logits[k], temperature), u_sample)
