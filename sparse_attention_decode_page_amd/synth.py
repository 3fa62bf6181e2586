"""Seeded synthetic inputs for page-sparse decode attention.

This module is the single source of inputs shared by the CPU oracle tests, the
GPU parity tests and the benchmark. It holds no step of the method itself (no
page statistics, scores, selection, attention or acceptance arithmetic): it only
draws numbers, rounds them to the storage dtype and lays them out the way the
paged cache expects.

Workloads
---------
The five workloads follow the shapes the pages talk about: Qwen3 decode-layer
head geometry, contexts of 8K-131K tokens, page size 16 (Sparrow project page,
"Control Study 2"), KV budgets of a few thousand tokens (Sparrow project page,
"Insights" section) that grow with generation length ("Control Study 1",
sparsity scheduling), and a 151936-entry vocabulary for the acceptance rows.
The pages measure on real rollouts of Qwen3 models; no weights or datasets are
used here, the seeded draws below stand in for them.

Recipe
------
* Every stream is a numpy PCG64 generator seeded by
  ``SeedSequence(seed, spawn_key=(tag, ...))`` so any (sequence, KV head) unit
  can be regenerated on its own without drawing the rest of the cache.
* Queries, keys and values are standard normal draws; bf16 storage is the
  round-to-nearest-even of the float32 draw, kept as raw ``uint16`` bits.
* "Outlier channels": for each KV head, 4 distinct channels (drawn once per
  workload, shared by all sequences and tokens) of the KEYS are multiplied by
  8 (exact in bf16).
* "Planted block" (long-context page-size sweep): per (sequence, KV head) a
  block of 64 consecutive tokens starting at a uniform offset in
  [64, L-128] gets keys ``8*sign(sum of the group's query heads) + N(0,1)``.
* Ragged lengths: uniform integers in [8192, 32768], one per sequence; the
  budget schedule grows linearly from 1024 to 4096 tokens with length:
  ``tokens = 1024 + 3072*(L-8192)//24576``; budget pages = tokens // page_size.
* Physical placement: every sequence owns ``ceil((L+headroom)/ps)`` logical
  pages that map to a seeded random permutation of the physical pages, so
  gathers are never contiguous. Unused page-table entries are -1.
* Grouped prompts (the shared-prefix workload): 8 consecutive sequences form a
  group that shares a 16384-token prompt drawn once per (group, KV head) from
  its own streams; each sample then has 1024-4096 generated tokens of its own.
  Full prompt pages are the same physical pages in every member's page table.
* Slots of the pool that hold no token (the tail of a partial last page and
  headroom pages) are filled with a poison value (1000.0) so that a kernel
  that forgets to mask them produces visibly wrong results.
* Logit rows: tiny case a, b ~ N(0, 2) independent; acceptance case
  a ~ N(0, 3), b = a + N(0, 0.3), and round(0.05*R) rows chosen by a seeded
  permutation get N(0, 3) noise instead (heavy tail). N(mu, x) means standard
  deviation x.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# Stream tags (spawn keys); fixed so a stream never depends on another's draws.
_T_Q, _T_K, _T_V, _T_OUTLIER, _T_PLANT, _T_LENS, _T_PERM = 1, 2, 3, 4, 5, 6, 7
_T_LOGIT_A, _T_NOISE, _T_HEAVY, _T_APPEND, _T_PROMPT = 8, 9, 10, 11, 12

POISON = 1000.0


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of float32 values to bf16, returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32 (used for input plumbing only)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str                      # "f32" or "bf16"
    lens: tuple                     # ("fixed", L) or ("uniform", lo, hi)
    budget: tuple                   # ("tokens", n) or ("linear", lo_tok, hi_tok, lo_len, hi_len)
    outlier_channels: int = 0
    outlier_scale: float = 8.0
    planted_block: int = 0
    logits: Optional[tuple] = None  # ("independent", rows, vocab, sigma) / ("noisy", rows, vocab, sa, sn, frac_heavy, s_heavy)
    temperature: float = 1.0
    prompt: Optional[tuple] = None  # ("shared", group_size, prompt_tokens): groups of consecutive sequences share a prompt

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _specs() -> dict:
    s = {}
    s["tiny"] = Spec("tiny", 2, 4, 2, 64, 16, "f32", ("fixed", 1024), ("tokens", 256),
                     logits=("independent", 1, 4096, 2.0))
    s["qwen3-1.7b-L16k"] = Spec("qwen3-1.7b-L16k", 32, 16, 8, 128, 16, "bf16", ("fixed", 16384),
                                ("tokens", 2048), outlier_channels=4)
    s["qwen3-8b-ragged"] = Spec("qwen3-8b-ragged", 64, 32, 8, 128, 16, "bf16", ("uniform", 8192, 32768),
                                ("linear", 1024, 4096, 8192, 32768), outlier_channels=4,
                                logits=("noisy", 64, 151936, 3.0, 0.3, 0.05, 3.0))
    for ps in (8, 16, 32, 64):
        s[f"long-131k-ps{ps}"] = Spec(f"long-131k-ps{ps}", 4, 32, 8, 128, ps, "bf16", ("fixed", 131072),
                                      ("tokens", 4096), planted_block=64)
    # GRPO-style groups: 8 prompts x 8 samples, each sample = the group's 16K-token prompt + its own
    # 1K-4K generated tokens (shared prompt pages are the same physical pages)
    s["qwen3-8b-grouped"] = Spec("qwen3-8b-grouped", 64, 32, 8, 128, 16, "bf16", ("uniform", 1024, 4096),
                                 ("tokens", 2048), outlier_channels=4, prompt=("shared", 8, 16384))
    s["qwen3-8b-L32k-acceptance"] = Spec("qwen3-8b-L32k-acceptance", 64, 32, 8, 128, 16, "bf16",
                                         ("fixed", 32768), ("tokens", 4096), outlier_channels=4,
                                         logits=("noisy", 64, 151936, 3.0, 0.3, 0.05, 3.0))
    return s


SPECS = _specs()


def custom_spec(name="custom", **kw) -> Spec:
    """A free-form spec for edge-case tests (same recipe, any shape)."""
    base = dict(batch=1, num_q_heads=2, num_kv_heads=1, head_dim=64, page_size=16, dtype="f32",
                lens=("fixed", 64), budget=("tokens", 64))
    base.update(kw)
    return Spec(name, **base)


@dataclasses.dataclass
class Workload:
    spec: Spec
    seed: int
    lens: np.ndarray            # int32 [B] tokens in cache
    budget_pages: np.ndarray    # int32 [B]
    max_pages: int              # page-table row length
    num_phys: int
    page_table: np.ndarray      # int32 [B][max_pages], -1 = unmapped
    q: np.ndarray               # storage dtype [B][Hq][D]
    outliers: np.ndarray        # int [Hkv][n] key channels scaled (may be empty)
    plant_start: np.ndarray     # int [B][Hkv] planted block start (-1 if none)
    k_pool: Optional[np.ndarray] = None   # storage dtype [Nphys][Hkv][ps][D]
    v_pool: Optional[np.ndarray] = None
    logits_a: Optional[np.ndarray] = None  # float32 [R][V]
    logits_b: Optional[np.ndarray] = None
    heavy_rows: Optional[np.ndarray] = None
    shared_pages: Optional[np.ndarray] = None  # int32 [batch / group_size]: leading pages a group shares

    @property
    def storage_dtype(self):
        return np.uint16 if self.spec.dtype == "bf16" else np.float32

    def pages(self, b: int) -> int:
        ps = self.spec.page_size
        return (int(self.lens[b]) + ps - 1) // ps


def _to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def _poison(dtype: str):
    return f32_to_bf16_bits(np.float32([POISON]))[0] if dtype == "bf16" else np.float32(POISON)


def _lens(spec: Spec, seed: int) -> np.ndarray:
    if spec.lens[0] == "fixed":
        return np.full(spec.batch, spec.lens[1], dtype=np.int32)
    if spec.lens[0] == "uniform":
        lo, hi = spec.lens[1], spec.lens[2]
        return _rng(seed, _T_LENS).integers(lo, hi, size=spec.batch, endpoint=True).astype(np.int32)
    if spec.lens[0] == "list":
        return np.asarray(spec.lens[1], dtype=np.int32)
    raise ValueError(spec.lens)


def budget_tokens(spec: Spec, lens: np.ndarray) -> np.ndarray:
    """Per-sequence KV budget in tokens (the workload's schedule, an input)."""
    if spec.budget[0] == "tokens":
        return np.full(spec.batch, spec.budget[1], dtype=np.int64)
    if spec.budget[0] == "linear":
        lo_t, hi_t, lo_l, hi_l = spec.budget[1:]
        L = lens.astype(np.int64)
        return lo_t + ((hi_t - lo_t) * (L - lo_l)) // (hi_l - lo_l)
    if spec.budget[0] == "pages":
        return np.asarray(spec.budget[1], dtype=np.int64) * spec.page_size
    raise ValueError(spec.budget)


def make_workload(spec, seed: int = 0, headroom: int = 0, build_pool: bool = True,
                  threads: Optional[int] = None) -> Workload:
    """Draw the full workload for ``spec`` (a Spec or a key of SPECS)."""
    if isinstance(spec, str):
        spec = SPECS[spec]
    B, Hq, Hkv, D, ps = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size
    lens = _lens(spec, seed)
    shared = np.zeros(0, dtype=np.int32)
    if spec.prompt is not None:  # lens are the generated parts; every sequence starts with its group's prompt
        _, N, prompt = spec.prompt
        assert B % N == 0
        lens = (lens.astype(np.int64) + prompt).astype(np.int32)
        shared = np.full(B // N, prompt // ps, dtype=np.int32)  # only full pages are shared
    bpages = (budget_tokens(spec, lens) // ps).astype(np.int32)
    caps = (lens.astype(np.int64) + headroom + ps - 1) // ps
    max_pages = int(caps.max())
    own = caps.copy()
    if spec.prompt is not None:
        own -= np.repeat(shared, spec.prompt[1])
    num_phys = int(own.sum() + shared.sum())
    perm = _rng(seed, _T_PERM).permutation(num_phys).astype(np.int32)
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        first = 0
        if spec.prompt is not None:
            N = spec.prompt[1]
            n = b // N
            first = int(shared[n])
            if b % N == 0:  # the group's shared pages, allocated once
                page_table[b, :first] = perm[off:off + first]
                off += first
            else:
                page_table[b, :first] = page_table[n * N, :first]
        page_table[b, first:caps[b]] = perm[off:off + int(caps[b]) - first]
        off += int(caps[b]) - first
    q32 = _rng(seed, _T_Q).standard_normal((B, Hq, D), dtype=np.float32)
    q = _to_storage(q32, spec.dtype)
    if spec.outlier_channels:
        orng = _rng(seed, _T_OUTLIER)
        outliers = np.stack([orng.choice(D, spec.outlier_channels, replace=False) for _ in range(Hkv)])
    else:
        outliers = np.zeros((Hkv, 0), dtype=np.int64)
    plant = np.full((B, Hkv), -1, dtype=np.int64)
    if spec.planted_block:
        prng = _rng(seed, _T_PLANT)
        for b in range(B):
            for g in range(Hkv):
                plant[b, g] = prng.integers(64, int(lens[b]) - 128, endpoint=True)
    wl = Workload(spec, seed, lens, bpages, max_pages, num_phys, page_table, q, outliers, plant)
    if spec.prompt is not None:
        wl.shared_pages = shared
    if build_pool:
        build_pools(wl, threads=threads)
    if spec.logits is not None:
        wl.logits_a, wl.logits_b, wl.heavy_rows = make_logits(spec, seed)
    return wl


def unit_tokens(wl: Workload, b: int, g: int, n: Optional[int] = None):
    """K and V rows (storage dtype, [n][D]) of sequence b, KV head g.

    ``n`` defaults to the sequence's length; any n gives a prefix of the same
    draws, so a longer n also yields the tokens later appended by a decode loop.
    """
    spec = wl.spec
    n = int(wl.lens[b]) if n is None else n
    D = spec.head_dim
    k32 = _rng(wl.seed, _T_K, b, g).standard_normal((n, D), dtype=np.float32)
    v32 = _rng(wl.seed, _T_V, b, g).standard_normal((n, D), dtype=np.float32)
    if spec.prompt is not None:  # the group's prompt tokens come from the group's own streams
        _, N, prompt = spec.prompt
        m = min(prompt, n)
        grp = b // N
        k32[:m] = _rng(wl.seed, _T_PROMPT, _T_K, grp, g).standard_normal((m, D), dtype=np.float32)
        v32[:m] = _rng(wl.seed, _T_PROMPT, _T_V, grp, g).standard_normal((m, D), dtype=np.float32)
    if spec.outlier_channels:
        k32[:, wl.outliers[g]] *= np.float32(spec.outlier_scale)
    if spec.planted_block and wl.plant_start[b, g] >= 0:
        s0 = int(wl.plant_start[b, g])
        s1 = min(s0 + spec.planted_block, n)
        if s1 > s0:
            G = spec.group
            qsum = _q_f32(wl)[b, g * G:(g + 1) * G].sum(axis=0)
            sign = np.where(qsum >= 0, np.float32(1), np.float32(-1))
            prng = _rng(wl.seed, _T_PLANT, b, g)
            k32[s0:s1] = np.float32(8.0) * sign + prng.standard_normal((s1 - s0, D), dtype=np.float32)
    return _to_storage(k32, spec.dtype), _to_storage(v32, spec.dtype)


def append_tokens(wl: Workload, step: int):
    """New K/V rows [B][Hkv][D] for decode step ``step`` (independent of the cache draws)."""
    spec = wl.spec
    r = _rng(wl.seed, _T_APPEND, step)
    k32 = r.standard_normal((spec.batch, spec.num_kv_heads, spec.head_dim), dtype=np.float32)
    v32 = r.standard_normal((spec.batch, spec.num_kv_heads, spec.head_dim), dtype=np.float32)
    return _to_storage(k32, spec.dtype), _to_storage(v32, spec.dtype)


def _q_f32(wl: Workload) -> np.ndarray:
    return bf16_bits_to_f32(wl.q) if wl.spec.dtype == "bf16" else wl.q


def build_pools(wl: Workload, threads: Optional[int] = None):
    """Lay every unit's tokens into the physical K/V pools ([Nphys][Hkv][ps][D])."""
    spec = wl.spec
    B, Hkv, D, ps = spec.batch, spec.num_kv_heads, spec.head_dim, spec.page_size
    sd = wl.storage_dtype
    k_pool = np.empty((wl.num_phys, Hkv, ps, D), dtype=sd)
    v_pool = np.empty((wl.num_phys, Hkv, ps, D), dtype=sd)
    k_pool[...] = _poison(spec.dtype)
    v_pool[...] = _poison(spec.dtype)

    def fill(unit):
        b, g = divmod(unit, Hkv)
        L = int(wl.lens[b])
        P = (L + ps - 1) // ps
        kt, vt = unit_tokens(wl, b, g)
        phys = wl.page_table[b, :P]
        full = L // ps
        if full:
            k_pool[phys[:full], g] = kt[:full * ps].reshape(full, ps, D)
            v_pool[phys[:full], g] = vt[:full * ps].reshape(full, ps, D)
        rem = L - full * ps
        if rem:
            k_pool[phys[full], g, :rem] = kt[full * ps:]
            v_pool[phys[full], g, :rem] = vt[full * ps:]

    nthreads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(fill, range(B * Hkv)))
    wl.k_pool, wl.v_pool = k_pool, v_pool


def make_logits(spec: Spec, seed: int):
    kind = spec.logits[0]
    if kind == "independent":
        _, R, V, sigma = spec.logits
        r = _rng(seed, _T_LOGIT_A)
        a = (sigma * r.standard_normal((R, V), dtype=np.float32)).astype(np.float32)
        b = (sigma * _rng(seed, _T_NOISE).standard_normal((R, V), dtype=np.float32)).astype(np.float32)
        return a, b, np.zeros(0, dtype=np.int64)
    if kind == "noisy":
        _, R, V, sa, sn, frac, sh = spec.logits
        a = (np.float32(sa) * _rng(seed, _T_LOGIT_A).standard_normal((R, V), dtype=np.float32))
        noise = _rng(seed, _T_NOISE).standard_normal((R, V), dtype=np.float32)
        n_heavy = int(round(frac * R))
        heavy = np.sort(_rng(seed, _T_HEAVY).permutation(R)[:n_heavy])
        scale = np.full((R, 1), np.float32(sn), dtype=np.float32)
        scale[heavy] = np.float32(sh)
        b = (a + scale * noise).astype(np.float32)
        return a.astype(np.float32), b, heavy
    raise ValueError(kind)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Decoded float64 view of storage values (plumbing for tests)."""
    return bf16_bits_to_f32(x).astype(np.float64) if dtype == "bf16" else np.asarray(x, np.float64)
