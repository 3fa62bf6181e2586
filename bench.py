#!/usr/bin/env python3
"""Benchmark: query-aware page-sparse decode attention on one GPU.

The timed step is the sparse path of one decode layer, spdec_sparse_path: page
scores (Quest-style bounds over the page summaries), Top-B with sink and local
pages, attention over the kept pages with an LSE merge (one kernel on this
workload; select_pages then sparse_decode where that form does not apply), on a batch
shaped like a Qwen3-8B decode layer with ragged 8K-32K contexts (64 sequences,
32 query / 8 KV heads, head dim 128, page size 16, budgets 1024-4096 tokens
linear in length). Inputs are seeded synthetic data, resident in HBM before
timing starts.

Prints ONE JSON line. `value` is decode tokens/s of the sparse path: batch /
the path's time, each of K runs after a 1 GiB scrub read (so neither L2 nor
the last-level cache holds the previous run's pages) with the K scrubs' own
time subtracted, the median of three interleaved regions. `sparse` gives its
effective KV GB/s (selected K/V plus every page summary, valid tokens only)
and fraction of 8 TB/s, and the same step as the two calls select_pages and
sparse_decode, each also apart; `roofline` is for the dominant kernel, the
step's one kernel. `full_step` times the whole hot path
(append_kv, sparse_path, dense_decode, acceptance over 64 x
151936 logit rows) back to back, with a per-row breakdown and HIP-graph
replay. `dense` and `acceptance` time those calls alone; `qwen3_1_7b`,
`long_context` (4 sequences of 131072 tokens at page sizes 8/16/32/64) and
`acceptance_pass` (64 sequences of 32768 tokens, with the acceptance of 64
logit-row pairs, its mean and lower 5th percentile) repeat the measurement on
the other decode-layer shapes; `verify`, `shared_prefix`, `top_p` and
`monitor` (streaming tail statistics over a 2M-token window) and `budget_control` (the
controller in a closed loop fed by the monitor) time the next rows; `cpu_baseline` times the CPU oracle's
sparse path on the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse decode attn tokens/s + effective KV GB/s (% HBM peak), 1 MI355X"
HOST_CPU_SHARE = 16  # host cores per GPU on the measuring machine: worker pools stay within them
HBM_PEAK_GBPS = 8000.0
WORKLOAD = "qwen3-8b-ragged"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="bound on the CPU-oracle sample")
    ap.add_argument("--no-verify", action="store_true", help="skip the verification / speculative-sampling rows")
    ap.add_argument("--no-shared", action="store_true", help="skip the shared-prefix (grouped prompts) rows")
    ap.add_argument("--no-control", action="store_true", help="skip the closed-loop budget controller rows")
    ap.add_argument("--no-top-p", action="store_true", help="skip the score-mass (top-p) selection rows")
    ap.add_argument("--no-second-shape", action="store_true",
                    help="skip the Qwen3-1.7B-shaped decode layer (sparse path and dense decode)")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the 131072-token page-size sweep (4 sequences, page sizes 8/16/32/64)")
    ap.add_argument("--no-acceptance-pass", action="store_true",
                    help="skip the 32768-token batch with its acceptance over 64 x 151936 logit pairs")
    ap.add_argument("--layer", default=None,
                    help="profiling mode: only the layer rows of these comma-separated workloads (sparse path, its "
                         "two calls, dense decode, gather ceiling), one JSON line; no headline value")
    ap.add_argument("--features", default=None,
                    help="profiling mode: only these comma-separated next rows (verify, shared, top-p) on their "
                         "workloads, one JSON line; no headline value")
    ap.add_argument("--no-gather-ceiling", action="store_true",
                    help="skip the gather-read ceiling probe (the sparse path's page and summary gathers, no math)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3 --pmc)")
    return ap.parse_args()


def algorithmic_bytes(spec, lens, budget_pages, cap, rows, vocab):
    """Bytes each row must move per step (valid tokens / pages only)."""
    ps, D, Hkv = spec.page_size, spec.head_dim, spec.num_kv_heads
    elt = 2 if spec.dtype == "bf16" else 4
    L = lens.astype(np.int64)
    P = (L + ps - 1) // ps
    K = np.minimum(np.minimum(np.maximum(budget_pages.astype(np.int64), 2), cap), P)
    last = L - (P - 1) * ps
    sel_tokens = np.where(K >= P, L, (K - 1) * ps + last)
    kv_tok = 2 * D * elt                      # K + V row of one token, one KV head
    meta_page = 2 * D * elt                   # kmin + kmax of one page, one KV head
    scored = (K < P) & (K > 2)                # the step scores only units whose selection is not fixed
    return {
        "append_kv": int(spec.batch * Hkv * (kv_tok + 2 * meta_page)),
        "select_pages": int(Hkv * (P * meta_page).sum()),
        "sparse_decode": int(Hkv * (sel_tokens * kv_tok).sum()),
        "sparse_path": int(Hkv * (np.where(scored, P * meta_page, 0) + sel_tokens * kv_tok).sum()),
        "dense_decode": int(Hkv * (L * kv_tok).sum()),
        "acceptance": int(2 * rows * vocab * 4),
    }


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_counters_{workload}.md")


# Every device source of the library: a change to any of them voids the committed counter traffic.
KERNEL_SOURCES = tuple(sorted(f for f in os.listdir(os.path.join(ROOT, "sparse_attention_decode_page_amd", "csrc"))
                              if f.endswith((".hip", ".h"))))


def describe_lens(spec) -> str:
    kind = spec.lens[0]
    if kind == "uniform":
        return f"uniform {spec.lens[1]}..{spec.lens[2]} per sequence"
    if kind == "fixed":
        return f"{spec.lens[1]} per sequence"
    return str(spec.lens)


def describe_budget(spec) -> str:
    kind = spec.budget[0]
    if kind == "linear":
        return f"{spec.budget[1]}->{spec.budget[2]} tokens, linear in length"
    if kind == "tokens":
        return f"{spec.budget[1]} tokens"
    return str(spec.budget)


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_attention_decode_page_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload: str):
    """Per-dispatch HBM bytes on `workload` from its committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary.

    Returns {kernel: bytes} or None when the summary is missing or the kernel
    sources changed since the counters were taken.
    """
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    table, src = {}, None
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 2 and parts[0] == "source_hash":
                src = parts[1]
            elif len(parts) == 3 and parts[0] == "traffic_bytes":
                table[parts[1]] = int(parts[2])
    if src != kernel_source_hash():
        return None
    return table


def cpu_baseline(wl, steps_tokens, seconds: float):
    """Time the CPU oracle on the same step for as many sequences as fit in `seconds`."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return _cpu_baseline(O, wl, steps_tokens, seconds)


def _oracle_sequence(O, wl, kn, vn, b):
    """The oracle's step for sequence b (all KV heads); returns the timed seconds of the whole step and of its
    sparse path (page scores, selection, sparse attention), the cache as it stands before the step gathered,
    decoded and summarised untimed."""
    spec = wl.spec
    ps, G, D = spec.page_size, spec.group, spec.head_dim
    scale = 1.0 / math.sqrt(D)
    state = []
    for g in range(spec.num_kv_heads):
        L = int(wl.lens[b])
        K = O.to_f64(O.gather_tokens(wl.k_pool, wl.page_table[b], L, g, ps), spec.dtype)
        V = O.to_f64(O.gather_tokens(wl.v_pool, wl.page_table[b], L, g, ps), spec.dtype)
        kmin, kmax = O.page_minmax(K, ps)
        state.append((K, V, kmin, kmax))
    t_sparse = 0.0
    t0 = time.perf_counter()
    for g, (K, V, kmin, kmax) in enumerate(state):
        k_new = O.to_f64(kn[b, g], spec.dtype)
        v_new = O.to_f64(vn[b, g], spec.dtype)
        L = K.shape[0]
        K = np.concatenate([K, k_new[None]])
        V = np.concatenate([V, v_new[None]])
        p, slot = divmod(L, ps)
        if p == kmin.shape[0]:
            kmin = np.concatenate([kmin, k_new[None]])
            kmax = np.concatenate([kmax, k_new[None]])
        kmin[p], kmax[p] = O.append_minmax(kmin[p], kmax[p], k_new, slot)
        qg = O.to_f64(wl.q[b, g * G:(g + 1) * G], spec.dtype)
        ts = time.perf_counter()
        pages = O.select_pages(O.page_scores(qg, kmin, kmax), int(wl.budget_pages[b]))
        O.decode_unit(qg, K, V, pages, ps, scale)
        t_sparse += time.perf_counter() - ts
        O.dense_decode_unit(qg, K, V, ps, scale)
    O.acceptance(wl.logits_a[b], wl.logits_b[b], spec.temperature)
    return time.perf_counter() - t0, t_sparse


def _cpu_baseline(O, wl, steps_tokens, seconds):
    spec = wl.spec
    kn, vn = steps_tokens
    t_total, t_sparse, n_seq = 0.0, 0.0, 0
    for b in range(spec.batch):
        t, ts = _oracle_sequence(O, wl, kn, vn, b)
        t_total += t
        t_sparse += ts
        n_seq += 1
        if t_total >= seconds:
            break
    return {"value": n_seq / t_sparse, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"sparse path (page scores, Top-B selection, sparse attention) of {n_seq} of {spec.batch} "
                      f"sequences x {spec.num_kv_heads} KV heads, fp64 NumPy, 1 thread, timed inside the "
                      f"oracle's full step (append, select, sparse, dense, acceptance: {t_total:.1f} s of CPU time)",
            "full_step_tokens_per_s": n_seq / t_total}


_POOL_STATE = {}


def _pool_worker(seqs):
    import oracle as O
    from threadpoolctl import threadpool_limits
    st = _POOL_STATE
    with threadpool_limits(limits=1):
        ts = [_oracle_sequence(O, st["wl"], st["kn"], st["vn"], b) for b in seqs]
    return sum(t for t, _ in ts), sum(t for _, t in ts)


def cpu_baseline_pool(wl, steps_tokens):
    """The same oracle step over every sequence with one worker process per host core (forked, one BLAS
    thread each), sequences split into contiguous groups; throughput = sequences / the slowest worker's
    timed seconds. Runs before the GPU is touched, so the workers are plain forks of a CPU-only process."""
    import multiprocessing as mp
    affinity = len(os.sched_getaffinity(0))
    n = max(1, min(affinity, HOST_CPU_SHARE))
    spec = wl.spec
    _POOL_STATE.update(wl=wl, kn=steps_tokens[0], vn=steps_tokens[1])
    groups = [list(g) for g in np.array_split(np.arange(spec.batch), n) if len(g)]
    with mp.get_context("fork").Pool(len(groups)) as pool:
        res = pool.map(_pool_worker, groups)
    _POOL_STATE.clear()
    times = [t for t, _ in res]
    sparse_times = [t for _, t in res]
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": spec.batch / max(sparse_times), "unit": "tokens/s", "cores": len(groups), "kind": "oracle",
            "affinity_cores": affinity, "cpu_model": model,
            "sample": f"sparse path (page scores, Top-B selection, sparse attention) of all {spec.batch} sequences "
                      f"in {len(groups)} forked workers (one BLAS thread each; the host's share is "
                      f"{HOST_CPU_SHARE} cores per GPU); slowest worker {max(sparse_times):.2f} s",
            "full_step_tokens_per_s": spec.batch / max(times)}


def env_info(torch):
    """Device, runtime and library versions of the run."""
    p = torch.cuda.get_device_properties(0)
    return {"device": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "memory_GiB": round(p.total_memory / 2 ** 30, 1), "hip": torch.version.hip, "torch": torch.__version__}


VERIFY_POSITIONS = 7  # k = 6 drafted tokens plus the bonus position (S3R's measured setting)


def speculative_rows(args, spec, wl, cache, dev, up, timed_loop, lens):
    """Dense verification of a k = 6 draft and exact speculative sampling, on the same cache.

    The last 7 cached tokens of every sequence are the verified positions; the
    logits (64 x 7 verifier rows, 64 x 6 drafter rows of 151936) follow the
    acceptance workload's recipe (a ~ N(0, 3), drafter = a + N(0, 0.3)), the
    drafts are drawn from the drafter's softmax, the uniforms are seeded.
    """
    import torch
    from sparse_attention_decode_page_amd import spdec
    from sparse_attention_decode_page_amd import synth as S
    T, k = VERIFY_POSITIONS, VERIFY_POSITIONS - 1
    r = np.random.default_rng(args.seed + 101)
    B, V = spec.batch, wl.logits_a.shape[1]
    qv = up(S.f32_to_bf16_bits(r.standard_normal((B, T, spec.num_q_heads, spec.head_dim), dtype=np.float32)))
    ws_v = torch.zeros(spdec.verify_workspace_bytes(cache, T), dtype=torch.uint8, device=dev)
    o_v = torch.empty((B, T, spec.num_q_heads, spec.head_dim), dtype=torch.float32, device=dev)
    l_v = torch.empty((B, T, spec.num_q_heads), dtype=torch.float32, device=dev)
    for _ in range(3):
        spdec.verify_decode(cache, qv, out=o_v, lse=l_v, workspace=ws_v)
    t_v = timed_loop(lambda i: spdec.verify_decode(cache, qv, out=o_v, lse=l_v, workspace=ws_v))
    kv_bytes = int(2 * spec.num_kv_heads * lens.sum() * spec.head_dim * 2)

    p_log = (3.0 * r.standard_normal((B, T, V), dtype=np.float32))
    q_log = (p_log[:, :k] + 0.3 * r.standard_normal((B, k, V), dtype=np.float32)).astype(np.float32)
    draft = np.empty((B, k), dtype=np.int32)
    for b in range(B):
        for i in range(k):
            x = q_log[b, i].astype(np.float64)
            w = np.exp(x - x.max())
            draft[b, i] = r.choice(V, p=w / w.sum())
    ua = torch.from_numpy(r.random((B, k)).astype(np.float32)).to(dev)
    us = torch.from_numpy(r.random(B).astype(np.float32)).to(dev)
    pt, qt, dt = torch.from_numpy(p_log).to(dev), torch.from_numpy(q_log).to(dev), torch.from_numpy(draft).to(dev)
    ws_s = torch.zeros(spdec.spec_accept_workspace_bytes(B, k, V), dtype=torch.uint8, device=dev)
    n_acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, dtype=torch.int32, device=dev)

    def accept():
        spdec.spec_accept(pt, qt, dt, ua, us, 1.0, num_accepted=n_acc, next_token=tok, workspace=ws_s)

    for _ in range(3):
        accept()
    t_s = timed_loop(lambda i: accept())
    kept = n_acc.cpu().numpy()
    # bytes every call must read: all verifier and drafter rows once, plus the draw row(s) of each sequence
    draw_rows = int(sum(2 if n < k else 1 for n in kept))
    acc_bytes = int((B * (2 * k + 1) + draw_rows) * V * 4)
    return {
        "positions": T,
        "verify_us": t_v * 1e6, "verify_bytes": kv_bytes, "verify_GBps": kv_bytes / t_v / 1e9,
        "verify_frac_hbm": kv_bytes / t_v / 1e9 / HBM_PEAK_GBPS,
        "verified_tokens_per_s": B * T / t_v,
        "accept_us": t_s * 1e6, "accept_bytes": acc_bytes, "accept_GBps": acc_bytes / t_s / 1e9,
        "mean_kept_drafts": float(kept.mean()),
        "verify_traffic": traffic_sum(counter_traffic(f"verify_{spec.name}"),
                                      ["verify_stream_kernel<*,false>", "verify_merge_kernel<*>"]),
        "accept_traffic": traffic_sum(counter_traffic(f"verify_{spec.name}"),
                                      ["spec_stats_kernel<*>", "spec_decide_kernel", "spec_chunk_kernel<*>",
                                       "spec_sample_kernel"]),
        "timing": "each call K times back to back under one event pair",
    }


def make_timers(dev, K):
    """timed_loop(body): mean seconds per call of K calls back to back under one event pair (on torch's current
    stream, the stream every spdec call is enqueued on). scrubbed(body): seconds per call when each call follows
    a 1 GiB scrub read (so neither L2 nor the 256 MB last-level cache holds what the previous call read),
    K x (scrub, call) minus K x scrub, the two loops interleaved three times and the median taken."""
    import torch
    scrub = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    scrub_out = torch.empty((), dtype=torch.float32, device=dev)

    def scrub_read():
        # a read, not a write: written lines would be written back while the timed call runs
        torch.sum(scrub, dim=0, out=scrub_out)

    def timed_loop(body):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        evs[0].record()
        for i in range(K):
            body(i)
        evs[1].record()
        torch.cuda.synchronize()
        return evs[0].elapsed_time(evs[1]) * 1e-3 / K

    def scrubbed(body, reps=3, runs=None):
        for _ in range(2):
            scrub_read()
            body(0)
        diffs = []
        for _ in range(reps):
            t0 = timed_loop(lambda i: scrub_read())
            t1 = timed_loop(lambda i: (scrub_read(), body(i)))
            diffs.append(t1 - t0)
        if runs is not None:
            runs.extend(diffs)
        return float(np.median(diffs))

    return timed_loop, scrubbed, (scrub, scrub_out)


def _probe_lib():
    import ctypes
    from sparse_attention_decode_page_amd import build as B
    if not os.path.exists(B.PROBE_LIB_PATH):
        raise RuntimeError(f"{B.PROBE_LIB_PATH} is not built; run sparse_attention_decode_page_amd.build.build()")
    L = ctypes.CDLL(B.PROBE_LIB_PATH)
    L.spdec_probe_gather.restype = ctypes.c_int
    L.spdec_probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    L.spdec_probe_sink_words.restype = ctypes.c_int
    return L


def gather_ceiling(cache, spec, sel_idx, sel_cnt, scrubbed, t_select=None, t_decode=None, t_path=None):
    """The gather-read ceiling of the sparse path's two streams on this cache: a kernel with the stream
    kernels' access pattern and no arithmetic (libspdec_probe.so) reads (a) the kept pages' K and V blocks, in
    the decode's order, and (b) every page's summary, in the scoring pass's order; each timed like the calls
    (after a scrub read). The calls' times set against these give the fraction of the reachable rate."""
    import torch
    L = _probe_lib()
    dev = sel_idx.device
    B, H, cap = sel_idx.shape
    ps, D = spec.page_size, spec.head_dim
    pt = cache.page_table.long()
    keep = torch.arange(cap, device=dev)[None, None, :] < sel_cnt.long()[:, :, None]
    bi, gi, _ = keep.nonzero(as_tuple=True)                 # unit-major, entries ascending
    phys = pt[bi, sel_idx[keep].long()]
    kv_off = ((phys * H + gi) * (ps * D * 2)).contiguous()
    lens = cache.seq_lens.long()
    P = torch.clamp((lens + ps - 1) // ps, max=pt.shape[1])
    allp = (torch.arange(pt.shape[1], device=dev)[None, :] < P[:, None])[:, None, :].expand(B, H, pt.shape[1])
    bj, gj, pj = allp.nonzero(as_tuple=True)
    sm_off = ((pt[bj, pj] * H + gj) * (2 * D * 2)).contiguous()
    sink = torch.zeros(L.spdec_probe_sink_words(), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def probe(base0, base1, off, nbytes):
        rc = L.spdec_probe_gather(base0.data_ptr(), None if base1 is None else base1.data_ptr(), off.data_ptr(),
                                  off.numel(), nbytes, sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"spdec_probe_gather failed ({rc})")

    t_kv = scrubbed(lambda i: probe(cache.k_pool, cache.v_pool, kv_off, ps * D * 2))
    t_sm = scrubbed(lambda i: probe(cache.kminmax, None, sm_off, 2 * D * 2))
    b_kv = int(kv_off.numel()) * ps * D * 2 * 2
    b_sm = int(sm_off.numel()) * 2 * D * 2
    res = {"kv_pages": dict(_row(t_kv, b_kv), blocks=int(kv_off.numel()), block_bytes=ps * D * 2, pools=2),
           "summaries": dict(_row(t_sm, b_sm), blocks=int(sm_off.numel()), block_bytes=2 * D * 2, pools=1),
           "probe": "libspdec_probe.so: the stream kernels' walk (per-wave contiguous ranges, 64 offsets per "
                    "window, 16-byte non-temporal loads) with no arithmetic",
           "timing": "median of 3 x (K x (1 GiB scrub read, probe) minus K x scrub)"}
    if t_decode is not None:
        res["sparse_decode_over_ceiling"] = t_kv / t_decode
    if t_select is not None:
        res["select_pages_over_ceiling"] = t_sm / t_select
    if t_path is not None:
        res["sparse_path_over_ceiling"] = (t_kv + t_sm) / t_path
    del kv_off, sm_off, sink
    return res


def call_kernels(spec, form="one kernel", select_form="two calls"):
    """Name patterns (over the counter summaries' kernel names) of the kernels each call launches on a bf16
    workload of this shape; the merge's form and the Top-B's size class depend on the workload, the step's and
    the selection's forms (one kernel, sliced, or two calls / two kernels) on the batch."""
    D, G = spec.head_dim, spec.group
    dec = (lambda sp: f"decode_stream_g8_kernel<{D},{sp}>") if G == 8 else \
        (lambda sp: f"decode_stream_kernel<{D},{G},{sp}>")
    select = {"one kernel": [f"select_path_kernel<{D},{G}>"],
              "sliced": [f"slice_score_kernel<{D},{G}>", f"slice_select_kernel<{D},{G},false>"]}.get(
        select_form, [f"score_stream_kernel<BF16,{D},{G}>", "select_topk_reg_kernel<*>"])
    calls = {"select_pages": select,
             "sparse_decode": [dec("true"), f"stream_merge_kernel<{D},*,true>"],
             "dense_decode": [dec("false"), f"stream_merge_kernel<{D},*,false>"]}
    calls["sparse_path"] = {
        "one kernel": [f"sparse_path_kernel<{D},{G}>"],
        "sliced": [f"slice_score_kernel<{D},{G}>", f"slice_select_kernel<{D},{G},true>",
                   f"stream_merge_kernel<{D},64,4,true>"],
    }.get(form, calls["select_pages"] + calls["sparse_decode"])
    return calls


def copy_probe(torch, dev):
    """Three plain 1 GiB device-to-device copies: the known byte count that calibrates the HBM counters."""
    x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    n = int(x.numel() * 4)
    del x, y
    torch.cuda.empty_cache()
    return n


def traffic_sum(traffic, patterns):
    """Summed bytes per call of the kernels matching `patterns` (each must match exactly one kernel)."""
    import fnmatch
    if traffic is None:
        return None
    total = 0
    for pat in patterns:
        hits = [k for k in traffic if fnmatch.fnmatchcase(k, pat)]
        if len(hits) != 1:
            return None
        total += traffic[hits[0]]
    return int(total)


def acceptance_ceiling(la, lb, scrubbed, t_call=None):
    """The read-rate ceiling of the acceptance: the probe streams both logit arrays (contiguous, in 16 KiB
    blocks) with no arithmetic, after a scrub read like the call."""
    import torch
    L = _probe_lib()
    nbytes = la.numel() * la.element_size()
    blk = 16384
    if nbytes % blk or lb.numel() * lb.element_size() != nbytes or not (la.is_contiguous() and lb.is_contiguous()):
        return None
    off = torch.arange(nbytes // blk, dtype=torch.int64, device=la.device) * blk
    sink = torch.zeros(L.spdec_probe_sink_words(), dtype=torch.int32, device=la.device)
    stream = torch.cuda.current_stream().cuda_stream

    def probe(i=0):
        rc = L.spdec_probe_gather(la.data_ptr(), lb.data_ptr(), off.data_ptr(), off.numel(), blk, sink.data_ptr(),
                                  stream)
        if rc != 0:
            raise RuntimeError(f"spdec_probe_gather failed ({rc})")

    t = scrubbed(probe)
    res = dict(_row(t, 2 * nbytes), block_bytes=blk,
               timing="median of 3 x (K x (1 GiB scrub read, probe) minus K x scrub)")
    if t_call is not None:
        res["acceptance_over_ceiling"] = t / t_call
    return res


def _row(t, b):
    return {"us": t * 1e6, "bytes": int(b), "GBps": b / t / 1e9, "frac_hbm": b / t / 1e9 / HBM_PEAK_GBPS}


def upload_cache(wl, dev):
    import torch
    from sparse_attention_decode_page_amd import spdec
    spec = wl.spec

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    kmm = torch.zeros((wl.num_phys, spec.num_kv_heads, 2, spec.head_dim), dtype=torch.bfloat16, device=dev)
    cache = spdec.PagedCache(up(wl.k_pool), up(wl.v_pool), kmm, torch.from_numpy(wl.page_table).to(dev),
                             torch.from_numpy(wl.lens.astype(np.int32)).to(dev), spec.num_q_heads)
    spdec.build_meta(cache)
    return cache, up(wl.q)


def layer_rows(args, dev, timers, name, acceptance=False):
    """One decode-layer workload: the sparse path and its two calls (each call after a scrub read), the dense
    decode back to back, tokens/s, algorithmic GB/s and the fraction of 8 TB/s; with acceptance, the acceptance
    of the workload's logit rows (after a scrub read) and their mean and lower 5th percentile on the device."""
    import torch
    from sparse_attention_decode_page_amd import spdec
    from sparse_attention_decode_page_amd import synth as S
    timed_loop, scrubbed, _ = timers
    wl = S.make_workload(name, seed=args.seed)
    spec = wl.spec
    cache, q = upload_cache(wl, dev)
    budget = torch.from_numpy(wl.budget_pages.astype(np.int32)).to(dev)
    cap = int(max(2, wl.budget_pages.max()))
    sel_idx = torch.zeros((spec.batch, spec.num_kv_heads, cap), dtype=torch.int32, device=dev)
    sel_cnt = torch.zeros((spec.batch, spec.num_kv_heads), dtype=torch.int32, device=dev)
    ws_sel = torch.zeros(spdec.select_workspace_bytes(cache, cap), dtype=torch.uint8, device=dev)
    ws_sp = torch.zeros(spdec.decode_workspace_bytes(cache, cap), dtype=torch.uint8, device=dev)
    ws_de = torch.zeros(spdec.decode_workspace_bytes(cache, 0), dtype=torch.uint8, device=dev)
    ws_path = torch.zeros(spdec.sparse_path_workspace_bytes(cache, cap), dtype=torch.uint8, device=dev)
    o = torch.empty((spec.batch, spec.num_q_heads, spec.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((spec.batch, spec.num_q_heads), dtype=torch.float32, device=dev)
    form = spdec.sparse_path_form(cache, cap)
    select_form = spdec.select_pages_form(cache, cap)

    def path(i=0):
        spdec.sparse_path(cache, q, budget, cap, sel_idx=sel_idx, sel_cnt=sel_cnt, out=o, lse=lse, workspace=ws_path)

    def sel(i=0):
        spdec.select_pages(cache, q, budget, cap, sel_idx=sel_idx, sel_cnt=sel_cnt, workspace=ws_sel)

    def dec(i=0):
        spdec.sparse_decode(cache, q, sel_idx, sel_cnt, cap, out=o, lse=lse, workspace=ws_sp)

    def dense(i=0):
        spdec.dense_decode(cache, q, out=o, lse=lse, workspace=ws_de)

    for _ in range(3):
        path()
        sel()
        dec()
        dense()
    t_path = scrubbed(path)
    t_two = scrubbed(lambda i: (sel(), dec()))
    t_sel = scrubbed(sel)
    t_dec = scrubbed(dec)
    t_dense = timed_loop(dense)
    byt = algorithmic_bytes(spec, wl.lens, wl.budget_pages, cap, 0, 0)
    b_path = byt["sparse_path"]
    res = {
        "workload": spec.name, "batch": spec.batch, "q_heads": spec.num_q_heads, "kv_heads": spec.num_kv_heads,
        "head_dim": spec.head_dim, "page_size": spec.page_size, "context": describe_lens(spec),
        "budget": describe_budget(spec),
        "sparse_path": dict(_row(t_path, b_path), tokens_per_s=spec.batch / t_path, form=form),
        "two_calls": dict(_row(t_two, b_path), tokens_per_s=spec.batch / t_two),
        "select_pages": dict(_row(t_sel, byt["select_pages"]), form=select_form),
        "sparse_decode": _row(t_dec, byt["sparse_decode"]),
        "dense_decode": dict(_row(t_dense, byt["dense_decode"]), tokens_per_s=spec.batch / t_dense),
        "sparse_over_dense": t_dense / t_path,
        "timing": "sparse calls: median of 3 x (K x (1 GiB scrub read, call) minus K x scrub); dense: K calls back "
                  "to back",
    }
    traffic = counter_traffic(spec.name)
    ck = call_kernels(spec, form, select_form)
    for call in ("sparse_path", "select_pages", "sparse_decode", "dense_decode"):
        res[call]["traffic"] = traffic_sum(traffic, ck[call])
    res["two_calls"]["traffic"] = traffic_sum(traffic, ck["select_pages"] + ck["sparse_decode"])
    res["kernels"] = ck
    if not args.no_gather_ceiling:
        sel()
        res["gather_ceiling"] = gather_ceiling(cache, spec, sel_idx, sel_cnt, scrubbed, t_sel, t_dec, t_path)
    if acceptance:
        la = torch.from_numpy(wl.logits_a).to(dev)
        lb = torch.from_numpy(wl.logits_b).to(dev)
        R, V = wl.logits_a.shape
        ws_a = torch.zeros(spdec.acceptance_workspace_bytes(R, V), dtype=torch.uint8, device=dev)
        alpha = torch.empty(R, dtype=torch.float32, device=dev)
        tail = torch.empty(2, dtype=torch.float32, device=dev)

        def acc(i=0, path=-1):
            spdec.acceptance_ex(la, lb, spec.temperature, alpha=alpha, workspace=ws_a, force_path=path)

        t_acc = scrubbed(acc)
        t_acc2 = scrubbed(lambda i: acc(i, 2))
        acc()
        spdec.tail_stats(alpha, out=tail)
        torch.cuda.synchronize()
        res["acceptance"] = dict(_row(t_acc, 2 * R * V * 4), rows=R, vocab=V, temperature=spec.temperature,
                                 mean=float(tail[0]), p5=float(tail[1]),
                                 two_pass_us=t_acc2 * 1e6,
                                 timing="median of 3 x (K x (1 GiB scrub read, call) minus K x scrub)")
        if not args.no_gather_ceiling:
            res["acceptance"]["read_ceiling"] = acceptance_ceiling(la, lb, scrubbed, t_acc)
        del la, lb, ws_a
    del cache, q, ws_sel, ws_sp, ws_de, ws_path, sel_idx, sel_cnt
    torch.cuda.empty_cache()
    return res


def shared_prefix_rows(args, dev, timed_loop):
    """Dense decode of a grouped batch (8 prompts x 8 samples, 16K-token shared prompts), per sequence and with
    the shared prompt pages read once per group."""
    import torch
    from sparse_attention_decode_page_amd import spdec
    from sparse_attention_decode_page_amd import synth as S
    wl = S.make_workload("qwen3-8b-grouped", seed=args.seed)
    spec = wl.spec
    N = spec.prompt[1]

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    kmm = torch.zeros((wl.num_phys, spec.num_kv_heads, 2, spec.head_dim), dtype=torch.bfloat16, device=dev)
    cache = spdec.PagedCache(up(wl.k_pool), up(wl.v_pool), kmm, torch.from_numpy(wl.page_table).to(dev),
                             torch.from_numpy(wl.lens.astype(np.int32)).to(dev), spec.num_q_heads)
    q = up(wl.q)
    sh = torch.from_numpy(wl.shared_pages).to(dev)
    ws_d = torch.zeros(spdec.decode_workspace_bytes(cache, 0), dtype=torch.uint8, device=dev)
    ws_s = torch.zeros(spdec.shared_workspace_bytes(cache, N), dtype=torch.uint8, device=dev)
    o = torch.empty((spec.batch, spec.num_q_heads, spec.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((spec.batch, spec.num_q_heads), dtype=torch.float32, device=dev)
    for _ in range(3):
        spdec.dense_decode(cache, q, out=o, lse=lse, workspace=ws_d)
        spdec.dense_decode_shared(cache, q, N, sh, out=o, lse=lse, workspace=ws_s)
    t_d = timed_loop(lambda i: spdec.dense_decode(cache, q, out=o, lse=lse, workspace=ws_d))
    t_s = timed_loop(lambda i: spdec.dense_decode_shared(cache, q, N, sh, out=o, lse=lse, workspace=ws_s))
    # Page selection of the same batch: every sequence scores its own pages, or
    # the shared prompt pages are scored once per group.
    spdec.build_meta(cache)
    budget = torch.from_numpy(wl.budget_pages.astype(np.int32)).to(dev)
    kb = int(max(2, wl.budget_pages.max()))
    sel_idx = torch.zeros((spec.batch, spec.num_kv_heads, kb), dtype=torch.int32, device=dev)
    sel_cnt = torch.zeros((spec.batch, spec.num_kv_heads), dtype=torch.int32, device=dev)
    ws_sel = torch.zeros(spdec.select_workspace_bytes(cache, kb), dtype=torch.uint8, device=dev)
    ws_sp = torch.zeros(spdec.decode_workspace_bytes(cache, kb), dtype=torch.uint8, device=dev)

    def sel(shared):
        if shared:
            spdec.select_pages_shared(cache, q, N, sh, budget, kb, sel_idx, sel_cnt, workspace=ws_sel)
        else:
            spdec.select_pages(cache, q, budget, kb, sel_idx, sel_cnt, workspace=ws_sel)

    def path(shared):
        sel(shared)
        spdec.sparse_decode(cache, q, sel_idx, sel_cnt, kb, out=o, lse=lse, workspace=ws_sp)

    for _ in range(3):
        path(False)
        path(True)
    t_sel = timed_loop(lambda i: sel(False))
    t_sel_s = timed_loop(lambda i: sel(True))
    t_path = timed_loop(lambda i: path(False))
    t_path_s = timed_loop(lambda i: path(True))
    L = wl.lens.astype(np.int64)
    per_tok = 2 * spec.num_kv_heads * spec.head_dim * 2
    shared_tokens = int(wl.shared_pages.sum()) * spec.page_size
    bytes_dense = int(L.sum() * per_tok)
    bytes_shared = int((L.sum() - (N - 1) * shared_tokens) * per_tok)
    P = (L + spec.page_size - 1) // spec.page_size
    per_summary = spec.num_kv_heads * 2 * spec.head_dim * 2
    sum_bytes = int(P.sum() * per_summary)
    sum_bytes_s = int((P.sum() - (N - 1) * int(wl.shared_pages.sum())) * per_summary)
    del cache, kmm, q, ws_d, ws_s, ws_sel, ws_sp
    torch.cuda.empty_cache()
    traffic = counter_traffic(f"shared_{spec.name}")
    return {
        "select_us": t_sel * 1e6, "select_shared_us": t_sel_s * 1e6, "select_speedup": t_sel / t_sel_s,
        "select_summary_bytes": sum_bytes, "select_shared_summary_bytes": sum_bytes_s,
        "sparse_path_us": t_path * 1e6, "sparse_path_shared_select_us": t_path_s * 1e6,
        "workload": spec.name, "groups": spec.batch // N, "group_size": N, "prompt_tokens": spec.prompt[2],
        "dense_us": t_d * 1e6, "dense_bytes": bytes_dense, "dense_GBps": bytes_dense / t_d / 1e9,
        "shared_us": t_s * 1e6, "shared_bytes": bytes_shared, "shared_GBps": bytes_shared / t_s / 1e9,
        "shared_frac_hbm": bytes_shared / t_s / 1e9 / HBM_PEAK_GBPS, "speedup": t_d / t_s,
        "tokens_per_s": spec.batch / t_s,
        "dense_traffic": traffic_sum(traffic, ["decode_stream_kernel<128,4,false>", "stream_merge_kernel<128,*,false>"]),
        "shared_traffic": traffic_sum(traffic, ["verify_stream_kernel<*,true>", "decode_stream_kernel<128,4,false>@suffix",
                                                "shared_merge_kernel<*>"]),
        "select_shared_traffic": traffic_sum(traffic, ["score_grouped_kernel<*>", "select_topk_reg_kernel<*>"]),
        "timing": "each call K times back to back under one event pair",
    }


def budget_control_rows(args, spec, cache, q, dev, sel_idx, sel_cnt, ws_path, cap, timed_loop):
    """Closed loop of the sparsity-schedule controller on the device: budgets -> selection -> sparse decode ->
    a seeded random LM head (the plant stand-in: no model weights) -> acceptance against the dense output's
    logits -> streaming tail monitor over the last steps' tokens -> controller -> budgets, with no host round
    trip inside the loop."""
    import torch
    from sparse_attention_decode_page_amd import spdec
    B, H = spec.batch, spec.num_q_heads * spec.head_dim
    vocab, sigma, steps, window_steps = 151936, 3.0, 30, 4
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 17)
    w_lm = torch.randn((H, vocab), generator=gen, device=dev, dtype=torch.float32) * (sigma / H ** 0.5)
    o_d, _ = spdec.dense_decode(cache, q)           # the reference on the cache as it now stands
    logit_d = torch.matmul(o_d.reshape(B, H), w_lm)
    logit_s = torch.empty_like(logit_d)
    o_s = torch.empty_like(o_d)
    l_s = torch.empty((B, spec.num_q_heads), dtype=torch.float32, device=dev)
    al = torch.empty(B, dtype=torch.float32, device=dev)
    ws_a = torch.zeros(spdec.acceptance_workspace_bytes(B, vocab), dtype=torch.uint8, device=dev)
    mon = spdec.TailMonitor(window_steps * B)   # the tail over the last window_steps steps' tokens
    prm = spdec.BudgetParams(target=0.86, gain=6.0, scale_min=1.0 / 64, scale_max=4.0, base_tokens=1024.0,
                             tokens_per_token=0.1, page_size=spec.page_size, max_budget_pages=cap)
    scale = torch.full((1,), 1.0 / 16, dtype=torch.float32, device=dev)   # start aggressive
    bud = torch.empty(B, dtype=torch.int32, device=dev)
    tails = torch.zeros((steps + 1, 2), dtype=torch.float32, device=dev)
    tails[0, 1] = float("nan")                       # first step: no monitor value yet, schedule as it stands
    buds = torch.zeros((steps, B), dtype=torch.int32, device=dev)

    def control_step(k):
        spdec.budget_update(tails[k], scale, cache.seq_lens, prm, budget_pages=bud)
        buds[k].copy_(bud)
        spdec.sparse_path(cache, q, bud, cap, sel_idx=sel_idx, sel_cnt=sel_cnt, out=o_s, lse=l_s, workspace=ws_path)
        torch.matmul(o_s.reshape(B, H), w_lm, out=logit_s)
        spdec.acceptance(logit_s, logit_d, 1.0, alpha=al, workspace=ws_a)
        mon.append(al)
        mon.stats(out=tails[k + 1])

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for k in range(steps):
        control_step(k)
    ev[1].record()
    torch.cuda.synchronize()
    t_loop = ev[0].elapsed_time(ev[1]) * 1e-3 / steps
    p5 = tails[1:, 1].cpu().numpy()
    mb = buds.float().mean(dim=1).cpu().numpy()
    within = np.abs(p5 - 0.86) <= 0.02
    settled = next((k for k in range(steps) if within[k:].all()), None)
    tail_fix = torch.tensor([0.0, 0.86], dtype=torch.float32, device=dev)
    s_fix = torch.ones(1, dtype=torch.float32, device=dev)
    for _ in range(3):
        spdec.budget_update(tail_fix, s_fix, cache.seq_lens, prm, budget_pages=bud)
    t_upd = timed_loop(lambda i: spdec.budget_update(tail_fix, s_fix, cache.seq_lens, prm, budget_pages=bud))
    del w_lm, logit_d, logit_s, ws_a
    torch.cuda.empty_cache()
    return {
        "plant": f"sparse vs dense attention outputs of this cache through a seeded N(0, {sigma}^2/{H}) LM head, "
                 f"vocab {vocab}, T = 1",
        "target_p5": 0.86, "gain": 6.0, "schedule": "s * (1024 + 0.1 * L) tokens, pages of 16, 2 .. cap",
        "start_scale": 1.0 / 16, "steps": steps, "p5": [round(float(x), 4) for x in p5],
        "mean_budget_pages": [round(float(x), 1) for x in mb], "final_scale": float(scale.item()),
        "settled_step": settled, "final_p5": float(p5[-1]),
        "monitor_window_tokens": window_steps * B,
        "control_step_us": t_loop * 1e6, "update_us": t_upd * 1e6,
        "timing": "control_step: the whole loop body (update, select, sparse decode, LM-head GEMM, acceptance, "
                  "monitor append and statistics) averaged over the steps under one event pair; update: the "
                  "controller call alone, K times back to back",
    }


def monitor_rows(args, dev, timed_loop, batch=64, tokens=32768):
    """The streaming tail monitor over a rollout's tokens: a window of batch x tokens per-token acceptance values
    (2,097,152 for 64 sequences of 32768 tokens), filled with acceptance-like values; the append of one decode
    step's batch and the statistics (mean and exact lower 5th percentile) of the full window."""
    import torch
    from sparse_attention_decode_page_amd import spdec
    cap = batch * tokens
    r = np.random.default_rng(args.seed + 23)
    vals = np.clip(1.0 - np.abs(r.standard_normal(cap)) * 0.03 - (r.random(cap) < 0.05) * r.random(cap) * 0.5,
                   0, 1).astype(np.float32)
    mon = spdec.TailMonitor(cap, device=dev)
    mon.append(torch.from_numpy(vals).to(dev))
    step_vals = torch.from_numpy(vals[:batch].copy()).to(dev)
    out = torch.empty(2, dtype=torch.float32, device=dev)
    for _ in range(3):
        mon.stats(out=out)
    t_stats = timed_loop(lambda i: mon.stats(out=out))
    t_append = timed_loop(lambda i: mon.append(step_vals))
    mon.stats(out=out)
    torch.cuda.synchronize()
    res = {"window": cap, "stats_us": t_stats * 1e6, "append_us": t_append * 1e6, "append_values": batch,
           "stats_GBps": cap * 4 * 3 / t_stats / 1e9, "mean": float(out[0]), "p5": float(out[1]),
           "timing": "each call K times back to back under one event pair (stats reads the window in three "
                     "histogram passes and, when no tie covers the next rank, once more)"}
    del mon, step_vals
    torch.cuda.empty_cache()
    return res


def top_p_rows(spec, cache, q, budget, dev, timed_loop):
    """Score-mass (top-p) selection on the step's cache: its time beside the Top-B selection's, the pages it
    keeps without a cap (the budget then follows the query) and under the per-sequence budgets, and the
    sparse path with it."""
    import torch
    from sparse_attention_decode_page_amd import spdec
    cap = cache.max_pages
    sel_idx = torch.zeros((spec.batch, spec.num_kv_heads, cap), dtype=torch.int32, device=dev)
    sel_cnt = torch.zeros((spec.batch, spec.num_kv_heads), dtype=torch.int32, device=dev)
    ws_sel = torch.zeros(spdec.select_workspace_bytes(cache, cap), dtype=torch.uint8, device=dev)
    ws_sp = torch.zeros(spdec.decode_workspace_bytes(cache, cap), dtype=torch.uint8, device=dev)
    o_s = torch.empty((spec.batch, spec.num_q_heads, spec.head_dim), dtype=torch.float32, device=dev)
    l_s = torch.empty((spec.batch, spec.num_q_heads), dtype=torch.float32, device=dev)
    res = {"score_scale": 1.0 / (spec.group * math.sqrt(spec.head_dim))}

    def topb():
        spdec.select_pages(cache, q, budget, cap, sel_idx=sel_idx, sel_cnt=sel_cnt, workspace=ws_sel)

    for _ in range(3):
        topb()
    res["select_top_b_us"] = timed_loop(lambda i: topb()) * 1e6
    res["top_b_mean_pages"] = float(sel_cnt.float().mean())
    for name, p, bud in (("p0.5", 0.5, None), ("p0.9", 0.9, None), ("p0.9_budget_capped", 0.9, budget)):
        def sel(p=p, bud=bud):
            spdec.select_pages_top_p(cache, q, p, cap, budget_pages=bud, sel_idx=sel_idx, sel_cnt=sel_cnt,
                                     workspace=ws_sel)

        def path(p=p, bud=bud):
            sel(p, bud)
            spdec.sparse_decode(cache, q, sel_idx, sel_cnt, cap, out=o_s, lse=l_s, workspace=ws_sp)

        for _ in range(3):
            path()
        t_sel = timed_loop(lambda i: sel())
        kept = sel_cnt.float()
        t_path = timed_loop(lambda i: path())
        res[name] = {"select_us": t_sel * 1e6, "mean_pages": float(kept.mean()), "min_pages": float(kept.min()),
                     "max_pages": float(kept.max()), "sparse_path_us": t_path * 1e6}
    del sel_idx, sel_cnt, ws_sel, ws_sp
    torch.cuda.empty_cache()
    # the top-p selection takes one kernel where the Top-B selection does, else the scoring and top-p kernels
    one = spdec.select_pages_form(cache, cap) == "one kernel"
    topp_kernels = [f"select_topp_path_kernel<{spec.head_dim},{spec.group}>"] if one else \
        ["score_stream_kernel<*>", "select_topp_reg_kernel<*>"]
    res["select_top_p_form"] = "one kernel" if one else "two kernels"
    res["select_top_p_kernels"] = " + ".join(topp_kernels)
    res["select_top_p_traffic"] = traffic_sum(counter_traffic(f"top-p_{spec.name}"), topp_kernels)
    res["timing"] = "each call K times back to back under one event pair"
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this path has no multi-GPU mode "
              "(the per-(sequence, KV head) work shards without any exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from sparse_attention_decode_page_amd import spdec
    from sparse_attention_decode_page_amd import synth as S

    K_steps, W = args.steps, args.warmup
    if args.layer:
        if not os.path.exists(spdec.LIB_PATH):
            from sparse_attention_decode_page_amd import build
            build.build()
        spdec.lib()
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        timers = make_timers(dev, K_steps)
        layers = {}
        for name in args.layer.split(","):
            layers[name] = layer_rows(args, dev, timers, name, acceptance=S.SPECS[name].logits is not None)
            print(f"layer {name} done", file=sys.stderr, flush=True)
        out = {"mode": "layer", "steps": K_steps, "layers": layers, "env": env_info(torch)}
        if args.copy_probe:
            out["copy_probe_bytes"] = copy_probe(torch, dev)
        print(json.dumps(out), flush=True)
        return
    t_setup = time.perf_counter()
    wl = S.make_workload(args.workload, seed=args.seed, headroom=5 * K_steps + 2 * W + 2)
    spec = wl.spec
    pool_baseline = None
    if not args.no_cpu_baseline:
        # all of the host's share of cores, before any GPU state exists in this process (the workers are forks)
        t_first = S.append_tokens(wl, 0)
        pool_baseline = cpu_baseline_pool(wl, (t_first[0], t_first[1]))
        t_setup = time.perf_counter()
    if not os.path.exists(spdec.LIB_PATH):
        from sparse_attention_decode_page_amd import build
        build.build()
    spdec.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    assert spec.logits is not None, "the step needs logit rows for the acceptance row"
    tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32

    def up(x):
        if spec.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)

    k_pool, v_pool = up(wl.k_pool), up(wl.v_pool)
    kminmax = torch.zeros((wl.num_phys, spec.num_kv_heads, 2, spec.head_dim), dtype=tdt, device=dev)
    page_table = torch.from_numpy(wl.page_table).to(dev)
    seq_lens = torch.from_numpy(wl.lens.astype(np.int32)).to(dev)
    cache = spdec.PagedCache(k_pool, v_pool, kminmax, page_table, seq_lens, spec.num_q_heads)
    q = up(wl.q)
    budget = torch.from_numpy(wl.budget_pages.astype(np.int32)).to(dev)
    cap = int(wl.budget_pages.max())
    new_tokens = [S.append_tokens(wl, s) for s in range(2 * K_steps + W)]
    k_new = [up(t[0]) for t in new_tokens]
    v_new = [up(t[1]) for t in new_tokens]
    la = torch.from_numpy(wl.logits_a).to(dev)
    lb = torch.from_numpy(wl.logits_b).to(dev)
    R, V = wl.logits_a.shape
    # preallocated outputs and workspaces: the timed loops allocate nothing
    sel_idx = torch.zeros((spec.batch, spec.num_kv_heads, cap), dtype=torch.int32, device=dev)
    sel_cnt = torch.zeros((spec.batch, spec.num_kv_heads), dtype=torch.int32, device=dev)
    ws_sel = torch.zeros(spdec.select_workspace_bytes(cache, cap), dtype=torch.uint8, device=dev)
    ws_sp = torch.zeros(spdec.decode_workspace_bytes(cache, cap), dtype=torch.uint8, device=dev)
    ws_de = torch.zeros(spdec.decode_workspace_bytes(cache, 0), dtype=torch.uint8, device=dev)
    ws_path = torch.zeros(spdec.sparse_path_workspace_bytes(cache, cap), dtype=torch.uint8, device=dev)
    ws_acc = torch.zeros(spdec.acceptance_workspace_bytes(R, V), dtype=torch.uint8, device=dev)
    o_s = torch.empty((spec.batch, spec.num_q_heads, spec.head_dim), dtype=torch.float32, device=dev)
    l_s = torch.empty((spec.batch, spec.num_q_heads), dtype=torch.float32, device=dev)
    o_d, l_d = torch.empty_like(o_s), torch.empty_like(l_s)
    alpha = torch.empty(R, dtype=torch.float32, device=dev)
    spdec.build_meta(cache)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup
    if args.features:
        timed_loop, _, _ = make_timers(dev, K_steps)
        want = set(args.features.split(","))
        out = {"mode": "features", "steps": K_steps, "env": env_info(torch)}
        if "verify" in want:
            out["verify"] = speculative_rows(args, spec, wl, cache, dev, up, timed_loop, wl.lens.astype(np.int64))
        if "top-p" in want:
            out["top_p"] = top_p_rows(spec, cache, q, budget, dev, timed_loop)
        if "shared" in want:
            del cache, k_pool, v_pool, kminmax
            torch.cuda.empty_cache()
            out["shared_prefix"] = shared_prefix_rows(args, dev, timed_loop)
        if args.copy_probe:
            out["copy_probe_bytes"] = copy_probe(torch, dev)
        print(json.dumps(out), flush=True)
        return

    def sel(i=0):
        spdec.select_pages(cache, q, budget, cap, sel_idx=sel_idx, sel_cnt=sel_cnt, workspace=ws_sel)

    def dec(i=0):
        spdec.sparse_decode(cache, q, sel_idx, sel_cnt, cap, out=o_s, lse=l_s, workspace=ws_sp)

    form = spdec.sparse_path_form(cache, cap)
    select_form = spdec.select_pages_form(cache, cap)

    def sparse_path(i=0):
        spdec.sparse_path(cache, q, budget, cap, sel_idx=sel_idx, sel_cnt=sel_cnt, out=o_s, lse=l_s,
                          workspace=ws_path)

    def two_calls(i=0):
        sel()
        dec()

    def dense(i=0):
        spdec.dense_decode(cache, q, out=o_d, lse=l_d, workspace=ws_de)

    def acc(i=0, path=-1):
        spdec.acceptance_ex(la, lb, spec.temperature, alpha=alpha, workspace=ws_acc, force_path=path)

    rows = ["append_kv", "sparse_path", "dense_decode", "acceptance"]
    row_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(rows) + 1)] for _ in range(K_steps)]

    def step(i, events=None):
        rec = (lambda j: events[j].record()) if events is not None else (lambda j: None)
        rec(0)
        spdec.append_kv(cache, k_new[i], v_new[i])
        rec(1)
        sparse_path()
        rec(2)
        dense()
        rec(3)
        spdec.acceptance(la, lb, spec.temperature, alpha=alpha, workspace=ws_acc)
        rec(4)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    appended = W
    timers = make_timers(dev, K_steps)
    timed_loop, scrubbed, _ = timers

    # --- value: the sparse path (spdec_sparse_path) on the cache as it stands, each of K runs after a 1 GiB scrub
    # read, the K scrubs' own time subtracted; three interleaved regions, median. Then the same step as its two
    # calls, and each call apart.
    lens_sparse = wl.lens.astype(np.int64) + appended
    t0 = time.perf_counter()
    value_runs = []
    sp_t = scrubbed(sparse_path, reps=3, runs=value_runs)
    wall = time.perf_counter() - t0
    two_t = scrubbed(two_calls)
    sel_t = scrubbed(sel)
    dec_t = scrubbed(dec)
    sp_t_warm = timed_loop(sparse_path)
    ceiling = None
    if not args.no_gather_ceiling:
        sel()
        ceiling = gather_ceiling(cache, spec, sel_idx, sel_cnt, scrubbed, sel_t, dec_t, sp_t)
    byt_sp = algorithmic_bytes(spec, lens_sparse, wl.budget_pages, cap, R, V)
    sp_b = byt_sp["sparse_path"]
    value = spec.batch / sp_t

    # --- the whole hot path (all five rows) back to back, K steps under one event pair; then K steps with an
    # event between rows (each row's time then includes the short hold-up after the event before it).
    lens_full = wl.lens.astype(np.int64) + appended
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for i in range(K_steps):
        step(W + i)
    ev[1].record()
    torch.cuda.synchronize()
    full_t = ev[0].elapsed_time(ev[1]) * 1e-3 / K_steps
    appended += K_steps
    for i in range(K_steps):
        step((W + K_steps + i) % len(new_tokens), row_ev[i])
    torch.cuda.synchronize()
    appended += K_steps
    per_row = {r: [] for r in rows}
    for i in range(K_steps):
        for j, r in enumerate(rows):
            per_row[r].append(row_ev[i][j].elapsed_time(row_ev[i][j + 1]) * 1e-3)
    byt_full = {r: 0.0 for r in rows}
    for i in range(K_steps):
        b_i = algorithmic_bytes(spec, lens_full + i + 1, wl.budget_pages, cap, R, V)
        for r in rows:
            byt_full[r] += b_i[r] / K_steps
    mean_t = {r: float(np.mean(per_row[r])) for r in rows}
    rows_out = {r: {"us_mean": mean_t[r] * 1e6, "us_median": float(np.median(per_row[r])) * 1e6,
                    "bytes": int(byt_full[r]), "GBps": byt_full[r] / mean_t[r] / 1e9,
                    "frac_hbm": byt_full[r] / mean_t[r] / 1e9 / HBM_PEAK_GBPS} for r in rows}

    # --- calls on the cache as it now stands: dense decode back to back, acceptance after a scrub read
    lens_now = wl.lens.astype(np.int64) + appended
    byt_now = algorithmic_bytes(spec, lens_now, wl.budget_pages, cap, R, V)
    de_t = timed_loop(dense)
    acc_t = scrubbed(acc)
    acc2_t = scrubbed(lambda i: acc(i, 2))
    acc_warm = timed_loop(acc)
    acc_ceiling = acceptance_ceiling(la, lb, scrubbed, acc_t) if not args.no_gather_ceiling else None
    # --- the whole step captured once into a HIP graph and replayed K times (each replay appends the same
    # captured token)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(0)
    for _ in range(W):
        graph.replay()
    gr_t = timed_loop(lambda i: graph.replay())
    appended += W + K_steps
    del graph
    # --- on-device tail statistics of the step's acceptance values
    tail_out = torch.empty(2, dtype=torch.float32, device=dev)
    for _ in range(3):
        spdec.tail_stats(alpha, out=tail_out)
    t_tail = timed_loop(lambda i: spdec.tail_stats(alpha, out=tail_out))
    tail = {"us": t_tail * 1e6, "rows": R, "mean": float(tail_out[0]), "p5": float(tail_out[1]),
            "timing": "K times back to back under one event pair"}
    verify = speculative_rows(args, spec, wl, cache, dev, up, timed_loop, wl.lens.astype(np.int64) + appended) \
        if not args.no_verify else None
    topp = top_p_rows(spec, cache, q, budget, dev, timed_loop) if not args.no_top_p else None
    monitor = monitor_rows(args, dev, timed_loop) if not args.no_control else None
    control = budget_control_rows(args, spec, cache, q, dev, sel_idx, sel_cnt, ws_path, cap,
                                  timed_loop) if not args.no_control else None
    del cache, k_pool, v_pool, kminmax, k_new, v_new, ws_sp, ws_de, ws_sel, ws_path
    torch.cuda.empty_cache()
    shared = shared_prefix_rows(args, dev, timed_loop) if not args.no_shared else None
    shape2 = layer_rows(args, dev, timers, "qwen3-1.7b-L16k") if not args.no_second_shape else None
    long_ctx = None
    if not args.no_long:
        long_ctx = {f"ps{ps}": layer_rows(args, dev, timers, f"long-131k-ps{ps}") for ps in (8, 16, 32, 64)}
    acc_pass = layer_rows(args, dev, timers, "qwen3-8b-L32k-acceptance", acceptance=True) \
        if not args.no_acceptance_pass else None

    # HBM traffic measured by rocprofv3 counters for these kernels (bytes per call), if still current
    traffic = counter_traffic(spec.name)
    ck = call_kernels(spec, form, select_form)
    dec_kernels, sel_kernels, dense_kernels = ck["sparse_decode"], ck["select_pages"], ck["dense_decode"]
    path_kernels = ck["sparse_path"]
    acc_kernels = ["acc_one_read_kernel<true>"]

    def traffic_of(names):
        return traffic_sum(traffic, names)

    dec_gbps = byt_sp["sparse_decode"] / dec_t / 1e9
    sparse_gbps = sp_b / sp_t / 1e9
    if form == "one kernel":
        # the step is one kernel: it is the dominant (only) kernel of the path
        roofline = {"bound": "hbm", "achieved": sparse_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": sparse_gbps / HBM_PEAK_GBPS, "traffic": traffic_of(path_kernels),
                    "kernel": "spdec_sparse_path: " + " + ".join(path_kernels),
                    "bytes_per_launch": int(sp_b), "us_per_launch": sp_t * 1e6,
                    "timing": "median of 3 x (K x (1 GiB scrub read, sparse_path) minus K x scrub)"}
    else:
        roofline = {"bound": "hbm", "achieved": dec_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": dec_gbps / HBM_PEAK_GBPS, "traffic": traffic_of(dec_kernels),
                    "kernel": "sparse_decode call: " + " + ".join(dec_kernels),
                    "bytes_per_launch": int(byt_sp["sparse_decode"]), "us_per_launch": dec_t * 1e6,
                    "timing": "median of 3 x (K x (1 GiB scrub read, sparse_decode) minus K x scrub)"}
    acc_bytes = 2 * R * V * 4
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": W,
        "ms_per_step": sp_t * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": f"synthetic (seeded draws of the {spec.name} workload; no weights or datasets)",
        "config": {"workload": spec.name, "batch": spec.batch, "q_heads": spec.num_q_heads,
                   "kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim, "page_size": spec.page_size,
                   "context": describe_lens(spec), "budget": describe_budget(spec), "accumulate": "fp32",
                   "step": "spdec_sparse_path (page scores, Top-B, attention over the kept pages, LSE merge; "
                           + form
                           + "), each step after a 1 GiB scrub read",
                   "tokens_per_step": spec.batch},
        "roofline": roofline,
        "sparse": {"tokens_per_s": value, "us": sp_t * 1e6, "bytes": int(sp_b), "eff_GBps": sparse_gbps,
                   "frac_hbm": sparse_gbps / HBM_PEAK_GBPS, "form": form,
                   "traffic": traffic_of(path_kernels), "kernels": " + ".join(path_kernels),
                   "timing": "median of 3 x (K x (1 GiB scrub read, sparse_path) minus K x scrub)",
                   "us_no_scrub": sp_t_warm * 1e6,
                   "two_calls": dict(_row(two_t, sp_b), tokens_per_s=spec.batch / two_t,
                                     traffic=traffic_of(sel_kernels + dec_kernels),
                                     kernels=" + ".join(sel_kernels + dec_kernels),
                                     timing="median of 3 x (K x (1 GiB scrub read, select_pages, sparse_decode) "
                                            "minus K x scrub)"),
                   "select_pages": dict(_row(sel_t, byt_sp["select_pages"]), traffic=traffic_of(sel_kernels),
                                        form=select_form, kernels=" + ".join(sel_kernels)),
                   "sparse_decode": dict(_row(dec_t, byt_sp["sparse_decode"]), traffic=traffic_of(dec_kernels))},
        "gather_ceiling": ceiling,
        "value_runs": {"tokens_per_s": [spec.batch / t for t in value_runs], "median": value,
                       "timing": "three interleaved regions of K (scrub, sparse path) and K scrubs"},
        "dense": dict(_row(de_t, byt_now["dense_decode"]), tokens_per_s=spec.batch / de_t,
                      traffic=traffic_of(dense_kernels), kernels=" + ".join(dense_kernels),
                      timing="dense_decode K times back to back, one event pair"),
        "acceptance": dict(_row(acc_t, acc_bytes), traffic=traffic_of(acc_kernels), rows=R, vocab=V,
                           two_pass_us=acc2_t * 1e6, us_no_scrub=acc_warm * 1e6, kernels=" + ".join(acc_kernels),
                           read_ceiling=acc_ceiling,
                           timing="median of 3 x (K x (1 GiB scrub read, acceptance) minus K x scrub)"),
        "full_step": {"tokens_per_s": spec.batch / full_t, "ms_per_step": full_t * 1e3,
                      "step": "append_kv + sparse_path + dense_decode + acceptance",
                      "timing": "K steps back to back, one event pair", "rows": rows_out,
                      "graph_ms_per_step": gr_t * 1e3,
                      "graph_timing": "the step captured once in a HIP graph, replayed K times, one event pair"},
        "tail_stats": tail,
        "monitor": monitor,
        "verify": verify,
        "shared_prefix": shared,
        "qwen3_1_7b": shape2,
        "long_context": long_ctx,
        "acceptance_pass": acc_pass,
        "top_p": topp,
        "budget_control": control,
        "env": env_info(torch),
        "wall_s_value_region": wall,
        "setup_s": t_setup,
    }
    if args.copy_probe:
        result["copy_probe_bytes"] = copy_probe(torch, dev)
    if not args.no_cpu_baseline:
        kn = np.stack([t[0] for t in new_tokens[:1]])[0]
        vn = np.stack([t[1] for t in new_tokens[:1]])[0]
        result["cpu_baseline"] = cpu_baseline(wl, (kn, vn), args.cpu_seconds)
        result["cpu_baseline_all_cores"] = pool_baseline
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
