"""The bench's algorithmic byte counts (the roofline numerators), checked by brute force on tiny shapes.

Every valid token's K and V row once for the dense decode; the valid tokens of the pages the oracle's
Top-B selection keeps for the sparse decode (whatever the scores, since the kept pages other than the
last are always full); kmin + kmax of every page for the selection (and, for the one-call step, of the pages
of units whose selection the scores decide: fewer pages kept than there are, more than the two forced ones);
both logit rows for the acceptance.
"""
import numpy as np
import pytest

import bench
import oracle as O
from sparse_attention_decode_page_amd import synth as S


@pytest.mark.parametrize("dtype,D,ps", [("bf16", 128, 16), ("f32", 64, 8), ("bf16", 64, 32)])
def test_algorithmic_bytes_brute_force(dtype, D, ps):
    rng = np.random.default_rng(D + ps)
    B, Hkv = 5, 3
    spec = S.custom_spec("bytes", batch=B, num_q_heads=2 * Hkv, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                         dtype=dtype, lens=("list", [1, ps, ps + 1, 7 * ps - 3, 40 * ps]), budget=("pages", [1] * B))
    lens = np.asarray(spec.lens[1], dtype=np.int64)
    budget = rng.integers(0, 12, size=B)
    cap, rows, vocab = 9, 3, 1000
    elt = 2 if dtype == "bf16" else 4
    got = bench.algorithmic_bytes(spec, lens, budget, cap, rows, vocab)
    sparse = dense = meta = meta_step = 0
    for b in range(B):
        L = int(lens[b])
        P = (L + ps - 1) // ps
        valid = [min(ps, L - p * ps) for p in range(P)]
        for g in range(Hkv):
            keep = O.select_pages(rng.standard_normal(P), min(int(budget[b]), cap))
            sparse += sum(valid[p] for p in keep) * 2 * D * elt
            dense += L * 2 * D * elt
            meta += P * 2 * D * elt
            if 2 < len(keep) < P:
                meta_step += P * 2 * D * elt
    assert got["sparse_decode"] == sparse
    assert got["dense_decode"] == dense
    assert got["select_pages"] == meta
    assert got["sparse_path"] == sparse + meta_step
    assert got["acceptance"] == 2 * rows * vocab * 4
    assert got["append_kv"] == B * Hkv * (2 * D * elt + 2 * 2 * D * elt)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asking for more exits with status 2 and says why (before touching any GPU)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_counter_summaries_parse_and_match_patterns(tmp_path, monkeypatch):
    """The bench reads a counter summary only while its source hash is current, and a call's kernels are found
    by name pattern, each pattern matching exactly one kernel."""
    text = "\n".join([
        "# header", "```",
        f"source_hash {bench.kernel_source_hash()}",
        "traffic_bytes decode_stream_kernel<128,4,true> 1000",
        "traffic_bytes stream_merge_kernel<128,64,4,true> 20",
        "traffic_bytes stream_merge_kernel<128,64,4,false> 30",
        "traffic_bytes decode_stream_kernel<128,4,false>@suffix 7",
        "```", ""])
    (tmp_path / "traffic_counters_w.md").write_text(text)
    (tmp_path / "traffic_counters_stale.md").write_text(text.replace(bench.kernel_source_hash(), "0" * 16))
    monkeypatch.setattr(bench, "traffic_file", lambda w: str(tmp_path / f"traffic_counters_{w}.md"))
    t = bench.counter_traffic("w")
    assert t["decode_stream_kernel<128,4,false>@suffix"] == 7
    assert bench.traffic_sum(t, ["decode_stream_kernel<128,4,true>", "stream_merge_kernel<128,*,true>"]) == 1020
    assert bench.traffic_sum(t, ["stream_merge_kernel<128,*>"]) is None          # two kernels match
    assert bench.traffic_sum(t, ["score_stream_kernel<*>"]) is None              # none matches
    assert bench.traffic_sum(t, ["decode_stream_kernel<128,4,false>"]) is None   # the suffix pass is apart
    assert bench.counter_traffic("stale") is None
    assert bench.counter_traffic("missing") is None
    spec = S.SPECS["qwen3-1.7b-L16k"]
    ck = bench.call_kernels(spec)
    assert ck["sparse_decode"] == ["decode_stream_kernel<128,2,true>", "stream_merge_kernel<128,*,true>"]
    assert ck["sparse_path"] == ["sparse_path_kernel<128,2>"]
    assert bench.call_kernels(spec, "two calls")["sparse_path"] == ck["select_pages"] + ck["sparse_decode"]
    assert bench.call_kernels(spec, "sliced")["sparse_path"][0] == "slice_score_kernel<128,2>"
    assert ck["select_pages"] == ["score_stream_kernel<BF16,128,2>", "select_topk_reg_kernel<*>"]
    assert bench.call_kernels(spec, "one kernel", "one kernel")["select_pages"] == ["select_path_kernel<128,2>"]
    assert bench.call_kernels(spec, "sliced", "sliced")["select_pages"] == [
        "slice_score_kernel<128,2>", "slice_select_kernel<128,2,false>"]
    assert bench.call_kernels(spec, "two calls", "one kernel")["sparse_path"][0] == "select_path_kernel<128,2>"
    assert bench.call_kernels(S.custom_spec("g8", num_q_heads=64, num_kv_heads=8, head_dim=128))[
        "dense_decode"][0] == "decode_stream_g8_kernel<128,false>"
