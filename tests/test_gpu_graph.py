"""HIP graph capture of the decode step.

Every ABI call is stream-ordered, allocates nothing and never synchronises the
host, so a whole step (append_kv -> select_pages -> sparse_decode ->
dense_decode -> acceptance) captured once into a graph must replay to the same
bits as the same step run eagerly, step after step (the decode path is
replayed from graphs on the S3R page, Table 3). Each replay is checked against
an eager twin of the cache, with eager work and host synchronisations between
the replays.
"""
import os
import sys

import numpy as np
import pytest
import torch

from sparse_attention_decode_page_amd import spdec
from sparse_attention_decode_page_amd import synth as S

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gpu_support as GS  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(spdec.LIB_PATH):
        from sparse_attention_decode_page_amd import build
        build.build()
    spdec.lib()
    assert torch.cuda.is_available()


class _Step:
    """Preallocated outputs and workspaces for one cache, and the step itself."""

    def __init__(self, dw, la, lb, temperature):
        c, dev = dw.cache, dw.q.device
        spec = dw.wl.spec
        self.dw, self.la, self.lb, self.t = dw, la, lb, temperature
        cap = dw.max_budget
        self.sel_idx = torch.zeros((spec.batch, spec.num_kv_heads, cap), dtype=torch.int32, device=dev)
        self.sel_cnt = torch.zeros((spec.batch, spec.num_kv_heads), dtype=torch.int32, device=dev)
        self.ws_sel = torch.zeros(spdec.select_workspace_bytes(c, cap), dtype=torch.uint8, device=dev)
        self.ws_sp = torch.zeros(spdec.decode_workspace_bytes(c, cap), dtype=torch.uint8, device=dev)
        self.ws_de = torch.zeros(spdec.decode_workspace_bytes(c, 0), dtype=torch.uint8, device=dev)
        self.ws_acc = torch.zeros(spdec.acceptance_workspace_bytes(*la.shape), dtype=torch.uint8, device=dev)
        shape = (spec.batch, spec.num_q_heads, spec.head_dim)
        self.o_s = torch.empty(shape, dtype=torch.float32, device=dev)
        self.o_d = torch.empty(shape, dtype=torch.float32, device=dev)
        self.l_s = torch.empty(shape[:2], dtype=torch.float32, device=dev)
        self.l_d = torch.empty(shape[:2], dtype=torch.float32, device=dev)
        self.alpha = torch.empty(la.shape[0], dtype=torch.float32, device=dev)

    def run(self, k_new, v_new):
        dw, c = self.dw, self.dw.cache
        spdec.append_kv(c, k_new, v_new)
        spdec.select_pages(c, dw.q, dw.budget, dw.max_budget, sel_idx=self.sel_idx, sel_cnt=self.sel_cnt,
                           workspace=self.ws_sel)
        spdec.sparse_decode(c, dw.q, self.sel_idx, self.sel_cnt, dw.max_budget, out=self.o_s, lse=self.l_s,
                            workspace=self.ws_sp)
        spdec.dense_decode(c, dw.q, out=self.o_d, lse=self.l_d, workspace=self.ws_de)
        spdec.acceptance(self.la, self.lb, self.t, alpha=self.alpha, workspace=self.ws_acc)

    def snapshot(self):
        dw = self.dw
        return {n: t.clone() for n, t in (("seq_lens", dw.seq_lens), ("kminmax", dw.kminmax),
                                            ("k_pool", dw.k_pool), ("v_pool", dw.v_pool),
                                            ("sel_idx", self.sel_idx), ("sel_cnt", self.sel_cnt),
                                            ("o_s", self.o_s), ("l_s", self.l_s), ("o_d", self.o_d),
                                            ("l_d", self.l_d), ("alpha", self.alpha))}


@pytest.mark.parametrize("dtype,D,ps", [("bf16", 128, 16), ("f32", 64, 8)])
def test_graph_replay_matches_eager(dtype, D, ps):
    steps = 5
    spec = S.custom_spec("graph", batch=5, num_q_heads=8, num_kv_heads=2, head_dim=D, page_size=ps, dtype=dtype,
                         lens=("uniform", 200, 1500), budget=("tokens", 256), outlier_channels=2,
                         logits=("noisy", 3, 5003, 3.0, 0.3, 0.34, 3.0))
    wl = S.make_workload(spec, seed=3, headroom=steps + 1)
    print(f"graph replay: {dtype} D={D} ps={ps}", flush=True)
    la = torch.from_numpy(wl.logits_a).cuda()
    lb = torch.from_numpy(wl.logits_b).cuda()
    eager = _Step(GS.DeviceWorkload(wl), la, lb, spec.temperature)
    graphed = _Step(GS.DeviceWorkload(wl), la, lb, spec.temperature)
    spdec.build_meta(eager.dw.cache)
    spdec.build_meta(graphed.dw.cache)
    tokens = [S.append_tokens(wl, i) for i in range(steps)]
    k_static = GS.to_device_storage(tokens[0][0], dtype)
    v_static = GS.to_device_storage(tokens[0][1], dtype)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run(k_static, v_static)
    torch.cuda.synchronize()

    for i in range(steps):
        k_i = GS.to_device_storage(tokens[i][0], dtype)
        v_i = GS.to_device_storage(tokens[i][1], dtype)
        eager.run(k_i, v_i)
        torch.cuda.synchronize()
        k_static.copy_(k_i)
        v_static.copy_(v_i)
        g.replay()
        torch.cuda.synchronize()
        a, b = eager.snapshot(), graphed.snapshot()
        for name in a:
            assert torch.equal(a[name], b[name]), (i, name)
        # eager work between replays, on the graphed cache's buffers too
        graphed.o_s.fill_(float("nan"))
        graphed.alpha.zero_()
    lens = graphed.dw.seq_lens.cpu().numpy()
    assert np.array_equal(lens, wl.lens + steps)


def test_control_loop_graph_replay_matches_eager():
    """The on-device loop of the next rows: tail statistics -> budget controller -> Top-B and top-p selection ->
    sparse decode, captured once; every replay must equal the same calls run eagerly (state carried in the
    controller's scale on the device between steps, no host round trip)."""
    steps = 4
    spec = S.custom_spec("graph-ctl", batch=6, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                         dtype="bf16", lens=("uniform", 300, 3000), budget=("tokens", 256), outlier_channels=2)
    wl = S.make_workload(spec, seed=8)
    r = np.random.default_rng(8)
    alphas = [torch.from_numpy(np.clip(1 - r.exponential(0.05 + 0.03 * i, 64), 0, 1).astype(np.float32)).cuda()
              for i in range(steps)]
    prm = spdec.BudgetParams(target=0.86, gain=4.0, scale_min=0.05, scale_max=4.0, base_tokens=256.0,
                             tokens_per_token=0.05, page_size=16, max_budget_pages=64)

    class Loop:
        def __init__(self):
            self.dw = GS.DeviceWorkload(wl)
            spdec.build_meta(self.dw.cache)
            c, dev = self.dw.cache, "cuda"
            self.alpha = torch.empty(64, dtype=torch.float32, device=dev)
            self.tail = torch.empty(2, dtype=torch.float32, device=dev)
            self.scale = torch.ones(1, dtype=torch.float32, device=dev)
            self.budget = torch.empty(spec.batch, dtype=torch.int32, device=dev)
            self.si = torch.zeros((spec.batch, spec.num_kv_heads, 64), dtype=torch.int32, device=dev)
            self.sc = torch.zeros((spec.batch, spec.num_kv_heads), dtype=torch.int32, device=dev)
            self.pi = torch.zeros_like(self.si)
            self.pc = torch.zeros_like(self.sc)
            self.ws_sel = torch.zeros(spdec.select_workspace_bytes(c, 64), dtype=torch.uint8, device=dev)
            self.ws_sp = torch.zeros(spdec.decode_workspace_bytes(c, 64), dtype=torch.uint8, device=dev)
            self.o = torch.empty((spec.batch, spec.num_q_heads, spec.head_dim), dtype=torch.float32, device=dev)
            self.lse = torch.empty((spec.batch, spec.num_q_heads), dtype=torch.float32, device=dev)

        def run(self):
            c, q = self.dw.cache, self.dw.q
            spdec.tail_stats(self.alpha, out=self.tail)
            spdec.budget_update(self.tail, self.scale, self.dw.seq_lens, prm, budget_pages=self.budget)
            spdec.select_pages(c, q, self.budget, 64, sel_idx=self.si, sel_cnt=self.sc, workspace=self.ws_sel)
            spdec.select_pages_top_p(c, q, 0.9, 64, budget_pages=self.budget, sel_idx=self.pi, sel_cnt=self.pc,
                                     workspace=self.ws_sel)
            spdec.sparse_decode(c, q, self.pi, self.pc, 64, out=self.o, lse=self.lse, workspace=self.ws_sp)

        def snapshot(self):
            return {n: t.clone() for n, t in (("tail", self.tail), ("scale", self.scale), ("budget", self.budget),
                                                ("si", self.si), ("sc", self.sc), ("pi", self.pi), ("pc", self.pc),
                                                ("o", self.o), ("lse", self.lse))}

    eager, graphed = Loop(), Loop()
    graphed.alpha.copy_(alphas[0])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run()
    torch.cuda.synchronize()
    for i in range(steps):
        eager.alpha.copy_(alphas[i])
        eager.run()
        torch.cuda.synchronize()
        graphed.alpha.copy_(alphas[i])
        g.replay()
        torch.cuda.synchronize()
        a, b = eager.snapshot(), graphed.snapshot()
        for name in a:
            assert torch.equal(a[name], b[name]), (i, name)
        graphed.o.fill_(float("nan"))
    assert float(graphed.scale.item()) != 1.0      # the controller moved the schedule


def test_side_streams_and_concurrent_calls_match_the_default_stream():
    """Calls follow torch's current stream: the path run on two side streams at once (two caches, separate
    workspaces) gives bitwise the results of the same calls run one after the other on the default stream."""
    wls = []
    for i, (B, Hq, Hkv, lens) in enumerate(((6, 32, 8, ("uniform", 3000, 9000)), (4, 16, 8, ("uniform", 2000, 6000)))):
        spec = S.custom_spec(f"streams{i}", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128, page_size=16,
                             dtype="bf16", lens=lens, budget=("tokens", 1024), outlier_channels=4)
        wls.append(GS.DeviceWorkload(S.make_workload(spec, seed=70 + i)))

    def run(dw):
        c = dw.cache
        spdec.build_meta(c)
        idx, cnt = spdec.select_pages(c, dw.q, dw.budget, dw.max_budget)
        o_s, l_s = spdec.sparse_decode(c, dw.q, idx, cnt, dw.max_budget)
        o_d, l_d = spdec.dense_decode(c, dw.q)
        return [idx, cnt, o_s, l_s, o_d, l_d]

    ref = [run(dw) for dw in wls]
    torch.cuda.synchronize()
    ref = [[t.clone() for t in r] for r in ref]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for s, dw in zip(streams, wls):
        with torch.cuda.stream(s):
            outs.append(run(dw))
    torch.cuda.synchronize()
    for r, o in zip(ref, outs):
        for a, b in zip(r, o):
            assert torch.equal(a, b)


def test_one_kernel_step_graph_replay_matches_eager():
    """append_kv -> sparse_path on a batch that takes the one-kernel form (32 sequences x 8 KV heads), captured
    once: every replay equals the eager step bit for bit (selection, scores, outputs)."""
    steps = 4
    spec = S.custom_spec("graph-path", batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                         dtype="bf16", lens=("uniform", 200, 3000), budget=("pages", [24] * 32), outlier_channels=2)
    wl = S.make_workload(spec, seed=6, headroom=steps + 1)
    print("graph replay: one-kernel sparse step", flush=True)

    class Step:
        def __init__(self):
            self.dw = GS.DeviceWorkload(wl)
            spdec.build_meta(self.dw.cache)
            c, dev = self.dw.cache, "cuda"
            self.si = torch.zeros((spec.batch, spec.num_kv_heads, 24), dtype=torch.int32, device=dev)
            self.sc = torch.zeros((spec.batch, spec.num_kv_heads), dtype=torch.int32, device=dev)
            self.scores = torch.zeros((spec.batch, spec.num_kv_heads, c.max_pages), dtype=torch.float32, device=dev)
            self.ws = torch.zeros(spdec.sparse_path_workspace_bytes(c, 24), dtype=torch.uint8, device=dev)
            self.o = torch.empty((spec.batch, spec.num_q_heads, spec.head_dim), dtype=torch.float32, device=dev)
            self.lse = torch.empty((spec.batch, spec.num_q_heads), dtype=torch.float32, device=dev)

        def run(self, k_new, v_new):
            c = self.dw.cache
            spdec.append_kv(c, k_new, v_new)
            spdec.sparse_path(c, self.dw.q, self.dw.budget, 24, sel_idx=self.si, sel_cnt=self.sc,
                              scores_out=self.scores, out=self.o, lse=self.lse, workspace=self.ws)

        def snapshot(self):
            return {n: t.clone() for n, t in (("si", self.si), ("sc", self.sc), ("scores", self.scores),
                                                ("o", self.o), ("lse", self.lse), ("lens", self.dw.seq_lens))}

    eager, graphed = Step(), Step()
    assert spdec.sparse_path_form(graphed.dw.cache, 24) == ("one kernel" if spec.batch * spec.num_kv_heads >= (
        torch.cuda.get_device_properties(0).multi_processor_count) else "two calls")
    tokens = [S.append_tokens(wl, i) for i in range(steps)]
    k_static = GS.to_device_storage(tokens[0][0], "bf16")
    v_static = GS.to_device_storage(tokens[0][1], "bf16")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run(k_static, v_static)
    torch.cuda.synchronize()
    for i in range(steps):
        k_i = GS.to_device_storage(tokens[i][0], "bf16")
        v_i = GS.to_device_storage(tokens[i][1], "bf16")
        eager.run(k_i, v_i)
        torch.cuda.synchronize()
        k_static.copy_(k_i)
        v_static.copy_(v_i)
        g.replay()
        torch.cuda.synchronize()
        a, b = eager.snapshot(), graphed.snapshot()
        for name in a:
            assert torch.equal(a[name].view(torch.int32) if a[name].dtype == torch.float32 else a[name],
                               b[name].view(torch.int32) if b[name].dtype == torch.float32 else b[name]), (i, name)
        graphed.o.fill_(float("nan"))
