"""GPU parity of the shared-prefix dense decode (spdec_dense_decode_shared).

Groups of N consecutive sequences share their prompt pages; the result must
be the dense decode of every sequence: within 1e-2 max-abs of the fp64 oracle
(bf16 KV) on every unit, and close to the per-sequence dense decode.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_decode_page_amd import spdec
from sparse_attention_decode_page_amd import synth as S

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gpu_support as GS  # noqa: E402

pytestmark = pytest.mark.gpu
TOL = 1e-2
SAME = 1e-5  # against the per-sequence dense decode


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(spdec.LIB_PATH):
        from sparse_attention_decode_page_amd import build
        build.build()
    spdec.lib()
    assert torch.cuda.is_available()


def _check(wl, shared, N, units):
    spec = wl.spec
    print(f"shared {spec.name}: N={N} G={spec.group} D={spec.head_dim} ps={spec.page_size} "
          f"shared pages {shared.tolist()[:4]}", flush=True)
    dw = GS.DeviceWorkload(wl)
    sh = torch.from_numpy(shared.astype(np.int32)).cuda()
    pre = spdec.check_inputs(dw.cache, q=dw.q, group_size=N, shared_pages=sh)  # the documented preconditions hold
    assert pre["first_bad_sequence"] == spec.batch, pre
    out, lse = spdec.dense_decode_shared(dw.cache, dw.q, N, sh)
    od, ld = spdec.dense_decode(dw.cache, dw.q)
    torch.cuda.synchronize()
    out_h, lse_h = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(out_h)) and np.all(np.isfinite(lse_h))
    # the prefix pass feeds P.V each weight's whole significand: the per-sequence decode up to summation order
    assert (out - od).abs().max().item() < SAME and (lse - ld).abs().max().item() < SAME
    G = spec.group
    scale = 1.0 / math.sqrt(spec.head_dim)
    worst = [0.0, 0.0]
    for (b, g) in units:
        K, V = GS.unit_kv_f64(wl, b, g)
        o, l = O.dense_decode_unit(GS.q_group_f64(wl, b, g), K, V, spec.page_size, scale)
        e = np.abs(out_h[b, g * G:(g + 1) * G] - o).max()
        el = np.abs(lse_h[b, g * G:(g + 1) * G] - l).max()
        worst = [max(worst[0], e), max(worst[1], el)]
        assert e <= TOL and el <= TOL, (b, g, e, el)
    print(f"  {len(units)} units, worst out {worst[0]:.2e} lse {worst[1]:.2e}", flush=True)
    return out, lse, dw, sh


CASES = [
    # (batch, Hq, Hkv, D, ps, gen lens, N, prompt tokens)
    (8, 8, 2, 128, 16, ("uniform", 10, 300), 4, 200),     # prompt ends mid-page
    (6, 4, 2, 64, 8, ("uniform", 1, 90), 3, 96),          # page size 8, prompt on a page boundary
    (8, 16, 2, 128, 32, ("uniform", 40, 400), 4, 500),    # group 8: 32 rows per group unit
    (4, 4, 4, 128, 64, ("uniform", 5, 200), 2, 700),      # one query head per KV head
    (4, 8, 2, 128, 16, ("uniform", 50, 60), 1, 320),      # groups of one
    (16, 16, 2, 128, 16, ("uniform", 20, 300), 8, 600),   # group 8 x 8 samples: 64 rows, two 32-row passes
    (12, 8, 2, 64, 8, ("uniform", 1, 120), 12, 250),      # 12 samples x group 4: 48 rows (second pass 16)
    (6, 4, 2, 64, 8, ("list", [0, 0, 0, 0, 5, 1]), 3, 96),  # members holding only the prompt (no own page)
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_shared_prefix_all_units(case):
    B, Hq, Hkv, D, ps, gen, N, prompt = CASES[case]
    spec = S.custom_spec(f"shared{case}", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                         dtype="bf16", lens=gen, budget=("tokens", 64), outlier_channels=2,
                         prompt=("shared", N, prompt))
    wl = S.make_workload(spec, seed=case)
    _check(wl, wl.shared_pages, N, [(b, g) for b in range(B) for g in range(Hkv)])


@pytest.mark.parametrize("seed", range(6))
def test_shared_prefix_random_shapes(seed):
    """Seeded random groups: samples per group, group size (N * G up to 64), page size, prompt length."""
    r = np.random.default_rng(3000 + seed)
    G = int(r.choice([1, 2, 4, 8]))
    N = int(r.integers(1, min(12, 64 // G) + 1))
    groups = int(r.integers(1, 3))
    D = int(r.choice([64, 128]))
    ps = int(r.choice([8, 16, 32, 64]))
    prompt = int(r.integers(1, 30 * ps))
    spec = S.custom_spec(f"shared-rand{seed}", batch=N * groups, num_q_heads=2 * G, num_kv_heads=2, head_dim=D,
                         page_size=ps, dtype="bf16", lens=("uniform", 1, 10 * ps), budget=("tokens", 64),
                         outlier_channels=2, prompt=("shared", N, prompt))
    wl = S.make_workload(spec, seed=seed)
    _check(wl, wl.shared_pages, N, [(b, g) for b in range(N * groups) for g in range(2)])


def test_fewer_shared_pages_than_possible_and_none():
    spec = S.custom_spec("shared-partial", batch=8, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                         dtype="bf16", lens=("uniform", 30, 200), budget=("tokens", 64), prompt=("shared", 4, 400))
    wl = S.make_workload(spec, seed=11)
    units = [(b, g) for b in range(8) for g in range(2)]
    # any count up to the truly shared pages is a valid split, including none
    _check(wl, np.array([7, 0], dtype=np.int32), 4, units)
    _check(wl, np.zeros(2, dtype=np.int32), 4, units)


def test_shared_prefix_is_deterministic():
    spec = S.custom_spec("shared-det", batch=8, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                         dtype="bf16", lens=("uniform", 100, 900), budget=("tokens", 64), prompt=("shared", 4, 3000))
    wl = S.make_workload(spec, seed=12)
    dw = GS.DeviceWorkload(wl)
    sh = torch.from_numpy(wl.shared_pages).cuda()
    a = spdec.dense_decode_shared(dw.cache, dw.q, 4, sh)
    b = spdec.dense_decode_shared(dw.cache, dw.q, 4, sh)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])



def test_reused_workspace_after_members_lose_their_own_pages():
    """One workspace across calls: first nothing shared (every member's pages go through the per-sample pass),
    then the whole prompt shared, so members holding only the prompt have no per-sample chunk at all. The second
    call must equal the same call on a fresh workspace bit for bit (no count or partial left from the first)."""
    spec = S.custom_spec("shared-reuse", batch=6, num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=8,
                         dtype="bf16", lens=("list", [0, 0, 0, 0, 5, 1]), budget=("tokens", 64),
                         outlier_channels=2, prompt=("shared", 3, 96))
    wl = S.make_workload(spec, seed=13)
    dw = GS.DeviceWorkload(wl)
    ws = torch.zeros(spdec.shared_workspace_bytes(dw.cache, 3), dtype=torch.uint8, device="cuda")
    none = torch.zeros(2, dtype=torch.int32, device="cuda")
    full = torch.from_numpy(wl.shared_pages.astype(np.int32)).cuda()
    spdec.dense_decode_shared(dw.cache, dw.q, 3, none, workspace=ws)
    o1, l1 = spdec.dense_decode_shared(dw.cache, dw.q, 3, full, workspace=ws)
    o2, l2 = spdec.dense_decode_shared(dw.cache, dw.q, 3, full)
    o3, l3 = spdec.dense_decode_shared(dw.cache, dw.q, 3, none, workspace=ws)
    o4, l4 = spdec.dense_decode_shared(dw.cache, dw.q, 3, none)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
    od, ld = spdec.dense_decode(dw.cache, dw.q)
    torch.cuda.synchronize()
    assert (o1 - od).abs().max().item() < SAME and (l1 - ld).abs().max().item() < SAME

@pytest.mark.slow
@pytest.mark.timeout(600)
def test_shared_prefix_qwen3_8b_grouped_sampled():
    wl = S.make_workload("qwen3-8b-grouped", seed=0)
    _check(wl, wl.shared_pages, wl.spec.prompt[1], GS.sample_units(wl, 8, seed=5))
