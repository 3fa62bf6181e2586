"""GPU parity of the dense verification pass (causal multi-query decode).

Every (sequence, KV head) of small and edge-case shapes, sampled units of a
Qwen3-8B-shaped batch at k = 6 (T = 7 verified positions), all compared with
the fp64 oracle: out within 1e-2 max-abs (bf16 KV), lse within 1e-2.
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


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(spdec.LIB_PATH):
        from sparse_attention_decode_page_amd import build
        build.build()
    spdec.lib()
    assert torch.cuda.is_available()


def _queries(spec, T, seed):
    r = np.random.default_rng(seed)
    q32 = r.standard_normal((spec.batch, T, spec.num_q_heads, spec.head_dim), dtype=np.float32)
    return S.f32_to_bf16_bits(q32)


def _check(wl, T, units, seed=0):
    spec = wl.spec
    print(f"verify {spec.name}: T={T} G={spec.group} D={spec.head_dim} ps={spec.page_size}", flush=True)
    dw = GS.DeviceWorkload(wl)
    qh = _queries(spec, T, seed)
    q = GS.to_device_storage(qh, "bf16")
    out, lse = spdec.verify_decode(dw.cache, q)
    torch.cuda.synchronize()
    out_h, lse_h = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(out_h)) and np.all(np.isfinite(lse_h))
    G = spec.group
    scale = 1.0 / math.sqrt(spec.head_dim)
    worst = [0.0, 0.0]
    for (b, g) in units:
        K, V = GS.unit_kv_f64(wl, b, g)
        qr = O.decode_bf16(qh[b, :, g * G:(g + 1) * G])
        o, l = O.verify_decode_unit(qr, K, V, scale)
        e = np.abs(out_h[b, :, g * G:(g + 1) * G] - o).max()
        el = np.abs(lse_h[b, :, g * G:(g + 1) * G] - l).max()
        worst = [max(worst[0], e), max(worst[1], el)]
        assert e <= TOL and el <= TOL, (b, g, e, el)
    print(f"  {len(units)} units, worst out {worst[0]:.2e} lse {worst[1]:.2e}", flush=True)
    return out, lse, dw, q


CASES = [
    # (batch, Hq, Hkv, D, ps, lens, T)
    (3, 8, 2, 128, 16, ("uniform", 300, 1500), 7),    # Qwen3-8B-like group 4: 28 rows
    (2, 4, 2, 64, 8, ("uniform", 40, 333), 3),        # page size 8, group 2
    (2, 16, 2, 128, 32, ("uniform", 500, 900), 4),    # group 8: 32 rows
    (2, 2, 2, 128, 64, ("uniform", 70, 700), 1),      # one row per unit
    (2, 4, 2, 64, 16, ("uniform", 200, 260), 16),     # 16 positions, group 2
    (4, 8, 2, 128, 16, ("fixed", 7), 7),              # the cache holds only the verified tokens
    (3, 8, 2, 128, 16, ("uniform", 17, 40), 7),       # shorter than two pages
    (2, 16, 2, 128, 16, ("uniform", 300, 1800), 7),   # group 8 at k = 6: 56 rows, two 32-row passes
    (2, 8, 2, 64, 8, ("uniform", 100, 700), 16),      # group 4, 16 positions: 64 rows
    (3, 16, 2, 128, 32, ("uniform", 40, 1200), 5),    # group 8: 40 rows (second pass 8 rows)
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_verify_small_all_units(case):
    B, Hq, Hkv, D, ps, lens, T = CASES[case]
    spec = S.custom_spec(f"verify{case}", batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                         dtype="bf16", lens=lens, budget=("tokens", 64), outlier_channels=2)
    wl = S.make_workload(spec, seed=case)
    _check(wl, T, [(b, g) for b in range(B) for g in range(Hkv)], seed=case)


@pytest.mark.parametrize("seed", range(8))
def test_verify_random_shapes(seed):
    """Seeded random shapes: group, positions (G * T up to 64), head dim, page size, ragged lengths."""
    r = np.random.default_rng(2000 + seed)
    G = int(r.choice([1, 2, 4, 8]))
    T = int(r.integers(1, min(16, 64 // G) + 1))
    Hkv = int(r.choice([1, 2]))
    D = int(r.choice([64, 128]))
    ps = int(r.choice([8, 16, 32, 64]))
    B = int(r.integers(1, 4))
    spec = S.custom_spec(f"verify-rand{seed}", batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                         page_size=ps, dtype="bf16", lens=("uniform", T, 40 * ps), budget=("tokens", 64),
                         outlier_channels=2)
    wl = S.make_workload(spec, seed=seed)
    _check(wl, T, [(b, g) for b in range(B) for g in range(Hkv)], seed=seed)


def test_verify_one_position_matches_dense_decode():
    spec = S.custom_spec("verify-dense", batch=3, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                         dtype="bf16", lens=("uniform", 100, 2000), budget=("tokens", 64))
    wl = S.make_workload(spec, seed=9)
    out, lse, dw, q = _check(wl, 1, [(b, g) for b in range(3) for g in range(2)], seed=9)
    od, ld = spdec.dense_decode(dw.cache, q[:, 0].contiguous())
    torch.cuda.synchronize()
    # each weight enters P.V with its whole significand: the same attention up to summation order
    assert (out[:, 0] - od).abs().max().item() < 1e-5
    assert (lse[:, 0] - ld).abs().max().item() < 1e-5


@pytest.mark.parametrize("G,T", [(4, 7), (8, 7), (2, 16)])
def test_verify_every_position_matches_dense_decode(G, T):
    """Position t of T attends to the cache up to L - T + t: the dense decode of a cache cut to that length with
    query t gives the same output and lse within 1e-5 (S3R page, abstract: the verifier is the dense policy)."""
    spec = S.custom_spec(f"verify-dense-{G}-{T}", batch=3, num_q_heads=2 * G, num_kv_heads=2, head_dim=128,
                         page_size=16, dtype="bf16", lens=("uniform", 200, 3000), budget=("tokens", 64))
    wl = S.make_workload(spec, seed=11 + G)
    dw = GS.DeviceWorkload(wl)
    q = GS.to_device_storage(_queries(spec, T, 11 + G), "bf16")
    out, lse = spdec.verify_decode(dw.cache, q)
    full = dw.seq_lens.clone()
    worst = 0.0
    for t in range(T):
        dw.seq_lens.copy_(full - (T - 1 - t))
        od, ld = spdec.dense_decode(dw.cache, q[:, t].contiguous())
        torch.cuda.synchronize()
        worst = max(worst, (out[:, t] - od).abs().max().item(), (lse[:, t] - ld).abs().max().item())
    dw.seq_lens.copy_(full)
    print(f"  G={G} T={T}: worst |verify - dense| {worst:.2e}", flush=True)
    assert worst < 1e-5


def test_verify_is_deterministic():
    spec = S.custom_spec("verify-det", batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                         dtype="bf16", lens=("uniform", 1000, 3000), budget=("tokens", 64))
    wl = S.make_workload(spec, seed=4)
    dw = GS.DeviceWorkload(wl)
    q = GS.to_device_storage(_queries(spec, 7, 4), "bf16")
    o1, l1 = spdec.verify_decode(dw.cache, q)
    o2, l2 = spdec.verify_decode(dw.cache, q)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)



def test_verify_reused_workspace_across_position_counts():
    """One workspace across verification calls of 7, 1, 16 and 7 positions (different row counts and chunk
    layouts): each equals the same call on a fresh workspace bit for bit."""
    spec = S.custom_spec("verify-reuse", batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                         dtype="bf16", lens=("list", [3000, 40, 1200, 700]), budget=("tokens", 64))
    wl = S.make_workload(spec, seed=15)
    dw = GS.DeviceWorkload(wl)
    nbytes = max(spdec.verify_workspace_bytes(dw.cache, T) for T in (1, 7, 16))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for k, T in enumerate((7, 1, 16, 7)):
        q = GS.to_device_storage(_queries(spec, T, 20 + k), "bf16")
        o1, l1 = spdec.verify_decode(dw.cache, q, workspace=ws)
        o2, l2 = spdec.verify_decode(dw.cache, q)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), T

def test_verify_rejects_unsupported():
    spec = S.custom_spec("verify-f32", batch=1, num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                         dtype="f32", lens=("fixed", 64), budget=("tokens", 64))
    dw = GS.DeviceWorkload(S.make_workload(spec, seed=0))
    q = torch.zeros((1, 2, 4, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError):
        spdec.verify_decode(dw.cache, q)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_verify_qwen3_8b_ragged_sampled():
    wl = S.make_workload("qwen3-8b-ragged", seed=0)
    _check(wl, 7, GS.sample_units(wl, 8, seed=3), seed=11)
