"""GPU: both forms of the acceptance kernel against the oracle, and the single-read form's cross-workgroup
exchange (bounded wait, its fallback, the sync region left zero).

Bar: alpha within 1e-5 of the fp64 oracle (Sparrow project page, "Insights": per-token mismatch against the
dense model; the wispaper blog's "acceptance rate").
"""
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

SYNC_BYTES = 96 * 1024


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(spdec.LIB_PATH):
        from sparse_attention_decode_page_amd import build
        build.build()
    spdec.lib()
    assert torch.cuda.is_available()


def _logits(R, V, seed, noise=0.3):
    r = np.random.default_rng(seed)
    a = r.normal(0, 3, (R, V)).astype(np.float32)
    b = (a + r.normal(0, noise, (R, V))).astype(np.float32)
    return a, b


def _oracle(a, b, T):
    return np.array([O.acceptance(a[i], b[i], T) for i in range(a.shape[0])])


def _sync_clear(ws):
    return int(torch.count_nonzero(ws[:SYNC_BYTES]).item()) == 0


def test_single_read_full_size_no_fallback():
    """64 rows of 151936 (the acceptance workload): one read, nobody stops waiting, both forms match the oracle
    and each other within the bar, the sync region is zero afterwards."""
    say("case acceptance single read 64 x 151936")
    spec = S.SPECS["qwen3-8b-L32k-acceptance"]
    a, b, heavy = S.make_logits(spec, 0)
    want = _oracle(a, b, spec.temperature)
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    ws = torch.zeros(spdec.acceptance_workspace_bytes(*a.shape), dtype=torch.uint8, device="cuda")
    fb = torch.zeros(1, dtype=torch.int32, device="cuda")
    one, path1 = spdec.acceptance_ex(ta, tb, spec.temperature, workspace=ws, force_path=1, fallbacks=fb)
    two, path2 = spdec.acceptance_ex(ta, tb, spec.temperature, workspace=ws, force_path=2)
    auto, path0 = spdec.acceptance_ex(ta, tb, spec.temperature, workspace=ws)
    torch.cuda.synchronize()
    assert (path1, path2, path0) == (1, 2, 1)
    assert int(fb.item()) == 0
    e1 = np.abs(one.cpu().numpy() - want).max()
    e2 = np.abs(two.cpu().numpy() - want).max()
    say(f"  max |alpha - oracle|: single read {e1:.2e}, two passes {e2:.2e}")
    assert e1 <= GS.TOL_ALPHA and e2 <= GS.TOL_ALPHA
    assert torch.equal(one, auto)
    assert _sync_clear(ws)
    assert np.all(one.cpu().numpy()[heavy] < np.delete(one.cpu().numpy(), heavy).min())


@pytest.mark.parametrize("R,V", [(64, 151936), (5, 30001), (1, 4), (3, 10240), (2, 10244)])
def test_fallback_gives_identical_bits(R, V):
    """A wait limit of 0 makes every chunk that does not find its row complete at its first poll read the row
    itself: alpha is bitwise the default single read's."""
    say(f"case acceptance fallback R={R} V={V}")
    a, b = _logits(R, V, seed=R * 7 + V)
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    ws = torch.zeros(spdec.acceptance_workspace_bytes(R, V), dtype=torch.uint8, device="cuda")
    fb = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref, p = spdec.acceptance_ex(ta, tb, 1.0, workspace=ws, force_path=1)
    got, q = spdec.acceptance_ex(ta, tb, 1.0, workspace=ws, force_path=1, spin_limit=0, fallbacks=fb)
    torch.cuda.synchronize()
    assert p == q == 1
    nchunk = -(-V // 10240)
    say(f"  fallbacks {int(fb.item())} of {R * nchunk} chunks")
    if R * nchunk >= 10:  # many equal chunks: some finish their first poll before the others publish
        assert int(fb.item()) > 0
    assert torch.equal(ref, got)
    assert _sync_clear(ws)
    assert np.abs(got.cpu().numpy() - _oracle(a, b, 1.0)).max() <= GS.TOL_ALPHA


def test_two_passes_when_chunks_exceed_the_device():
    """More chunks than resident workgroups: the automatic form is two passes, within the bar."""
    say("case acceptance two passes 1500 x 20480")
    R, V = 1500, 20480
    a, b = _logits(R, V, seed=5)
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    got, path = spdec.acceptance_ex(ta, tb, 0.8)
    torch.cuda.synchronize()
    assert path == 2
    rows = np.random.default_rng(6).choice(R, 48, replace=False)
    err = np.abs(got.cpu().numpy()[rows] - _oracle(a[rows], b[rows], 0.8)).max()
    assert err <= GS.TOL_ALPHA, err
    with pytest.raises(RuntimeError):
        spdec.acceptance_ex(ta, tb, 0.8, force_path=1)


def test_reused_workspace_across_forms_and_shapes():
    """One workspace through single-read and two-pass calls of different shapes (the two-pass data lies past
    the sync region): every call equals a fresh workspace bitwise and leaves the sync region zero."""
    say("case acceptance workspace across forms")
    shapes = [(64, 151936, 1.0, -1), (1500, 20480, 1.0, -1), (8, 50000, 0.7, 2), (8, 50000, 0.7, 1),
              (3, 1001, 1.3, -1), (64, 151936, 1.0, 1)]
    nbytes = max(spdec.acceptance_workspace_bytes(R, V) for R, V, _, _ in shapes)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for i, (R, V, T, f) in enumerate(shapes):
        a, b = _logits(R, V, seed=100 + i)
        ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
        x1, p1 = spdec.acceptance_ex(ta, tb, T, workspace=ws, force_path=f)
        x2, p2 = spdec.acceptance_ex(ta, tb, T, force_path=f)
        torch.cuda.synchronize()
        assert p1 == p2
        assert torch.equal(x1, x2), (R, V, T, f)
        assert _sync_clear(ws), (R, V, T, f)


def test_unaligned_rows_and_odd_vocab():
    """Row stride and vocabulary not multiples of 4 (scalar loads), both forms."""
    say("case acceptance unaligned")
    R, V = 6, 30003
    a, b = _logits(R, V, seed=9)
    buf_a = torch.zeros((R, V + 1), dtype=torch.float32, device="cuda")
    buf_b = torch.zeros((R, V + 1), dtype=torch.float32, device="cuda")
    buf_a[:, :V] = torch.from_numpy(a)
    buf_b[:, :V] = torch.from_numpy(b)
    want = _oracle(a, b, 1.7)
    for f in (1, 2):
        got, p = spdec.acceptance_ex(buf_a[:, :V], buf_b[:, :V], 1.7, force_path=f)
        torch.cuda.synchronize()
        assert p == f
        assert np.abs(got.cpu().numpy() - want).max() <= GS.TOL_ALPHA
