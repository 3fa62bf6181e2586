"""GPU: the allocation-free acceptance entry point (the library's own per-GPU scratch array) against the entry
point with a caller workspace, through the C ABI: two calls in a row, the second on a smaller input, then a
two-pass shape inside the array's limit and a shape beyond it."""
import os

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_decode_page_amd import spdec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(spdec.LIB_PATH):
        from sparse_attention_decode_page_amd import build
        build.build()
    spdec.lib()
    assert torch.cuda.is_available()


def _pair(R, V, seed):
    r = np.random.default_rng(seed)
    a = r.normal(0, 3, (R, V)).astype(np.float32)
    b = (a + r.normal(0, 0.3, (R, V))).astype(np.float32)
    return a, b


@pytest.mark.parametrize("shapes", [[(64, 151936, 1.0), (5, 30001, 0.7)], [(1000, 20480, 1.0), (3, 4096, 1.3)]])
def test_noalloc_equals_workspace_entry_point(shapes):
    print(f"case acceptance no-alloc {shapes}", flush=True)
    for i, (R, V, T) in enumerate(shapes):
        a, b = _pair(R, V, seed=31 + i)
        ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
        want = spdec.acceptance(ta, tb, T)
        got = spdec.acceptance_noalloc(ta, tb, T)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (R, V, T)
        rows = np.arange(min(R, 16))
        err = np.abs(got.cpu().numpy()[rows] - np.array([O.acceptance(a[j], b[j], T) for j in rows])).max()
        assert err <= 1e-5, err


def test_noalloc_refuses_shapes_beyond_its_array():
    ta = torch.zeros((1333, 151936), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError):
        spdec.acceptance_noalloc(ta, ta, 1.0)
