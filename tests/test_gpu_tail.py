"""GPU parity of the on-device acceptance tail statistics (mean, lower 5th percentile)."""
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


@pytest.mark.parametrize("n", [1, 2, 3, 19, 20, 21, 64, 1000, 4097, 8192])
def test_tail_stats_match_oracle(n):
    r = np.random.default_rng(n)
    # acceptance-like values: mostly near 1 with a heavy lower tail, plus exact ties
    a = np.clip(1.0 - np.abs(r.standard_normal(n)) * 0.03 - (r.random(n) < 0.05) * r.random(n) * 0.5, 0, 1)
    a = a.astype(np.float32)
    if n > 10:
        a[: n // 10] = a[0]
    out = spdec.tail_stats(torch.from_numpy(a).cuda())
    torch.cuda.synchronize()
    mean, p5 = O.tail_stats(a.astype(np.float64))
    got = out.cpu().numpy().astype(np.float64)
    assert abs(got[0] - mean) <= 1e-7 * max(1.0, abs(mean)), (got[0], mean)
    assert abs(got[1] - p5) <= 1e-7 * max(1.0, abs(p5)), (got[1], p5)


def test_tail_stats_rejects_too_many_rows():
    with pytest.raises(RuntimeError):
        spdec.tail_stats(torch.zeros(8193, dtype=torch.float32, device="cuda"))
