"""GPU: the gather-read ceiling probe (libspdec_probe.so, which bench.py times beside the kernels) reads exactly
the blocks it is given, each once, from one or two bases: the XOR of its per-wave words equals the XOR of those
blocks' 32-bit words computed on the host, for every block size and for lists that are ragged against the
64-entry windows and the per-wave ranges."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    from sparse_attention_decode_page_amd import build as B
    if not os.path.exists(B.PROBE_LIB_PATH):
        B.build()
    L = ctypes.CDLL(B.PROBE_LIB_PATH)
    L.spdec_probe_gather.restype = ctypes.c_int
    L.spdec_probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    L.spdec_probe_sink_words.restype = ctypes.c_int
    assert torch.cuda.is_available()
    return L


def _xor_words(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(a.view(np.uint32).ravel())) if a.size else 0


@pytest.mark.parametrize("block_bytes,nblocks,two", [(512, 1, False), (512, 3001, True), (4096, 65, False),
                                                      (4096, 20000, True), (16384, 777, True), (2048, 128, False)])
def test_probe_reads_each_listed_block_once(P, block_bytes, nblocks, two):
    print(f"case probe block {block_bytes} B x {nblocks}, two bases {two}", flush=True)
    r = np.random.default_rng(block_bytes + nblocks)
    pool_blocks = nblocks * 2 + 5
    words = block_bytes // 4
    a = r.integers(0, 2 ** 32, size=(pool_blocks, words), dtype=np.uint32)
    b = r.integers(0, 2 ** 32, size=(pool_blocks, words), dtype=np.uint32)
    pick = r.choice(pool_blocks, nblocks, replace=False)
    ta = torch.from_numpy(a.view(np.int32)).cuda()
    tb = torch.from_numpy(b.view(np.int32)).cuda()
    off = torch.from_numpy(pick.astype(np.int64) * block_bytes).cuda()
    sink = torch.zeros(P.spdec_probe_sink_words(), dtype=torch.int32, device="cuda")
    rc = P.spdec_probe_gather(ta.data_ptr(), tb.data_ptr() if two else None, off.data_ptr(), nblocks, block_bytes,
                              sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = _xor_words(sink.cpu().numpy())
    want = _xor_words(a[pick]) ^ (_xor_words(b[pick]) if two else 0)
    assert got == want
