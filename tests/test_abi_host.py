"""The C ABI library loads, exports every declared symbol and rejects bad
arguments before launching anything (CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest

from sparse_attention_decode_page_amd import spdec as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# These checks pass fake device addresses that a rejected call never touches;
# where a GPU is visible a wrong expectation could let one reach a kernel, so
# the module only runs on hosts without one.
pytestmark = pytest.mark.skipif(_gpu_visible(), reason="host-only checks with fake device addresses")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(S.LIB_PATH):
        from sparse_attention_decode_page_amd import build
        build.build()
    return S.lib()


def _declared():
    text = open(os.path.join(ROOT, "include", "spdec.h")).read()
    return sorted(set(re.findall(r"\b(spdec_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported(L):
    names = _declared()
    assert len(names) == len(S.ABI_FUNCTIONS) == 34
    assert set(names) == set(S.ABI_FUNCTIONS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    for code in (0, -1, -2, -3, -4):
        assert S.status_string(code).startswith("SPDEC_")
    assert "unknown" in S.status_string(7)
    assert L.spdec_version() == 100


FAKE = 0x7F0000000000  # 4 KiB-aligned address that is never dereferenced by a rejected call


def _sliced_bytes(units, G, D):
    """The sliced forms' workspace: every unit's 4096 candidate slots (page, score, page-table entry), 16 slices'
    counts and partials (acc, then (m, l)), one partial count per unit; regions rounded up to 256 bytes."""
    r = lambda x: (x + 255) // 256 * 256
    return (r(units * 4096 * 4) * 3 + r(units * 16 * 4) + r(units * 16 * G * D * 4) + r(units * 16 * G * 2 * 4)
            + r(units * 4))


def _desc(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, max_pages_per_seq=64,
                num_phys_pages=128, dtype=S.SPDEC_BF16, reserved=0, k_pool=FAKE, v_pool=FAKE + 0x100000,
                kminmax=FAKE + 0x200000, page_table=FAKE + 0x300000, seq_lens=FAKE + 0x400000)
    base.update(kw)
    return S.CacheDesc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), S.SPDEC_ERR_UNSUPPORTED),
    (dict(page_size=12), S.SPDEC_ERR_UNSUPPORTED),
    (dict(page_size=128), S.SPDEC_ERR_UNSUPPORTED),
    (dict(num_q_heads=6, num_kv_heads=2), S.SPDEC_ERR_UNSUPPORTED),    # group 3
    (dict(num_q_heads=32, num_kv_heads=2), S.SPDEC_ERR_UNSUPPORTED),   # group 16
    (dict(num_q_heads=7, num_kv_heads=2), S.SPDEC_ERR_INVALID),        # not a multiple
    (dict(dtype=5), S.SPDEC_ERR_UNSUPPORTED),
    (dict(batch=0), S.SPDEC_ERR_INVALID),
    (dict(max_pages_per_seq=40000), S.SPDEC_ERR_UNSUPPORTED),
    (dict(page_table=None), S.SPDEC_ERR_INVALID),
    (dict(seq_lens=None), S.SPDEC_ERR_INVALID),
    (dict(k_pool=FAKE + 8), S.SPDEC_ERR_INVALID),                      # misaligned pool
])
def test_descriptor_validation(L, kw, code):
    d = _desc(**kw)
    assert L.spdec_append_kv(ctypes.byref(d), FAKE, FAKE, None) == code
    if "k_pool" not in kw:
        assert L.spdec_select_pages(ctypes.byref(d), FAKE, FAKE, 16, FAKE, FAKE, FAKE, None, 0, None) == code


def test_null_descriptor_and_pointers(L):
    assert L.spdec_append_kv(None, FAKE, FAKE, None) == S.SPDEC_ERR_INVALID
    d = _desc()
    assert L.spdec_append_kv(ctypes.byref(d), None, FAKE, None) == S.SPDEC_ERR_INVALID
    assert L.spdec_select_pages(ctypes.byref(d), None, FAKE, 16, FAKE, FAKE, None, FAKE, 1 << 20, None) == -1
    assert L.spdec_sparse_decode(ctypes.byref(d), FAKE, None, FAKE, 16, 0.1, FAKE, None, FAKE, 1 << 30, None) == -1
    assert L.spdec_dense_decode(ctypes.byref(d), FAKE, 0.1, None, None, FAKE, 1 << 30, None) == -1


def test_budget_scale_and_workspace_checks(L):
    d = _desc()
    # max_budget_pages below 2
    assert L.spdec_select_pages(ctypes.byref(d), FAKE, FAKE, 1, FAKE, FAKE, None, FAKE, 1 << 30, None) == -1
    # select workspace, needed unless scores_out is given: the scores, or for a shape the sliced form takes
    # (bf16, G <= 4, at most 128 units, max_budget_pages <= 4096) the candidate slots, whichever is larger
    need = L.spdec_select_workspace_bytes(ctypes.byref(d), 16)
    assert need == _sliced_bytes(units=4, G=4, D=128)
    d32 = _desc(dtype=S.SPDEC_F32)
    assert L.spdec_select_workspace_bytes(ctypes.byref(d32), 16) == 2 * 2 * 64 * 4
    assert L.spdec_select_workspace_bytes(ctypes.byref(d), 5000) == 2 * 2 * 64 * 4
    assert L.spdec_select_workspace_bytes(ctypes.byref(d), 1) == 0
    assert L.spdec_select_pages(ctypes.byref(d), FAKE, FAKE, 16, FAKE, FAKE, None, FAKE, need - 1, None) == -3
    assert L.spdec_select_pages(ctypes.byref(d), FAKE, FAKE, 16, FAKE, FAKE, None, None, 0, None) == -3
    assert L.spdec_select_pages_form(ctypes.byref(_desc(head_dim=96)), 16) == S.SPDEC_ERR_UNSUPPORTED
    assert L.spdec_select_pages_form(ctypes.byref(d), 1) == S.SPDEC_ERR_INVALID
    assert L.spdec_select_pages_form(None, 16) == S.SPDEC_ERR_INVALID
    # decode: bad scale, then short workspace
    dw = L.spdec_decode_workspace_bytes(ctypes.byref(d), 0)
    sw = L.spdec_decode_workspace_bytes(ctypes.byref(d), 16)
    assert dw > 0 and sw > 0
    assert L.spdec_dense_decode(ctypes.byref(d), FAKE, 0.0, FAKE, None, FAKE, dw, None) == -1
    assert L.spdec_dense_decode(ctypes.byref(d), FAKE, float("nan"), FAKE, None, FAKE, dw, None) == -1
    assert L.spdec_dense_decode(ctypes.byref(d), FAKE, 0.1, FAKE, None, FAKE, dw - 1, None) == -3
    assert L.spdec_sparse_decode(ctypes.byref(d), FAKE, FAKE, FAKE, 16, 0.1, FAKE, None, FAKE, sw - 1, None) == -3
    assert L.spdec_sparse_decode(ctypes.byref(d), FAKE, FAKE, FAKE, 0, 0.1, FAKE, None, FAKE, sw, None) == -1


def test_sparse_path_checks(L):
    d = _desc()
    sp = L.spdec_sparse_path
    need = L.spdec_sparse_path_workspace_bytes(ctypes.byref(d), 16)
    # the two calls' needs (scores rounded up to 256 bytes, then the decode's workspace) or the sliced form's
    # (every unit's candidates: 4096 page, score and page-table triples, 16 slices' counts and partials), whichever
    # is larger
    scores = 2 * 2 * 64 * 4
    two = (scores + 255) // 256 * 256 + L.spdec_decode_workspace_bytes(ctypes.byref(d), 16)
    assert need == max(two, _sliced_bytes(units=4, G=4, D=128))
    assert L.spdec_sparse_path_workspace_bytes(ctypes.byref(d), 1) == 0
    assert L.spdec_sparse_path_workspace_bytes(None, 16) == 0
    args = lambda **kw: [kw.get(k, v) for k, v in (
        ("desc", ctypes.byref(d)), ("q", FAKE), ("budget", FAKE), ("cap", 16), ("scale", 0.1), ("idx", FAKE),
        ("cnt", FAKE), ("scores", None), ("out", FAKE), ("lse", None), ("ws", FAKE), ("wsb", need), ("s", None))]
    assert sp(*args(cap=1)) == -1
    assert sp(*args(scale=0.0)) == -1
    assert sp(*args(scale=float("inf"))) == -1
    assert sp(*args(budget=None)) == -1
    assert sp(*args(idx=None)) == -1
    assert sp(*args(out=None)) == -1
    assert sp(*args(q=FAKE + 4)) == -1
    assert sp(*args(wsb=need - 1)) == -3
    assert sp(*args(ws=None)) == -3
    assert sp(*args(desc=None)) == -1
    bad = _desc(head_dim=96)
    assert sp(*args(desc=ctypes.byref(bad))) == S.SPDEC_ERR_UNSUPPORTED
    # the form query rejects what the call rejects, before it looks at the device
    assert L.spdec_sparse_path_form(ctypes.byref(bad), 16) == S.SPDEC_ERR_UNSUPPORTED
    assert L.spdec_sparse_path_form(ctypes.byref(d), 1) == S.SPDEC_ERR_INVALID
    assert L.spdec_sparse_path_form(None, 16) == S.SPDEC_ERR_INVALID


def test_acceptance_checks(L):
    ws = L.spdec_acceptance_workspace_bytes(64, 151936)
    # per-row chunk partials (max and sum of both rows, then the chunk's sum of
    # minima): at least one chunk per row, and far less than the logits
    assert 64 * 5 * 4 <= ws < 64 * 151936 * 4 // 100
    assert L.spdec_acceptance_workspace_bytes(64, 2 * 151936) > ws
    assert L.spdec_acceptance_workspace_bytes(0, 10) == 0
    assert L.spdec_acceptance(FAKE, FAKE, 64, 151936, 151936, 0.0, FAKE, FAKE, ws, None) == -1   # T = 0
    assert L.spdec_acceptance(FAKE, FAKE, 64, 151936, 100, 1.0, FAKE, FAKE, ws, None) == -1      # stride < vocab
    assert L.spdec_acceptance(FAKE, FAKE, 0, 151936, 151936, 1.0, FAKE, FAKE, ws, None) == -1
    assert L.spdec_acceptance(FAKE, FAKE, 64, 151936, 151936, 1.0, FAKE, FAKE, ws - 1, None) == -3
    assert L.spdec_acceptance(None, FAKE, 64, 151936, 151936, 1.0, FAKE, FAKE, ws, None) == -1
    # the single-read form's sync region leads every workspace (zero between calls)
    assert L.spdec_acceptance_workspace_bytes(1, 1) >= 96 * 1024


def test_acceptance_noalloc_checks(L):
    na = L.spdec_acceptance_noalloc
    assert na(FAKE, FAKE, 64, 151936, 151936, 0.0, FAKE, None) == -1      # T = 0
    assert na(FAKE, FAKE, 64, 151936, 100, 1.0, FAKE, None) == -1         # stride < vocab
    assert na(None, FAKE, 64, 151936, 151936, 1.0, FAKE, None) == -1
    assert na(FAKE, FAKE, 0, 151936, 151936, 1.0, FAKE, None) == -1
    # beyond the library's scratch array (2 MiB): refused before anything touches the runtime
    assert L.spdec_acceptance_workspace_bytes(1333, 151936) > (2 << 20) >= L.spdec_acceptance_workspace_bytes(1332, 151936)
    assert na(FAKE, FAKE, 1333, 151936, 151936, 1.0, FAKE, None) == -2


def test_acceptance_ex_checks(L):
    ws = L.spdec_acceptance_workspace_bytes(64, 151936)
    ex = L.spdec_acceptance_ex
    assert ex(FAKE, FAKE, 64, 151936, 151936, 1.0, FAKE, FAKE, ws, 3, -1, None, None, None) == -1     # bad form
    assert ex(FAKE, FAKE, 64, 151936, 151936, 1.0, FAKE, FAKE, ws, 0, -1, None, None, None) == -1
    assert ex(FAKE, FAKE, 64, 151936, 151936, 1.0, FAKE, FAKE, ws, 1, -2, None, None, None) == -1     # bad limit
    assert ex(FAKE, FAKE, 64, 151936, 151936, 0.0, FAKE, FAKE, ws, -1, -1, None, None, None) == -1    # T = 0
    assert ex(FAKE, FAKE, 64, 151936, 151936, 1.0, FAKE, FAKE, ws - 1, 2, 0, None, None, None) == -3
    assert ex(FAKE, None, 64, 151936, 151936, 1.0, FAKE, FAKE, ws, -1, -1, None, None, None) == -1


def test_struct_layout_matches_header():
    assert ctypes.sizeof(S.CacheDesc) == 80
    assert S.CacheDesc.num_phys_pages.offset == 24 and S.CacheDesc.k_pool.offset == 40


def test_verify_checks(L):
    d = _desc()  # bf16, G = 4
    ws = L.spdec_verify_workspace_bytes(ctypes.byref(d), 7)
    assert ws > 0
    assert L.spdec_verify_workspace_bytes(ctypes.byref(d), 9) > ws            # G * T = 36: two 32-row passes
    assert L.spdec_verify_workspace_bytes(ctypes.byref(d), 17) == 0           # T > 16
    assert L.spdec_verify_decode(ctypes.byref(d), FAKE, 17, 0.1, FAKE, None, FAKE, ws, None) == -2
    d8 = _desc(num_q_heads=16)                                                  # G = 8
    assert L.spdec_verify_workspace_bytes(ctypes.byref(d8), 8) > 0            # G * T = 64
    assert L.spdec_verify_workspace_bytes(ctypes.byref(d8), 9) == 0           # G * T = 72 > 64
    assert L.spdec_verify_decode(ctypes.byref(d8), FAKE, 9, 0.1, FAKE, None, FAKE, ws, None) == -2
    assert L.spdec_verify_decode(ctypes.byref(d), FAKE, 0, 0.1, FAKE, None, FAKE, ws, None) == -1
    assert L.spdec_verify_decode(ctypes.byref(d), FAKE, 7, 0.0, FAKE, None, FAKE, ws, None) == -1
    assert L.spdec_verify_decode(ctypes.byref(d), FAKE, 7, 0.1, None, None, FAKE, ws, None) == -1
    assert L.spdec_verify_decode(ctypes.byref(d), FAKE, 7, 0.1, FAKE, None, FAKE, ws - 1, None) == -3
    f = _desc(dtype=S.SPDEC_F32)
    assert L.spdec_verify_workspace_bytes(ctypes.byref(f), 7) == 0
    assert L.spdec_verify_decode(ctypes.byref(f), FAKE, 7, 0.1, FAKE, None, FAKE, ws, None) == -2
    # more positions need more workspace
    assert L.spdec_verify_workspace_bytes(ctypes.byref(d), 8) > L.spdec_verify_workspace_bytes(ctypes.byref(d), 4)


def test_spec_accept_checks(L):
    ws = L.spdec_spec_accept_workspace_bytes(64, 6, 151936)
    assert ws > 0
    assert L.spdec_spec_accept_workspace_bytes(0, 6, 100) == 0
    assert L.spdec_spec_accept_workspace_bytes(4, 65, 100) == 0
    args = dict(p=FAKE, q=FAKE, B=64, k=6, V=151936, stride=151936, d=FAKE, ua=FAKE, us=FAKE, T=1.0,
                n=FAKE, t=FAKE, ws=FAKE, nbytes=ws)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return L.spdec_spec_accept(a["p"], a["q"], a["B"], a["k"], a["V"], a["stride"], a["d"], a["ua"], a["us"],
                                   a["T"], a["n"], a["t"], a["ws"], a["nbytes"], None)

    assert call(T=0.0) == -1
    assert call(stride=100) == -1
    assert call(q=None) == -1              # drafts need the drafter's logits
    # k = 0 needs no drafter inputs; with no workspace it is still rejected before any launch
    assert call(q=None, d=None, ua=None, k=0, ws=None, nbytes=0) == -3
    assert call(nbytes=ws - 1) == -3
    assert call(k=65) == -2
    assert call(B=70000) == -2
    assert call(us=None) == -1


def test_shared_prefix_checks(L):
    d = _desc(batch=4)  # bf16, G = 4
    ws = L.spdec_shared_workspace_bytes(ctypes.byref(d), 2)
    assert ws > 0
    assert L.spdec_shared_workspace_bytes(ctypes.byref(d), 3) == 0            # batch % N != 0
    d32 = _desc(batch=32)
    assert L.spdec_shared_workspace_bytes(ctypes.byref(d32), 16) > 0          # N * G = 64: two 32-row passes
    assert L.spdec_shared_workspace_bytes(ctypes.byref(d32), 32) == 0         # N * G > 64
    assert L.spdec_dense_decode_shared(ctypes.byref(d), FAKE, 3, FAKE, 0.1, FAKE, None, FAKE, ws, None) == -1
    assert L.spdec_dense_decode_shared(ctypes.byref(d), FAKE, 0, FAKE, 0.1, FAKE, None, FAKE, ws, None) == -1
    assert L.spdec_dense_decode_shared(ctypes.byref(d), FAKE, 2, None, 0.1, FAKE, None, FAKE, ws, None) == -1
    assert L.spdec_dense_decode_shared(ctypes.byref(d), FAKE, 4, FAKE, 0.1, FAKE, None, FAKE, 0, None) == -3
    assert L.spdec_dense_decode_shared(ctypes.byref(d), FAKE, 2, FAKE, 0.1, FAKE, None, FAKE, ws - 1, None) == -3
    assert L.spdec_dense_decode_shared(ctypes.byref(d), FAKE, 2, FAKE, float("inf"), FAKE, None, FAKE, ws, None) == -1
    f = _desc(batch=4, dtype=S.SPDEC_F32)
    assert L.spdec_dense_decode_shared(ctypes.byref(f), FAKE, 2, FAKE, 0.1, FAKE, None, FAKE, ws, None) == -2


def test_select_shared_checks(L):
    d = _desc(batch=4)  # bf16, G = 4
    need = L.spdec_select_workspace_bytes(ctypes.byref(d), 16)

    def call(N=2, sh=FAKE, q=FAKE, budget=FAKE, kmax=16, scores=None, ws=FAKE, nbytes=need, desc=d):
        return L.spdec_select_pages_shared(ctypes.byref(desc), q, N, sh, budget, kmax, FAKE, FAKE, scores, ws,
                                           nbytes, None)

    assert call(N=3) == -1                 # batch % N != 0
    assert call(N=0) == -1
    assert call(sh=None) == -1
    assert call(q=None) == -1
    assert call(budget=None) == -1
    assert call(kmax=1) == -1
    assert call(nbytes=need - 1) == -3     # no scores_out: the scores live in the workspace
    assert call(ws=None, nbytes=0) == -3
    e = _desc(batch=16)
    assert call(N=16, desc=e) == -2        # more than 8 members per group
    f = _desc(batch=4, dtype=S.SPDEC_F32)
    assert call(desc=f) == -2


def test_select_top_p_checks(L):
    d = _desc(batch=4)
    need = L.spdec_select_workspace_bytes(ctypes.byref(d), 16)

    def call(p=0.9, c=0.05, kmax=16, q=FAKE, ws=FAKE, nbytes=need, desc=d):
        return L.spdec_select_pages_top_p(ctypes.byref(desc), q, p, c, None, kmax, FAKE, FAKE, None, ws, nbytes, None)

    assert call(p=0.0) == -1
    assert call(p=1.5) == -1
    assert call(p=float("nan")) == -1
    assert call(c=-1.0) == -1
    assert call(c=float("inf")) == -1
    assert call(kmax=1) == -1
    assert call(q=None) == -1
    assert call(nbytes=need - 1) == -3
    assert call(ws=None, nbytes=0) == -3
    f = _desc(batch=4, dtype=S.SPDEC_F32)
    assert call(desc=f, q=None) == -1


def test_budget_update_checks(L):
    def call(batch=64, tail=FAKE, scale=FAKE, lens=FAKE, out=FAKE, **kw):
        p = dict(target=0.86, gain=0.5, scale_min=0.125, scale_max=8.0, base_tokens=1024.0, tokens_per_token=0.125,
                 page_size=16, max_budget_pages=256)
        p.update(kw)
        prm = S.BudgetParams(**p)
        return L.spdec_budget_update(tail, scale, lens, batch, ctypes.byref(prm), out, None)

    assert call(tail=None) == -1
    assert call(scale=None) == -1
    assert call(lens=None) == -1
    assert call(out=None) == -1
    assert call(batch=0) == -1
    assert call(batch=65537) == -1
    assert call(target=0.0) == -1
    assert call(target=1.5) == -1
    assert call(target=float("nan")) == -1
    assert call(gain=-0.1) == -1
    assert call(gain=float("inf")) == -1
    assert call(scale_min=0.0) == -1
    assert call(scale_min=2.0, scale_max=1.0) == -1
    assert call(base_tokens=-1.0) == -1
    assert call(tokens_per_token=-0.5) == -1
    assert call(page_size=12) == -1
    assert call(page_size=0) == -1
    assert call(max_budget_pages=1) == -1
    assert call(max_budget_pages=40000) == -1


def test_tail_stats_checks(L):
    assert L.spdec_tail_stats(None, 10, FAKE, None) == -1
    assert L.spdec_tail_stats(FAKE, 0, FAKE, None) == -1
    assert L.spdec_tail_stats(FAKE, 10, None, None) == -1
    assert L.spdec_tail_stats(FAKE, 8193, FAKE, None) == -2


def test_check_inputs_checks(L):
    d = _desc(batch=4)
    chk = L.spdec_check_inputs
    assert chk(ctypes.byref(d), FAKE, FAKE, FAKE, 8, 2, FAKE, None, None) == -1       # no report
    assert chk(ctypes.byref(d), None, FAKE, None, 8, 1, None, FAKE, None) == -1       # sel_idx without sel_cnt
    assert chk(ctypes.byref(d), None, None, FAKE, 8, 1, None, FAKE, None) == -1       # sel_cnt without sel_idx
    assert chk(ctypes.byref(d), None, FAKE, FAKE, 0, 1, None, FAKE, None) == -1       # selection with no capacity
    assert chk(ctypes.byref(d), None, None, None, 0, 3, FAKE, FAKE, None) == -1       # group does not divide batch
    assert chk(ctypes.byref(d), None, None, None, 0, 0, FAKE, FAKE, None) == -1
    assert chk(None, None, None, None, 0, 1, None, FAKE, None) == -1
    bad = _desc(batch=4, head_dim=96)
    assert chk(ctypes.byref(bad), None, None, None, 0, 1, None, FAKE, None) == -2


def test_probe_library_rejects_bad_arguments():
    """The gather-ceiling probe (a separate library that bench.py times) loads, exports its two calls and
    rejects bad arguments before touching the GPU."""
    from sparse_attention_decode_page_amd import build as B
    if not os.path.exists(B.PROBE_LIB_PATH):
        B.build()
    P = ctypes.CDLL(B.PROBE_LIB_PATH)
    P.spdec_probe_gather.restype = ctypes.c_int
    P.spdec_probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    P.spdec_probe_sink_words.restype = ctypes.c_int
    assert P.spdec_probe_sink_words() == 65536
    assert P.spdec_probe_gather(None, None, FAKE, 4, 4096, FAKE, None) == -1     # no base
    assert P.spdec_probe_gather(FAKE, None, None, 4, 4096, FAKE, None) == -1     # no offsets
    assert P.spdec_probe_gather(FAKE, None, FAKE, 4, 4096, None, None) == -1     # no sink
    assert P.spdec_probe_gather(FAKE, None, FAKE, 0, 4096, FAKE, None) == -1     # empty list
    assert P.spdec_probe_gather(FAKE, None, FAKE, 4, 3000, FAKE, None) == -1     # block not a power of two
    assert P.spdec_probe_gather(FAKE, None, FAKE, 4, 256, FAKE, None) == -1      # below 512 bytes


def test_default_scales(L):
    """The library's default softmax scale 1/sqrt(D) and top-p score scale 1/(G sqrt(D)), each the fp32
    rounding of the fp64 value; 0 for an invalid descriptor."""
    import math
    for D, Hq, Hkv in ((128, 8, 2), (64, 32, 4), (128, 8, 8)):
        d = _desc(head_dim=D, num_q_heads=Hq, num_kv_heads=Hkv)
        got = L.spdec_default_scale(ctypes.byref(d))
        assert np.float32(got) == np.float32(1.0 / math.sqrt(D))
        got = L.spdec_default_score_scale(ctypes.byref(d))
        assert np.float32(got) == np.float32(1.0 / ((Hq // Hkv) * math.sqrt(D)))
    bad = _desc(head_dim=96)
    assert L.spdec_default_scale(ctypes.byref(bad)) == 0.0
    assert L.spdec_default_score_scale(ctypes.byref(bad)) == 0.0
