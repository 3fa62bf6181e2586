"""Python binding of libspdec (ctypes): argument marshalling only.

Every step runs in the HIP kernels behind the C ABI declared in
``include/spdec.h``; this module only turns torch device tensors into raw
pointers, passes torch's current HIP stream, and raises on a non-OK status.
PyTorch provides device memory and streams. There is no fallback: if the
shared library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspdec.so")

SPDEC_OK, SPDEC_ERR_INVALID, SPDEC_ERR_UNSUPPORTED, SPDEC_ERR_WORKSPACE, SPDEC_ERR_HIP = 0, -1, -2, -3, -4
SPDEC_F32, SPDEC_BF16 = 0, 1

ABI_FUNCTIONS = (
    "spdec_default_scale", "spdec_default_score_scale",
    "spdec_status_string", "spdec_version", "spdec_append_kv", "spdec_build_meta",
    "spdec_select_workspace_bytes", "spdec_select_pages_form", "spdec_select_pages", "spdec_select_pages_shared", "spdec_select_pages_top_p",
    "spdec_decode_workspace_bytes",
    "spdec_sparse_decode", "spdec_sparse_path_workspace_bytes", "spdec_sparse_path_form", "spdec_sparse_path",
    "spdec_dense_decode",
    "spdec_shared_workspace_bytes", "spdec_dense_decode_shared",
    "spdec_verify_workspace_bytes", "spdec_verify_decode",
    "spdec_spec_accept_workspace_bytes", "spdec_spec_accept", "spdec_acceptance_workspace_bytes",
    "spdec_acceptance", "spdec_acceptance_ex", "spdec_acceptance_noalloc", "spdec_tail_stats",
    "spdec_monitor_workspace_bytes", "spdec_monitor_reset", "spdec_monitor_append", "spdec_monitor_stats", "spdec_budget_update", "spdec_check_inputs",
)
SPDEC_CHECK_WORDS, SPDEC_CHECK_FIRST = 8, 5


class CacheDesc(ctypes.Structure):
    """Mirror of ``struct spdec_cache``."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int64), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p), ("kminmax", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
    ]


class BudgetParams(ctypes.Structure):
    """Mirror of ``struct spdec_budget_params`` (controller settings)."""
    _fields_ = [
        ("target", ctypes.c_float), ("gain", ctypes.c_float), ("scale_min", ctypes.c_float),
        ("scale_max", ctypes.c_float), ("base_tokens", ctypes.c_float), ("tokens_per_token", ctypes.c_float),
        ("page_size", ctypes.c_int32), ("max_budget_pages", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libspdec.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run sparse_attention_decode_page_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    D = ctypes.POINTER(CacheDesc)
    sig = {
        "spdec_status_string": (ctypes.c_char_p, [I]),
        "spdec_version": (I, []),
        "spdec_default_scale": (ctypes.c_float, [D]),
        "spdec_default_score_scale": (ctypes.c_float, [D]),
        "spdec_append_kv": (I, [D, P, P, P]),
        "spdec_build_meta": (I, [D, P]),
        "spdec_select_workspace_bytes": (SZ, [D, I]),
        "spdec_select_pages_form": (I, [D, I]),
        "spdec_select_pages": (I, [D, P, P, I, P, P, P, P, SZ, P]),
        "spdec_select_pages_shared": (I, [D, P, I, P, P, I, P, P, P, P, SZ, P]),
        "spdec_select_pages_top_p": (I, [D, P, F, F, P, I, P, P, P, P, SZ, P]),
        "spdec_decode_workspace_bytes": (SZ, [D, I]),
        "spdec_sparse_decode": (I, [D, P, P, P, I, F, P, P, P, SZ, P]),
        "spdec_sparse_path_workspace_bytes": (SZ, [D, I]),
        "spdec_sparse_path_form": (I, [D, I]),
        "spdec_sparse_path": (I, [D, P, P, I, F, P, P, P, P, P, P, SZ, P]),
        "spdec_dense_decode": (I, [D, P, F, P, P, P, SZ, P]),
        "spdec_shared_workspace_bytes": (SZ, [D, I]),
        "spdec_dense_decode_shared": (I, [D, P, I, P, F, P, P, P, SZ, P]),
        "spdec_verify_workspace_bytes": (SZ, [D, I]),
        "spdec_verify_decode": (I, [D, P, I, F, P, P, P, SZ, P]),
        "spdec_spec_accept_workspace_bytes": (SZ, [I, I, I]),
        "spdec_spec_accept": (I, [P, P, I, I, I, I64, P, P, P, F, P, P, P, SZ, P]),
        "spdec_acceptance_workspace_bytes": (SZ, [I, I]),
        "spdec_acceptance": (I, [P, P, I, I, I64, F, P, P, SZ, P]),
        "spdec_acceptance_noalloc": (I, [P, P, I, I, I64, F, P, P]),
        "spdec_acceptance_ex": (I, [P, P, I, I, I64, F, P, P, SZ, I, I, P, ctypes.POINTER(ctypes.c_int32), P]),
        "spdec_tail_stats": (I, [P, I, P, P]),
        "spdec_monitor_workspace_bytes": (SZ, [I]),
        "spdec_monitor_reset": (I, [P, I, P]),
        "spdec_monitor_append": (I, [P, I, P, I, P]),
        "spdec_monitor_stats": (I, [P, I, P, P]),
        "spdec_budget_update": (I, [P, P, P, I, ctypes.POINTER(BudgetParams), P, P]),
        "spdec_check_inputs": (I, [D, P, P, P, I, I, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().spdec_status_string(status).decode()


def _check(status: int, what: str):
    if status != SPDEC_OK:
        raise RuntimeError(f"{what} failed: {status_string(status)}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _default_scale(cache) -> float:
    return lib().spdec_default_scale(ctypes.byref(cache.desc))


def _workspace(nbytes: int, device, given: Optional[torch.Tensor]) -> torch.Tensor:
    if given is not None:
        return given
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class PagedCache:
    """Paged KV cache: torch device tensors plus the ``spdec_cache`` descriptor over them.

    k_pool, v_pool: [num_phys_pages][Hkv][page_size][D] (bfloat16 or float32);
    kminmax: [num_phys_pages][Hkv][2][D] same dtype; page_table: int32
    [batch][max_pages]; seq_lens: int32 [batch].
    """

    def __init__(self, k_pool, v_pool, kminmax, page_table, seq_lens, num_q_heads: int):
        for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool"), (kminmax, "kminmax")):
            _need(t, n)
        _need(page_table, "page_table", torch.int32)
        _need(seq_lens, "seq_lens", torch.int32)
        if k_pool.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("cache dtype must be bfloat16 or float32")
        if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype or kminmax.dtype != k_pool.dtype:
            raise ValueError("k_pool, v_pool and kminmax must share dtype and pool shape")
        nphys, hkv, ps, d = k_pool.shape
        if tuple(kminmax.shape) != (nphys, hkv, 2, d):
            raise ValueError("kminmax must be [num_phys_pages][Hkv][2][D]")
        batch, max_pages = page_table.shape
        if tuple(seq_lens.shape) != (batch,):
            raise ValueError("seq_lens must be [batch]")
        self.k_pool, self.v_pool, self.kminmax = k_pool, v_pool, kminmax
        self.page_table, self.seq_lens = page_table, seq_lens
        self.batch, self.num_q_heads, self.num_kv_heads = batch, int(num_q_heads), hkv
        self.head_dim, self.page_size, self.max_pages, self.num_phys = d, ps, max_pages, nphys
        self.dtype = k_pool.dtype
        self.desc = CacheDesc(batch, self.num_q_heads, hkv, d, ps, max_pages, nphys,
                              SPDEC_BF16 if k_pool.dtype == torch.bfloat16 else SPDEC_F32, 0,
                              k_pool.data_ptr(), v_pool.data_ptr(), kminmax.data_ptr(),
                              page_table.data_ptr(), seq_lens.data_ptr())

    @property
    def device(self):
        return self.k_pool.device


def append_kv(cache: PagedCache, k_new: torch.Tensor, v_new: torch.Tensor):
    shape = (cache.batch, cache.num_kv_heads, cache.head_dim)
    _need(k_new, "k_new", cache.dtype, shape)
    _need(v_new, "v_new", cache.dtype, shape)
    _check(lib().spdec_append_kv(ctypes.byref(cache.desc), _ptr(k_new), _ptr(v_new), _stream()), "spdec_append_kv")


def build_meta(cache: PagedCache):
    _check(lib().spdec_build_meta(ctypes.byref(cache.desc), _stream()), "spdec_build_meta")


def select_workspace_bytes(cache: PagedCache, max_budget_pages: int) -> int:
    return int(lib().spdec_select_workspace_bytes(ctypes.byref(cache.desc), int(max_budget_pages)))


def select_pages_form(cache: PagedCache, max_budget_pages: int) -> str:
    """Which form select_pages takes for this shape on the current device with the full workspace:
    "one kernel", "sliced" or "two calls" (a scoring and a Top-k kernel)."""
    r = int(lib().spdec_select_pages_form(ctypes.byref(cache.desc), int(max_budget_pages)))
    _check(min(r, 0), "spdec_select_pages_form")
    return PATH_FORMS[r]


def select_pages(cache: PagedCache, q, budget_pages, max_budget_pages: int, sel_idx=None, sel_cnt=None,
                 scores_out=None, workspace=None):
    _need(q, "q", cache.dtype, (cache.batch, cache.num_q_heads, cache.head_dim))
    _need(budget_pages, "budget_pages", torch.int32, (cache.batch,))
    dev = cache.device
    if sel_idx is None:
        sel_idx = torch.zeros((cache.batch, cache.num_kv_heads, max_budget_pages), dtype=torch.int32, device=dev)
    if sel_cnt is None:
        sel_cnt = torch.zeros((cache.batch, cache.num_kv_heads), dtype=torch.int32, device=dev)
    _need(sel_idx, "sel_idx", torch.int32, (cache.batch, cache.num_kv_heads, max_budget_pages))
    _need(sel_cnt, "sel_cnt", torch.int32, (cache.batch, cache.num_kv_heads))
    if scores_out is not None:
        _need(scores_out, "scores_out", torch.float32, (cache.batch, cache.num_kv_heads, cache.max_pages))
        ws_ptr, ws_bytes = _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size()
    else:
        workspace = _workspace(select_workspace_bytes(cache, max_budget_pages), dev, workspace)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    _check(lib().spdec_select_pages(ctypes.byref(cache.desc), _ptr(q), _ptr(budget_pages), int(max_budget_pages),
                                    _ptr(sel_idx), _ptr(sel_cnt), _ptr(scores_out), ws_ptr, ws_bytes, _stream()),
           "spdec_select_pages")
    return sel_idx, sel_cnt


def select_pages_top_p(cache: PagedCache, q, top_p: float, max_budget_pages: int, score_scale: Optional[float] = None,
                       budget_pages=None, sel_idx=None, sel_cnt=None, scores_out=None, workspace=None):
    """Score-mass page selection: keep pages (sink, local, then by score) until top_p of the page mass;
    score_scale defaults to 1/(G*sqrt(D)); budget_pages (optional) caps each sequence."""
    _need(q, "q", cache.dtype, (cache.batch, cache.num_q_heads, cache.head_dim))
    if budget_pages is not None:
        _need(budget_pages, "budget_pages", torch.int32, (cache.batch,))
    if score_scale is None:
        score_scale = lib().spdec_default_score_scale(ctypes.byref(cache.desc))
    dev = cache.device
    if sel_idx is None:
        sel_idx = torch.zeros((cache.batch, cache.num_kv_heads, max_budget_pages), dtype=torch.int32, device=dev)
    if sel_cnt is None:
        sel_cnt = torch.zeros((cache.batch, cache.num_kv_heads), dtype=torch.int32, device=dev)
    _need(sel_idx, "sel_idx", torch.int32, (cache.batch, cache.num_kv_heads, max_budget_pages))
    _need(sel_cnt, "sel_cnt", torch.int32, (cache.batch, cache.num_kv_heads))
    if scores_out is not None:
        _need(scores_out, "scores_out", torch.float32, (cache.batch, cache.num_kv_heads, cache.max_pages))
        ws_ptr, ws_bytes = _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size()
    else:
        workspace = _workspace(select_workspace_bytes(cache, max_budget_pages), dev, workspace)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    _check(lib().spdec_select_pages_top_p(ctypes.byref(cache.desc), _ptr(q), float(top_p), float(score_scale),
                                          _ptr(budget_pages), int(max_budget_pages), _ptr(sel_idx), _ptr(sel_cnt),
                                          _ptr(scores_out), ws_ptr, ws_bytes, _stream()),
           "spdec_select_pages_top_p")
    return sel_idx, sel_cnt


def select_pages_shared(cache: PagedCache, q, group_size: int, shared_pages, budget_pages, max_budget_pages: int,
                        sel_idx=None, sel_cnt=None, scores_out=None, workspace=None):
    """select_pages where groups of group_size consecutive sequences share shared_pages[n] leading pages."""
    _need(q, "q", cache.dtype, (cache.batch, cache.num_q_heads, cache.head_dim))
    _need(budget_pages, "budget_pages", torch.int32, (cache.batch,))
    if int(group_size) < 1 or cache.batch % int(group_size) != 0:
        raise ValueError("batch must be a multiple of group_size")
    _need(shared_pages, "shared_pages", torch.int32, (cache.batch // int(group_size),))
    dev = cache.device
    if sel_idx is None:
        sel_idx = torch.zeros((cache.batch, cache.num_kv_heads, max_budget_pages), dtype=torch.int32, device=dev)
    if sel_cnt is None:
        sel_cnt = torch.zeros((cache.batch, cache.num_kv_heads), dtype=torch.int32, device=dev)
    _need(sel_idx, "sel_idx", torch.int32, (cache.batch, cache.num_kv_heads, max_budget_pages))
    _need(sel_cnt, "sel_cnt", torch.int32, (cache.batch, cache.num_kv_heads))
    if scores_out is not None:
        _need(scores_out, "scores_out", torch.float32, (cache.batch, cache.num_kv_heads, cache.max_pages))
        ws_ptr, ws_bytes = _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size()
    else:
        workspace = _workspace(select_workspace_bytes(cache, max_budget_pages), dev, workspace)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    _check(lib().spdec_select_pages_shared(ctypes.byref(cache.desc), _ptr(q), int(group_size), _ptr(shared_pages),
                                           _ptr(budget_pages), int(max_budget_pages), _ptr(sel_idx), _ptr(sel_cnt),
                                           _ptr(scores_out), ws_ptr, ws_bytes, _stream()),
           "spdec_select_pages_shared")
    return sel_idx, sel_cnt


def decode_workspace_bytes(cache: PagedCache, max_budget_pages: int) -> int:
    return int(lib().spdec_decode_workspace_bytes(ctypes.byref(cache.desc), int(max_budget_pages)))


def _outs(cache, out, lse):
    dev = cache.device
    if out is None:
        out = torch.empty((cache.batch, cache.num_q_heads, cache.head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((cache.batch, cache.num_q_heads), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (cache.batch, cache.num_q_heads, cache.head_dim))
    _need(lse, "lse", torch.float32, (cache.batch, cache.num_q_heads))
    return out, lse


def sparse_decode(cache: PagedCache, q, sel_idx, sel_cnt, max_budget_pages: int, scale: Optional[float] = None,
                  out=None, lse=None, workspace=None):
    _need(q, "q", cache.dtype, (cache.batch, cache.num_q_heads, cache.head_dim))
    _need(sel_idx, "sel_idx", torch.int32, (cache.batch, cache.num_kv_heads, max_budget_pages))
    _need(sel_cnt, "sel_cnt", torch.int32, (cache.batch, cache.num_kv_heads))
    out, lse = _outs(cache, out, lse)
    scale = _default_scale(cache) if scale is None else float(scale)
    ws = _workspace(decode_workspace_bytes(cache, max_budget_pages), cache.device, workspace)
    _check(lib().spdec_sparse_decode(ctypes.byref(cache.desc), _ptr(q), _ptr(sel_idx), _ptr(sel_cnt),
                                     int(max_budget_pages), scale, _ptr(out), _ptr(lse), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream()), "spdec_sparse_decode")
    return out, lse


def sparse_path_workspace_bytes(cache: PagedCache, max_budget_pages: int) -> int:
    return int(lib().spdec_sparse_path_workspace_bytes(ctypes.byref(cache.desc), int(max_budget_pages)))


PATH_FORMS = {0: "two calls", 1: "one kernel", 2: "sliced"}


def sparse_path_form(cache: PagedCache, max_budget_pages: int) -> str:
    """The form sparse_path takes for this cache shape on the current device: "one kernel", "sliced" or
    "two calls"."""
    r = int(lib().spdec_sparse_path_form(ctypes.byref(cache.desc), int(max_budget_pages)))
    _check(min(r, 0), "spdec_sparse_path_form")
    return PATH_FORMS[r]


def sparse_path(cache: PagedCache, q, budget_pages, max_budget_pages: int, scale: Optional[float] = None,
                sel_idx=None, sel_cnt=None, scores_out=None, out=None, lse=None, workspace=None):
    """One sparse decode step (select_pages, then sparse_decode over the kept pages) through spdec_sparse_path.
    Returns (out, lse, sel_idx, sel_cnt)."""
    _need(q, "q", cache.dtype, (cache.batch, cache.num_q_heads, cache.head_dim))
    _need(budget_pages, "budget_pages", torch.int32, (cache.batch,))
    dev = cache.device
    if sel_idx is None:
        sel_idx = torch.zeros((cache.batch, cache.num_kv_heads, max_budget_pages), dtype=torch.int32, device=dev)
    if sel_cnt is None:
        sel_cnt = torch.zeros((cache.batch, cache.num_kv_heads), dtype=torch.int32, device=dev)
    _need(sel_idx, "sel_idx", torch.int32, (cache.batch, cache.num_kv_heads, max_budget_pages))
    _need(sel_cnt, "sel_cnt", torch.int32, (cache.batch, cache.num_kv_heads))
    if scores_out is not None:
        _need(scores_out, "scores_out", torch.float32, (cache.batch, cache.num_kv_heads, cache.max_pages))
    out, lse = _outs(cache, out, lse)
    scale = _default_scale(cache) if scale is None else float(scale)
    ws = _workspace(sparse_path_workspace_bytes(cache, max_budget_pages), dev, workspace)
    _check(lib().spdec_sparse_path(ctypes.byref(cache.desc), _ptr(q), _ptr(budget_pages), int(max_budget_pages),
                                   scale, _ptr(sel_idx), _ptr(sel_cnt), _ptr(scores_out), _ptr(out), _ptr(lse),
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream()), "spdec_sparse_path")
    return out, lse, sel_idx, sel_cnt


def dense_decode(cache: PagedCache, q, scale: Optional[float] = None, out=None, lse=None, workspace=None):
    _need(q, "q", cache.dtype, (cache.batch, cache.num_q_heads, cache.head_dim))
    out, lse = _outs(cache, out, lse)
    scale = _default_scale(cache) if scale is None else float(scale)
    ws = _workspace(decode_workspace_bytes(cache, 0), cache.device, workspace)
    _check(lib().spdec_dense_decode(ctypes.byref(cache.desc), _ptr(q), scale, _ptr(out), _ptr(lse), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream()), "spdec_dense_decode")
    return out, lse


def shared_workspace_bytes(cache: PagedCache, group_size: int) -> int:
    return int(lib().spdec_shared_workspace_bytes(ctypes.byref(cache.desc), int(group_size)))


def dense_decode_shared(cache: PagedCache, q, group_size: int, shared_pages, scale: Optional[float] = None,
                        out=None, lse=None, workspace=None):
    """Dense decode where groups of group_size consecutive sequences share shared_pages[n] leading pages."""
    _need(q, "q", cache.dtype, (cache.batch, cache.num_q_heads, cache.head_dim))
    if cache.batch % int(group_size) != 0:
        raise ValueError("batch must be a multiple of group_size")
    _need(shared_pages, "shared_pages", torch.int32, (cache.batch // int(group_size),))
    out, lse = _outs(cache, out, lse)
    scale = _default_scale(cache) if scale is None else float(scale)
    ws = _workspace(shared_workspace_bytes(cache, group_size), cache.device, workspace)
    _check(lib().spdec_dense_decode_shared(ctypes.byref(cache.desc), _ptr(q), int(group_size), _ptr(shared_pages),
                                           scale, _ptr(out), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                           _stream()), "spdec_dense_decode_shared")
    return out, lse


def verify_workspace_bytes(cache: PagedCache, num_positions: int) -> int:
    return int(lib().spdec_verify_workspace_bytes(ctypes.byref(cache.desc), int(num_positions)))


def verify_decode(cache: PagedCache, q, scale: Optional[float] = None, out=None, lse=None, workspace=None):
    """Causal multi-query attention of the last T cached positions: q [batch][T][Hq][D] (bf16 cache)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [batch][T][Hq][D] tensor")
    T = int(q.shape[1])
    _need(q, "q", cache.dtype, (cache.batch, T, cache.num_q_heads, cache.head_dim))
    dev = cache.device
    if out is None:
        out = torch.empty((cache.batch, T, cache.num_q_heads, cache.head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((cache.batch, T, cache.num_q_heads), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (cache.batch, T, cache.num_q_heads, cache.head_dim))
    _need(lse, "lse", torch.float32, (cache.batch, T, cache.num_q_heads))
    scale = _default_scale(cache) if scale is None else float(scale)
    ws = _workspace(verify_workspace_bytes(cache, T), dev, workspace)
    _check(lib().spdec_verify_decode(ctypes.byref(cache.desc), _ptr(q), T, scale, _ptr(out), _ptr(lse), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream()), "spdec_verify_decode")
    return out, lse


def spec_accept_workspace_bytes(batch: int, num_draft: int, vocab: int) -> int:
    return int(lib().spdec_spec_accept_workspace_bytes(int(batch), int(num_draft), int(vocab)))


def spec_accept(p_logits, q_logits, draft, u_accept, u_sample, temperature: float = 1.0, num_accepted=None,
                next_token=None, workspace=None):
    """Exact speculative sampling: p_logits [batch][k+1][vocab], q_logits [batch][k][vocab] fp32,
    draft [batch][k] int32, u_accept [batch][k] / u_sample [batch] fp32 uniforms.
    Returns (num_accepted [batch], next_token [batch]) int32."""
    if not isinstance(p_logits, torch.Tensor) or p_logits.dim() != 3 or p_logits.dtype != torch.float32:
        raise ValueError("p_logits must be a [batch][k+1][vocab] float32 tensor")
    batch, k1, vocab = p_logits.shape
    k = k1 - 1
    if p_logits.stride(2) != 1 or p_logits.stride(0) != k1 * p_logits.stride(1):
        raise ValueError("p_logits rows must be contiguous and evenly strided")
    stride = p_logits.stride(1)
    dev = p_logits.device
    if k > 0:
        if (not isinstance(q_logits, torch.Tensor) or q_logits.dtype != torch.float32
                or tuple(q_logits.shape) != (batch, k, vocab)):
            raise ValueError("q_logits must be a [batch][k][vocab] float32 tensor")
        if q_logits.stride(2) != 1 or q_logits.stride(1) != stride or q_logits.stride(0) != k * stride:
            raise ValueError("q_logits must share p_logits' row stride")
        _need(draft, "draft", torch.int32, (batch, k))
        _need(u_accept, "u_accept", torch.float32, (batch, k))
    _need(u_sample, "u_sample", torch.float32, (batch,))
    if num_accepted is None:
        num_accepted = torch.empty(batch, dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty(batch, dtype=torch.int32, device=dev)
    _need(num_accepted, "num_accepted", torch.int32, (batch,))
    _need(next_token, "next_token", torch.int32, (batch,))
    ws = _workspace(spec_accept_workspace_bytes(batch, k, vocab), dev, workspace)
    _check(lib().spdec_spec_accept(_ptr(p_logits), _ptr(q_logits) if k > 0 else None, batch, k, vocab, stride,
                                   _ptr(draft) if k > 0 else None, _ptr(u_accept) if k > 0 else None,
                                   _ptr(u_sample), float(temperature), _ptr(num_accepted), _ptr(next_token),
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream()), "spdec_spec_accept")
    return num_accepted, next_token


def acceptance_workspace_bytes(rows: int, vocab: int) -> int:
    return int(lib().spdec_acceptance_workspace_bytes(int(rows), int(vocab)))


def acceptance(logits_a, logits_b, temperature: float = 1.0, alpha=None, workspace=None):
    """Per-row acceptance sum_v min(softmax(a/T), softmax(b/T)) of two [rows][vocab] fp32 tensors."""
    for t, n in ((logits_a, "logits_a"), (logits_b, "logits_b")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 or t.dim() != 2:
            raise ValueError(f"{n} must be a 2-D float32 GPU tensor")
        if t.stride(1) != 1:
            raise ValueError(f"{n} rows must be contiguous")
    if logits_a.shape != logits_b.shape or logits_a.stride(0) != logits_b.stride(0):
        raise ValueError("logits_a and logits_b must share shape and row stride")
    rows, vocab = logits_a.shape
    if alpha is None:
        alpha = torch.empty(rows, dtype=torch.float32, device=logits_a.device)
    _need(alpha, "alpha", torch.float32, (rows,))
    ws = _workspace(acceptance_workspace_bytes(rows, vocab), logits_a.device, workspace)
    _check(lib().spdec_acceptance(_ptr(logits_a), _ptr(logits_b), rows, vocab, logits_a.stride(0),
                                  float(temperature), _ptr(alpha), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream()), "spdec_acceptance")
    return alpha


def acceptance_noalloc(logits_a, logits_b, temperature: float = 1.0, alpha=None):
    """spdec_acceptance on the library's own per-GPU scratch array (no workspace argument, nothing allocated by
    the call; `alpha` may be passed in to keep the call allocation-free on the Python side too)."""
    for t, n in ((logits_a, "logits_a"), (logits_b, "logits_b")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 or t.dim() != 2:
            raise ValueError(f"{n} must be a 2-D float32 GPU tensor")
        if t.stride(1) != 1:
            raise ValueError(f"{n} rows must be contiguous")
    if logits_a.shape != logits_b.shape or logits_a.stride(0) != logits_b.stride(0):
        raise ValueError("logits_a and logits_b must share shape and row stride")
    rows, vocab = logits_a.shape
    if alpha is None:
        alpha = torch.empty(rows, dtype=torch.float32, device=logits_a.device)
    _need(alpha, "alpha", torch.float32, (rows,))
    _check(lib().spdec_acceptance_noalloc(_ptr(logits_a), _ptr(logits_b), rows, vocab, logits_a.stride(0),
                                          float(temperature), _ptr(alpha), _stream()), "spdec_acceptance_noalloc")
    return alpha


def acceptance_ex(logits_a, logits_b, temperature: float = 1.0, alpha=None, workspace=None, force_path: int = -1,
                  spin_limit: int = -1, fallbacks=None):
    """spdec_acceptance with its form and wait explicit: force_path -1 (automatic), 1 (single read) or 2 (two
    passes); spin_limit -1 (default) or the polls before a waiting chunk reads its row itself; fallbacks: an int32
    [1] GPU tensor incremented by every chunk that stopped waiting. Returns (alpha, path taken)."""
    for t, n in ((logits_a, "logits_a"), (logits_b, "logits_b")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 or t.dim() != 2:
            raise ValueError(f"{n} must be a 2-D float32 GPU tensor")
        if t.stride(1) != 1:
            raise ValueError(f"{n} rows must be contiguous")
    if logits_a.shape != logits_b.shape or logits_a.stride(0) != logits_b.stride(0):
        raise ValueError("logits_a and logits_b must share shape and row stride")
    rows, vocab = logits_a.shape
    if alpha is None:
        alpha = torch.empty(rows, dtype=torch.float32, device=logits_a.device)
    _need(alpha, "alpha", torch.float32, (rows,))
    if fallbacks is not None:
        _need(fallbacks, "fallbacks", torch.int32, (1,))
    ws = _workspace(acceptance_workspace_bytes(rows, vocab), logits_a.device, workspace)
    path = ctypes.c_int32(0)
    _check(lib().spdec_acceptance_ex(_ptr(logits_a), _ptr(logits_b), rows, vocab, logits_a.stride(0),
                                     float(temperature), _ptr(alpha), _ptr(ws), ws.numel() * ws.element_size(),
                                     int(force_path), int(spin_limit), _ptr(fallbacks), ctypes.byref(path),
                                     _stream()), "spdec_acceptance_ex")
    return alpha, int(path.value)


class TailMonitor:
    """Streaming tail monitor: a device ring of the `capacity` most recent per-token acceptance values, their
    mean and lower 5th percentile taken on the device (spdec_monitor_*)."""

    def __init__(self, capacity: int, device="cuda"):
        self.capacity = int(capacity)
        nbytes = int(lib().spdec_monitor_workspace_bytes(self.capacity))
        if nbytes == 0:
            raise ValueError("capacity must be in [1, 2^28]")
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)   # zero-filled: an empty window

    def reset(self):
        _check(lib().spdec_monitor_reset(_ptr(self.ws), self.capacity, _stream()), "spdec_monitor_reset")

    def append(self, alpha):
        if not isinstance(alpha, torch.Tensor) or alpha.dim() != 1:
            raise ValueError("alpha must be a 1-D tensor")
        _need(alpha, "alpha", torch.float32, (alpha.shape[0],))
        _check(lib().spdec_monitor_append(_ptr(self.ws), self.capacity, _ptr(alpha), int(alpha.shape[0]), _stream()),
               "spdec_monitor_append")

    def stats(self, out=None):
        if out is None:
            out = torch.empty(2, dtype=torch.float32, device=self.ws.device)
        _need(out, "out", torch.float32, (2,))
        _check(lib().spdec_monitor_stats(_ptr(self.ws), self.capacity, _ptr(out), _stream()), "spdec_monitor_stats")
        return out

    def count(self) -> int:
        return int(self.ws[:8].view(torch.int64).item())


def tail_stats(alpha, out=None):
    """Mean and lower 5th percentile (linear interpolation) of a 1-D float32 GPU tensor: a [2] tensor."""
    if not isinstance(alpha, torch.Tensor) or alpha.dim() != 1:
        raise ValueError("alpha must be a 1-D tensor")
    _need(alpha, "alpha", torch.float32, (alpha.shape[0],))
    if out is None:
        out = torch.empty(2, dtype=torch.float32, device=alpha.device)
    _need(out, "out", torch.float32, (2,))
    _check(lib().spdec_tail_stats(_ptr(alpha), int(alpha.shape[0]), _ptr(out), _stream()), "spdec_tail_stats")
    return out


def budget_update(tail, scale, seq_lens, params: BudgetParams, budget_pages=None):
    """One controller step on the device: tail [2] (mean, p5), scale [1] state (updated in place),
    seq_lens [batch] int32 -> budget_pages [batch] int32."""
    _need(tail, "tail", torch.float32, (2,))
    _need(scale, "scale", torch.float32, (1,))
    if not isinstance(seq_lens, torch.Tensor) or seq_lens.dim() != 1:
        raise ValueError("seq_lens must be a 1-D tensor")
    batch = int(seq_lens.shape[0])
    _need(seq_lens, "seq_lens", torch.int32, (batch,))
    if budget_pages is None:
        budget_pages = torch.empty(batch, dtype=torch.int32, device=seq_lens.device)
    _need(budget_pages, "budget_pages", torch.int32, (batch,))
    _check(lib().spdec_budget_update(_ptr(tail), _ptr(scale), _ptr(seq_lens), batch, ctypes.byref(params),
                                     _ptr(budget_pages), _stream()), "spdec_budget_update")
    return budget_pages


CHECK_FIELDS = ("bad_lengths", "bad_page_entries", "bad_selection_rows", "nonfinite_q", "bad_shared_groups",
                "first_bad_sequence")


def check_inputs(cache: PagedCache, q=None, sel_idx=None, sel_cnt=None, max_budget_pages: int = 0,
                 group_size: int = 1, shared_pages=None, report=None) -> dict:
    """Device-side precondition counts (``spdec_check_inputs``); synchronises to read them back."""
    if report is None:
        report = torch.empty(SPDEC_CHECK_WORDS, dtype=torch.int32, device=cache.page_table.device)
    _need(report, "report", torch.int32, (SPDEC_CHECK_WORDS,))
    if q is not None:
        _need(q, "q", cache.dtype, (cache.batch, cache.num_q_heads, cache.head_dim))
    if sel_idx is not None:
        _need(sel_idx, "sel_idx", torch.int32, (cache.batch, cache.num_kv_heads, max_budget_pages))
    if sel_cnt is not None:
        _need(sel_cnt, "sel_cnt", torch.int32, (cache.batch, cache.num_kv_heads))
    if shared_pages is not None:
        if group_size < 1 or cache.batch % group_size:
            raise ValueError("group_size must divide the batch")
        _need(shared_pages, "shared_pages", torch.int32, (cache.batch // group_size,))
    _check(lib().spdec_check_inputs(ctypes.byref(cache.desc), _ptr(q), _ptr(sel_idx), _ptr(sel_cnt),
                                    max_budget_pages, group_size, _ptr(shared_pages), _ptr(report), _stream()),
           "spdec_check_inputs")
    vals = report.cpu().tolist()
    return dict(zip(CHECK_FIELDS, vals[:len(CHECK_FIELDS)]))
