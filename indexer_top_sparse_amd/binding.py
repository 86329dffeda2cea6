"""Thin ctypes binding of ``libsa.so`` (the C ABI declared in include/sa.h).

Argument marshalling only: every step of the path runs in the library's HIP kernels. PyTorch
provides device memory and the current stream. There is no fallback: if the library is not
built, or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsa.so")

SA_OK, SA_ERR_INVALID, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP = range(5)
SA_BF16, SA_FP8_E4M3, SA_MXFP8, SA_FP8_E4M3_T128 = 0, 1, 2, 3


class SaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"sa status {status}: {message}")
        self.status = status


class sa_batch(C.Structure):
    _fields_ = [("num_seqs", C.c_int32), ("page_size", C.c_int32),
                ("pages_per_seq", C.c_int32), ("num_pages", C.c_int32),
                ("page_table", C.c_void_p), ("ctx_lens", C.c_void_p),
                ("ctx_lens_host", C.c_void_p), ("q_indptr", C.c_void_p),
                ("q_indptr_host", C.c_void_p), ("reuse", C.c_void_p),
                ("reuse_host", C.c_void_p)]


class sa_indexer(C.Structure):
    _fields_ = [("heads", C.c_int32), ("dim", C.c_int32), ("key_dtype", C.c_int),
                ("keys", C.c_void_p), ("key_scale", C.c_void_p), ("pooled", C.c_void_p),
                ("key_mx_scale", C.c_void_p)]


class sa_prolog(C.Structure):
    _fields_ = [("heads", C.c_int32), ("dim", C.c_int32), ("d_q", C.c_int32),
                ("d_model", C.c_int32), ("w_q", C.c_void_p), ("w_k", C.c_void_p),
                ("w_w", C.c_void_p), ("ln_gamma", C.c_void_p), ("ln_beta", C.c_void_p),
                ("ln_eps", C.c_float)]


class sa_kv(C.Structure):
    _fields_ = [("heads_q", C.c_int32), ("heads_kv", C.c_int32), ("dim_qk", C.c_int32),
                ("dim_v", C.c_int32), ("dtype", C.c_int), ("k", C.c_void_p), ("v", C.c_void_p),
                ("scale", C.c_void_p), ("softmax_scale", C.c_float)]


_lib = None
EXPORTS = ("sa_index_score", "sa_topk", "sa_sparse_attn", "sa_index_select", "sa_block_select",
           "sa_decode_step", "sa_decode_step_noalloc", "sa_cache_append", "sa_indexer_prolog", "sa_prolog_workspace_size",
           "sa_workspace_size", "sa_pool_create", "sa_pool_destroy", "sa_pool_stats", "sa_seq_new",
           "sa_seq_fork", "sa_seq_reserve", "sa_seq_free", "sa_seq_len", "sa_seq_page_table",
           "sa_pool_refcount", "sa_copy_pages",
           "sa_workspace_init", "sa_workspace_error", "sa_plan_selection",
           "sa_plan_latent_attention", "sa_status_string", "sa_last_error",
           "sa_version")


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
    lib = C.CDLL(path)
    P, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    pb, pi, pk = C.POINTER(sa_batch), C.POINTER(sa_indexer), C.POINTER(sa_kv)
    lib.sa_index_score.argtypes = [pb, pi, P, P, P, i64, P]
    lib.sa_topk.argtypes = [pb, P, i64, i32, P, P, sz, P]
    lib.sa_sparse_attn.argtypes = [pb, pk, P, P, i32, P, P, sz, P]
    lib.sa_index_select.argtypes = [pb, pi, P, P, i32, i32, P, P, sz, P]
    lib.sa_block_select.argtypes = [pb, pi, P, P, i32, P, P, sz, P]
    lib.sa_decode_step.argtypes = [pb, pi, pk, P, P, P, i32, i32, P, P, P, sz, P]
    lib.sa_decode_step_noalloc.argtypes = [pb, pi, pk, P, P, P, i32, i32, P, P, P, P]
    lib.sa_cache_append.argtypes = [pb, pi, pk, P, P, P, P]
    lib.sa_indexer_prolog.argtypes = [C.POINTER(sa_prolog), i32, P, P, P, P, P, P, sz, P]
    lib.sa_prolog_workspace_size.argtypes = [C.POINTER(sa_prolog), i32]
    lib.sa_pool_create.argtypes = [i32, i32, i32]
    lib.sa_pool_create.restype = P
    lib.sa_pool_destroy.argtypes = [P]
    lib.sa_pool_destroy.restype = None
    ip = C.POINTER(C.c_int32)
    lib.sa_pool_stats.argtypes = [P, ip, ip, ip]
    lib.sa_seq_new.argtypes = [P]
    lib.sa_seq_fork.argtypes = [P, i32]
    lib.sa_seq_reserve.argtypes = [P, i32, i32, i32, ip, i32, ip]
    lib.sa_seq_free.argtypes = [P, i32]
    lib.sa_seq_len.argtypes = [P, i32]
    lib.sa_seq_page_table.argtypes = [P, i32, ip, i32, ip]
    lib.sa_pool_refcount.argtypes = [P, i32]
    lib.sa_copy_pages.argtypes = [pi, pk, i32, P, i32, P]
    for fn in ("sa_pool_stats", "sa_seq_new", "sa_seq_fork", "sa_seq_reserve", "sa_seq_free",
               "sa_seq_len", "sa_seq_page_table", "sa_pool_refcount", "sa_copy_pages"):
        getattr(lib, fn).restype = C.c_int
    lib.sa_prolog_workspace_size.restype = sz
    lib.sa_workspace_size.argtypes = [pb, pk, i32, i32]
    lib.sa_workspace_size.restype = sz
    lib.sa_workspace_init.argtypes = [P, sz, P]
    lib.sa_workspace_error.argtypes = [P, C.POINTER(C.c_int32), P]
    lib.sa_plan_selection.argtypes = [P, i32, i32, ip, C.POINTER(i64)]
    lib.sa_plan_latent_attention.argtypes = [i32, i32, i32, i32, i32, ip, ip, ip, ip, ip]
    lib.sa_plan_selection.restype = C.c_int
    lib.sa_plan_latent_attention.restype = C.c_int
    lib.sa_status_string.argtypes = [C.c_int]
    lib.sa_status_string.restype = C.c_char_p
    lib.sa_last_error.restype = C.c_char_p
    lib.sa_version.restype = i32
    for fn in ("sa_index_score", "sa_topk", "sa_sparse_attn", "sa_index_select", "sa_block_select",
               "sa_decode_step", "sa_decode_step_noalloc", "sa_cache_append", "sa_indexer_prolog", "sa_workspace_init",
               "sa_workspace_error"):
        getattr(lib, fn).restype = C.c_int
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != SA_OK:
        lib = load()
        msg = lib.sa_last_error().decode() or lib.sa_status_string(status).decode()
        raise SaError(status, msg)


def _ptr(t):
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


class Batch:
    """Page table, lengths and query rows of one call (device tensors + host copies)."""

    def __init__(self, page_table: torch.Tensor, ctx_lens: torch.Tensor, ctx_lens_host,
                 page_size: int, num_pages: int, q_indptr: torch.Tensor | None = None,
                 q_indptr_host=None, reuse: torch.Tensor | None = None, reuse_host=None):
        self._pt = page_table
        self._ctx = ctx_lens
        self._ctx_host = (C.c_int32 * len(ctx_lens_host))(*[int(x) for x in ctx_lens_host])
        self._qi = q_indptr
        self._qi_host = None
        if q_indptr is not None:
            self._qi_host = (C.c_int32 * len(q_indptr_host))(*[int(x) for x in q_indptr_host])
        self._reuse = reuse
        self._reuse_host = None
        if reuse is not None:
            self._reuse_host = (C.c_int32 * len(reuse_host))(*[int(x) for x in reuse_host])
        self.s = sa_batch(len(ctx_lens_host), page_size, page_table.shape[1], num_pages,
                          page_table.data_ptr(), ctx_lens.data_ptr(),
                          C.cast(self._ctx_host, C.c_void_p),
                          q_indptr.data_ptr() if q_indptr is not None else None,
                          C.cast(self._qi_host, C.c_void_p) if self._qi_host is not None
                          else None,
                          reuse.data_ptr() if reuse is not None else None,
                          C.cast(self._reuse_host, C.c_void_p) if self._reuse_host is not None
                          else None)


def indexer_desc(heads, dim, keys, key_scale=None, pooled=None, key_mx_scale=None):
    if key_mx_scale is not None:
        dt = SA_MXFP8
    else:
        dt = SA_FP8_E4M3 if key_scale is not None else SA_BF16
    return sa_indexer(heads, dim, dt, keys.data_ptr(),
                      key_scale.data_ptr() if key_scale is not None else None,
                      pooled.data_ptr() if pooled is not None else None,
                      key_mx_scale.data_ptr() if key_mx_scale is not None else None)


def kv_desc(heads_q, dim_qk, dim_v, k, v=None, scale=None, softmax_scale=1.0, heads_kv=1):
    """E4M3 rows when ``scale`` is given: one scale per row ([pages, P]) or one per 128-entry
    tile ([pages, P, heads_kv, tiles])."""
    dt = SA_BF16
    if scale is not None:
        dt = SA_FP8_E4M3_T128 if scale.dim() == 4 else SA_FP8_E4M3
    return sa_kv(heads_q, heads_kv, dim_qk, dim_v, dt, k.data_ptr(),
                 v.data_ptr() if v is not None else None,
                 scale.data_ptr() if scale is not None else None, float(softmax_scale))


def workspace_size(batch: Batch, kv: sa_kv | None, k: int, block_k: int = 0) -> int:
    lib = load()
    n = lib.sa_workspace_size(C.byref(batch.s), C.byref(kv) if kv is not None else None, k,
                              block_k)
    if n == 0:
        _check(SA_ERR_INVALID)
    return int(n)


def plan_selection(ncand, capacity: int):
    """(chunk, workgroups) of one fused-selection launch (host-only planning, no device)."""
    arr = (C.c_int32 * len(ncand))(*[int(x) for x in ncand])
    chunk, groups = C.c_int32(0), C.c_int64(0)
    _check(load().sa_plan_selection(C.cast(arr, C.c_void_p), len(ncand), int(capacity),
                                    C.byref(chunk), C.byref(groups)))
    return int(chunk.value), int(groups.value)


def plan_latent_attention(rows: int, k: int, heads_q: int, capacity: int, row_records: int):
    """(splits, split_len, head_groups, merge, grid) of the latent attention launch; splits = 0
    when the other attention kernel runs (host-only planning, no device)."""
    o = [C.c_int32(0) for _ in range(5)]
    _check(load().sa_plan_latent_attention(int(rows), int(k), int(heads_q), int(capacity),
                                           int(row_records), *[C.byref(x) for x in o]))
    return tuple(int(x.value) for x in o)


def workspace_init(ws: torch.Tensor, stream=None) -> None:
    _check(load().sa_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def workspace_error(ws: torch.Tensor, stream=None) -> int:
    v = C.c_int32(0)
    _check(load().sa_workspace_error(_ptr(ws), C.byref(v), _stream(stream)))
    return int(v.value)


def new_workspace(batch: Batch, kv: sa_kv | None, k: int, block_k: int = 0,
                  device="cuda") -> torch.Tensor:
    """Allocate (through torch) and zero-initialise a workspace for these shapes."""
    n = workspace_size(batch, kv, k, block_k)
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + n]
    workspace_init(ws)
    return ws


def index_score(batch: Batch, ix: sa_indexer, q_idx, w, scores, stream=None) -> None:
    _check(load().sa_index_score(C.byref(batch.s), C.byref(ix), _ptr(q_idx), _ptr(w),
                                 _ptr(scores), scores.shape[1], _stream(stream)))


def topk(batch: Batch, scores, k: int, idx, ws=None, stream=None) -> None:
    _check(load().sa_topk(C.byref(batch.s), _ptr(scores), scores.shape[1], k, _ptr(idx),
                          _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def sparse_attn(batch: Batch, kv: sa_kv, q, idx, out, ws, stream=None) -> None:
    _check(load().sa_sparse_attn(C.byref(batch.s), C.byref(kv), _ptr(q), _ptr(idx),
                                 idx.shape[1], _ptr(out), _ptr(ws), ws.numel(),
                                 _stream(stream)))


def index_select(batch: Batch, ix: sa_indexer, q_idx, w, k: int, idx_out, ws, block_k: int = 0,
                 stream=None) -> None:
    _check(load().sa_index_select(C.byref(batch.s), C.byref(ix), _ptr(q_idx), _ptr(w), k,
                                  block_k, _ptr(idx_out), _ptr(ws), ws.numel(), _stream(stream)))


def block_select(batch: Batch, ix: sa_indexer, q_idx, w, block_k: int, blocks_out, ws,
                 stream=None) -> None:
    _check(load().sa_block_select(C.byref(batch.s), C.byref(ix), _ptr(q_idx), _ptr(w), block_k,
                                  _ptr(blocks_out), _ptr(ws), ws.numel(), _stream(stream)))


def decode_step(batch: Batch, ix: sa_indexer, kv: sa_kv, q_idx, w, q, k: int, out, ws,
                block_k: int = 0, idx_out=None, stream=None) -> None:
    _check(load().sa_decode_step(C.byref(batch.s), C.byref(ix), C.byref(kv), _ptr(q_idx),
                                 _ptr(w), _ptr(q), k, block_k, _ptr(idx_out), _ptr(out),
                                 _ptr(ws), ws.numel(), _stream(stream)))


def decode_step_noalloc(batch: Batch, ix: sa_indexer, kv: sa_kv, q_idx, w, q, k: int, out,
                        block_k: int = 0, idx_out=None, error_out=None, stream=None) -> None:
    """sa_decode_step with the library's fixed scratch instead of a workspace; ``error_out`` (a
    device int32 tensor, or None) receives the call's device error word."""
    _check(load().sa_decode_step_noalloc(C.byref(batch.s), C.byref(ix), C.byref(kv), _ptr(q_idx),
                                         _ptr(w), _ptr(q), k, block_k, _ptr(idx_out), _ptr(out),
                                         _ptr(error_out), _stream(stream)))


def cache_append(batch: Batch, ix: sa_indexer | None, kv: sa_kv | None, k_idx_new=None,
                 kv_new=None, v_new=None, stream=None) -> None:
    """New token rows into the caches that ``ix`` and ``kv`` describe (see sa_cache_append)."""
    _check(load().sa_cache_append(C.byref(batch.s), C.byref(ix) if ix is not None else None,
                                  C.byref(kv) if kv is not None else None, _ptr(k_idx_new),
                                  _ptr(kv_new), _ptr(v_new), _stream(stream)))


def prolog_desc(heads, dim, w_q, w_k, w_w, gamma, beta, eps=1e-6) -> sa_prolog:
    return sa_prolog(heads, dim, w_q.shape[1], w_k.shape[1], w_q.data_ptr(), w_k.data_ptr(),
                     w_w.data_ptr(), gamma.data_ptr(), beta.data_ptr(), float(eps))


def prolog_workspace(p: sa_prolog, rows: int, device="cuda") -> torch.Tensor:
    n = load().sa_prolog_workspace_size(C.byref(p), rows)
    if n == 0:
        _check(SA_ERR_INVALID)
    return torch.empty(n, dtype=torch.uint8, device=device)


def indexer_prolog(p: sa_prolog, x_q, x, q_out, k_out, w_out, ws, stream=None) -> None:
    """q_I, k_I and w of x_q.shape[0] new tokens (see sa_indexer_prolog)."""
    _check(load().sa_indexer_prolog(C.byref(p), x_q.shape[0], _ptr(x_q), _ptr(x), _ptr(q_out),
                                    _ptr(k_out), _ptr(w_out), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)))


class Pool:
    """Host-side paged cache allocator (see sa_pool_create): page numbers for sequences, shared
    prefixes with copy-on-write, coalesced free runs and an emergency reserve."""

    def __init__(self, num_pages: int, page_size: int, emergency_pages: int = 0):
        self.lib = load()
        self.h = self.lib.sa_pool_create(num_pages, page_size, emergency_pages)
        if not self.h:
            raise SaError(SA_ERR_INVALID, "sa_pool_create rejected its arguments")
        self.num_pages, self.page_size = num_pages, page_size

    def __del__(self):
        if getattr(self, "h", None):
            self.lib.sa_pool_destroy(self.h)
            self.h = None

    def stats(self):
        f, r, m = C.c_int32(), C.c_int32(), C.c_int32()
        _check(self.lib.sa_pool_stats(self.h, C.byref(f), C.byref(r), C.byref(m)))
        return f.value, r.value, m.value

    def new(self) -> int:
        s = self.lib.sa_seq_new(self.h)
        if s < 0:
            raise SaError(SA_ERR_INVALID, "sa_seq_new failed")
        return s

    def fork(self, parent: int) -> int:
        s = self.lib.sa_seq_fork(self.h, parent)
        if s < 0:
            raise SaError(SA_ERR_INVALID, "sa_seq_fork failed")
        return s

    def reserve(self, seq: int, new_len: int, urgent: bool = False):
        """Grow to new_len tokens; returns the copy-on-write (src, dst) page pairs."""
        cp = (C.c_int32 * 2)()
        n = C.c_int32()
        _check(self.lib.sa_seq_reserve(self.h, seq, new_len, int(urgent), cp, 1, C.byref(n)))
        return [(cp[0], cp[1])] if n.value else []

    def free(self, seq: int) -> None:
        _check(self.lib.sa_seq_free(self.h, seq))

    def length(self, seq: int) -> int:
        return self.lib.sa_seq_len(self.h, seq)

    def page_table(self, seq: int):
        buf = (C.c_int32 * self.num_pages)()
        n = C.c_int32()
        _check(self.lib.sa_seq_page_table(self.h, seq, buf, self.num_pages, C.byref(n)))
        return list(buf[:n.value])

    def refcount(self, page: int) -> int:
        return self.lib.sa_pool_refcount(self.h, page)


def copy_pages(ix: sa_indexer | None, kv: sa_kv | None, page_size: int, pairs, stream=None) -> None:
    """Device copies of whole pages (pairs: device int32 [n, 2])."""
    _check(load().sa_copy_pages(C.byref(ix) if ix is not None else None,
                                C.byref(kv) if kv is not None else None, page_size,
                                _ptr(pairs), pairs.shape[0], _stream(stream)))
