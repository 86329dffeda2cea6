"""Host-side checks of the C ABI: the library loads, exports every declared entry point, and
rejects invalid arguments before touching the device (these tests need no GPU)."""
import ctypes as C
import os
import re

import pytest
import torch

from indexer_top_sparse_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return B.load()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "sa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert "sa_decode_step" in names and len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(B.EXPORTS) == set(names)


def test_version_and_status_strings(lib):
    assert lib.sa_version() == 1
    for st in range(5):
        assert lib.sa_status_string(st)
    assert lib.sa_status_string(99) == b"unknown status"


class _FakeDev:
    """Host tensors standing in for device buffers: validation never dereferences them."""

    def __init__(self, B_=2, ctx=(100, 7), P=64, pages=4):
        self.pt = torch.zeros((B_, pages), dtype=torch.int32)
        self.ctx = torch.tensor(ctx, dtype=torch.int32)
        self.batch = B.Batch(self.pt, self.ctx, list(ctx), P, 8)
        self.keys = torch.zeros((8, P, 128), dtype=torch.bfloat16)
        self.kvc = torch.zeros((8, P, 576), dtype=torch.bfloat16)
        self.ix = B.indexer_desc(64, 128, self.keys)
        self.kv = B.kv_desc(128, 576, 512, self.kvc, softmax_scale=1 / 24)


def test_workspace_size_grows_with_batch(lib):
    a = _FakeDev()
    n1 = B.workspace_size(a.batch, a.kv, 2048)
    n2 = B.workspace_size(a.batch, a.kv, 4096)
    n3 = B.workspace_size(a.batch, a.kv, 2048, block_k=512)
    assert 0 < n1 < n2 and n1 < n3
    assert B.workspace_size(a.batch, None, 2048) < n1


def _decode(lib, a, **over):
    args = dict(batch=C.byref(a.batch.s), ix=C.byref(a.ix), kv=C.byref(a.kv),
                q_idx=C.c_void_p(a.keys.data_ptr()), w=C.c_void_p(a.keys.data_ptr()),
                q=C.c_void_p(a.kvc.data_ptr()), k=2048, block_k=0, idx=None,
                out=C.c_void_p(a.kvc.data_ptr()), ws=None, ws_bytes=0, stream=None)
    args.update(over)
    return lib.sa_decode_step(args["batch"], args["ix"], args["kv"], args["q_idx"], args["w"],
                              args["q"], args["k"], args["block_k"], args["idx"], args["out"],
                              args["ws"], args["ws_bytes"], args["stream"])


def test_invalid_arguments_are_rejected_on_the_host(lib):
    a = _FakeDev()
    assert _decode(lib, a, batch=None) == B.SA_ERR_INVALID
    assert _decode(lib, a, k=0) == B.SA_ERR_INVALID
    assert _decode(lib, a, q_idx=None) == B.SA_ERR_INVALID
    assert _decode(lib, a, block_k=64) == B.SA_ERR_INVALID  # no pooled summaries
    assert _decode(lib, a) == B.SA_ERR_WORKSPACE              # no workspace
    # unsupported shapes
    bad = B.kv_desc(128, 320, 256, a.kvc, softmax_scale=0.1)
    assert _decode(lib, a, kv=C.byref(bad)) == B.SA_ERR_UNSUPPORTED
    bad = B.indexer_desc(65, 128, a.keys)
    assert _decode(lib, a, ix=C.byref(bad)) == B.SA_ERR_UNSUPPORTED
    bad = B.kv_desc(128, 576, 512, a.kvc, softmax_scale=0.0)
    assert _decode(lib, a, kv=C.byref(bad)) == B.SA_ERR_INVALID
    # two-level selection needs bf16 keys: E4M3 keys with summaries are rejected before any launch
    codes = torch.zeros((8, 64, 128), dtype=torch.uint8)
    scale = torch.ones((8, 64), dtype=torch.float32)
    pooled = torch.zeros((8, 128), dtype=torch.bfloat16)
    e4 = B.indexer_desc(64, 128, codes, key_scale=scale, pooled=pooled)
    assert _decode(lib, a, ix=C.byref(e4), block_k=2) == B.SA_ERR_UNSUPPORTED
    assert b"bf16 indexer keys" in lib.sa_last_error()
    bf = B.indexer_desc(64, 128, a.keys, pooled=pooled)
    assert _decode(lib, a, ix=C.byref(bf), block_k=2) == B.SA_ERR_WORKSPACE  # accepted, no workspace
    # context longer than the page table can address
    b2 = B.Batch(a.pt, a.ctx, [100, 257], 64, 8)
    assert _decode(lib, a, batch=C.byref(b2.s)) == B.SA_ERR_INVALID
    # page size must be a power of two
    b3 = B.Batch(a.pt, a.ctx, [100, 7], 48, 8)
    assert _decode(lib, a, batch=C.byref(b3.s)) == B.SA_ERR_INVALID
    # decode takes one row per sequence
    qi = torch.tensor([0, 1, 2], dtype=torch.int32)
    b4 = B.Batch(a.pt, a.ctx, [100, 7], 64, 8, qi, [0, 1, 2])
    assert _decode(lib, a, batch=C.byref(b4.s)) == B.SA_ERR_INVALID
    assert b"q_indptr" in lib.sa_last_error()


def test_index_score_and_topk_validation(lib):
    a = _FakeDev()
    sc = torch.zeros((2, 100), dtype=torch.float32)
    P = C.c_void_p
    # ld smaller than the longest visible row
    st = lib.sa_index_score(C.byref(a.batch.s), C.byref(a.ix), P(a.keys.data_ptr()),
                            P(sc.data_ptr()), P(sc.data_ptr()), 50, None)
    assert st == B.SA_ERR_INVALID
    st = lib.sa_topk(C.byref(a.batch.s), P(sc.data_ptr()), 100, 0, P(sc.data_ptr()), None, 0,
                     None)
    assert st == B.SA_ERR_INVALID
    # misaligned indexer queries
    st = lib.sa_index_score(C.byref(a.batch.s), C.byref(a.ix), P(a.keys.data_ptr() + 2),
                            P(sc.data_ptr()), P(sc.data_ptr()), 100, None)
    assert st == B.SA_ERR_INVALID


def test_sparse_attn_needs_a_large_enough_workspace(lib):
    a = _FakeDev()
    need = B.workspace_size(a.batch, a.kv, 2048)
    ws = torch.zeros(need + 512, dtype=torch.uint8)
    base = ws.data_ptr() + ((-ws.data_ptr()) % 256)
    idx = torch.zeros((2, 2048), dtype=torch.int32)
    P = C.c_void_p
    st = lib.sa_sparse_attn(C.byref(a.batch.s), C.byref(a.kv), P(a.kvc.data_ptr()),
                            P(idx.data_ptr()), 2048, P(a.kvc.data_ptr()), P(base), need - 256,
                            None)
    assert st == B.SA_ERR_WORKSPACE
    st = lib.sa_sparse_attn(C.byref(a.batch.s), C.byref(a.kv), P(a.kvc.data_ptr()),
                            P(idx.data_ptr()), 2048, P(a.kvc.data_ptr()), P(base + 16), need,
                            None)
    assert st == B.SA_ERR_WORKSPACE  # not 256-byte aligned


def test_cache_append_validation(lib):
    a = _FakeDev()
    P = C.c_void_p
    new = torch.zeros((2, 576), dtype=torch.bfloat16)

    def app(ix=None, kv=None, k_idx=None, kv_new=None, v_new=None, batch=None):
        return lib.sa_cache_append(batch or C.byref(a.batch.s), ix, kv, k_idx, kv_new, v_new, None)

    # V rows for a latent cache (no separate V)
    assert app(kv=C.byref(a.kv), kv_new=P(new.data_ptr()), v_new=P(new.data_ptr())) == B.SA_ERR_INVALID
    # V rows without KV rows
    assert app(v_new=P(new.data_ptr())) == B.SA_ERR_INVALID
    # misaligned new rows
    assert app(kv=C.byref(a.kv), kv_new=P(new.data_ptr() + 2)) == B.SA_ERR_INVALID
    # indexer rows without a descriptor
    assert app(k_idx=P(new.data_ptr())) == B.SA_ERR_INVALID
    # block summaries are defined over bf16 keys only
    codes = torch.zeros((8, 64, 128), dtype=torch.uint8)
    scale = torch.ones((8, 64), dtype=torch.float32)
    pooled = torch.zeros((8, 128), dtype=torch.bfloat16)
    ix = B.indexer_desc(64, 128, codes, scale, pooled)
    assert app(ix=C.byref(ix), k_idx=P(new.data_ptr())) == B.SA_ERR_UNSUPPORTED
    # nothing to write is not an error
    assert app() == B.SA_OK


def test_prolog_validation(lib):
    z = torch.zeros(4096, dtype=torch.float32)
    P = C.c_void_p(z.data_ptr())

    def prolog(heads=4, dim=64, d_q=128, d_model=128, eps=1e-6, rows=2, ws=4096 * 4, x=P):
        p = B.sa_prolog(heads, dim, d_q, d_model, z.data_ptr(), z.data_ptr(), z.data_ptr(),
                        z.data_ptr(), z.data_ptr(), eps)
        return lib.sa_indexer_prolog(C.byref(p), rows, x, P, P, P, P, P, ws, None)

    assert prolog(dim=96) == B.SA_ERR_UNSUPPORTED
    assert prolog(d_q=100) == B.SA_ERR_UNSUPPORTED
    assert prolog(heads=65) == B.SA_ERR_UNSUPPORTED
    assert prolog(rows=0) == B.SA_ERR_INVALID
    assert prolog(eps=0.0) == B.SA_ERR_INVALID
    assert prolog(x=None) == B.SA_ERR_INVALID
    assert prolog(ws=100) == B.SA_ERR_WORKSPACE
    p = B.sa_prolog(4, 64, 128, 7168, 0, 0, 0, 0, 0, 1e-6)
    assert lib.sa_prolog_workspace_size(C.byref(p), 3) == 4 * 3 * (64 + 4) * 14


def _decode_noalloc(lib, a, k=2048):
    P = C.c_void_p
    return lib.sa_decode_step_noalloc(C.byref(a.batch.s), C.byref(a.ix), C.byref(a.kv),
                                      P(a.keys.data_ptr()), P(a.keys.data_ptr()),
                                      P(a.kvc.data_ptr()), k, 0, None, P(a.kvc.data_ptr()), None,
                                      None)


def test_noalloc_limits_are_checked_on_the_host(lib):
    """The fixed-scratch decode step refuses calls beyond its scratch before any device call."""
    a = _FakeDev(B_=65, ctx=[7] * 65)
    assert _decode_noalloc(lib, a) == B.SA_ERR_UNSUPPORTED
    assert b"64 sequences" in lib.sa_last_error()
    # 64 sequences with k = 65536 need far more than 48 MiB of partials and index sets
    a = _FakeDev(B_=64, ctx=[7] * 64)
    assert _decode_noalloc(lib, a, k=65536) == B.SA_ERR_UNSUPPORTED
    assert b"48 MiB" in lib.sa_last_error()
    # argument checks come first, as for sa_decode_step
    assert _decode_noalloc(lib, a, k=0) == B.SA_ERR_INVALID


def test_selection_reuse_is_validated_on_the_host(lib):
    """sa_batch.reuse: -1 or an earlier sequence that selects itself, of the same length."""
    a = _FakeDev(B_=3, ctx=[100, 7, 100])

    def with_reuse(r):
        t = torch.tensor(r, dtype=torch.int32)
        return B.Batch(a.pt, a.ctx, [100, 7, 100], 64, 8, reuse=t, reuse_host=r)

    for bad in ([-1, 2, -1],   # names a later sequence
                [-1, -1, 2],   # names itself
                [-1, 0, -1],   # different lengths (100 and 7)
                [-1, -1, -2]):
        b = with_reuse(bad)
        assert _decode(lib, a, batch=C.byref(b.s)) == B.SA_ERR_INVALID, bad
        assert b"reuse" in lib.sa_last_error()
    a2 = _FakeDev(B_=3, ctx=[100, 100, 100])
    t = torch.tensor([-1, 0, 1], dtype=torch.int32)  # 2 names 1, which itself reuses 0
    b = B.Batch(a2.pt, a2.ctx, [100, 100, 100], 64, 8, reuse=t, reuse_host=[-1, 0, 1])
    assert _decode(lib, a2, batch=C.byref(b.s)) == B.SA_ERR_INVALID
    # a valid reuse passes validation (the call then stops at the missing workspace)
    b = with_reuse([-1, -1, 0])
    assert _decode(lib, a, batch=C.byref(b.s)) == B.SA_ERR_WORKSPACE
    # one of the two pointers alone
    b = with_reuse([-1, -1, 0])
    b.s.reuse_host = None
    assert _decode(lib, a, batch=C.byref(b.s)) == B.SA_ERR_INVALID
