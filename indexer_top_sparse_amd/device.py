"""Move a generated workload to the GPU and call the library on it (marshalling only)."""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as B


@dataclass
class DeviceWorkload:
    wl: object
    batch: B.Batch
    ix: B.sa_indexer
    kv: B.sa_kv
    t: dict  # device tensors kept alive


def to_device(wl, device="cuda", prefill: bool | None = None) -> DeviceWorkload:
    """Copy a Workload's tensors to ``device`` and build the ABI descriptors."""
    dev = torch.device(device)
    prefill = any(n != 1 for n in wl.q_lens) if prefill is None else prefill
    t = {}

    def put(name, x):
        if x is None:
            return None
        t[name] = x.to(dev).contiguous()
        return t[name]

    put("page_table", wl.page_table)
    put("ctx_lens", torch.tensor(wl.ctx_lens, dtype=torch.int32))
    if prefill:
        put("q_indptr", wl.q_indptr())
    put("q_idx", wl.q_idx)
    put("w", wl.w)
    put("idx_keys", wl.idx_keys)
    put("idx_scale", wl.idx_scale)
    put("idx_mx_scale", getattr(wl, "idx_mx_scale", None))
    put("pooled", wl.pooled)
    put("q", wl.q)
    put("k_cache", wl.k_cache)
    put("v_cache", wl.v_cache)
    put("kv_scale", wl.kv_scale)
    batch = B.Batch(t["page_table"], t["ctx_lens"], wl.ctx_lens, wl.page_size, wl.num_pages,
                    t.get("q_indptr"), wl.q_indptr().tolist() if prefill else None)
    ix = B.indexer_desc(wl.idx_heads, wl.idx_dim, t["idx_keys"], t.get("idx_scale"),
                        t.get("pooled"), t.get("idx_mx_scale"))
    kv = B.kv_desc(wl.heads_q, wl.dim_qk, wl.dim_v, t["k_cache"], t.get("v_cache"),
                   t.get("kv_scale"), wl.softmax_scale, wl.heads_kv)
    return DeviceWorkload(wl, batch, ix, kv, t)


def new_workspace(dw: DeviceWorkload, k=None, block_k=None):
    k = dw.wl.topk if k is None else k
    block_k = dw.wl.block_topk if block_k is None else block_k
    return B.new_workspace(dw.batch, dw.kv, k, block_k, device=dw.t["q"].device)


def index_score(dw: DeviceWorkload, ncols=None):
    rows = dw.wl.num_queries
    ncols = ncols or max(dw.wl.ctx_lens)
    scores = torch.empty((rows, max(ncols, 1)), dtype=torch.float32, device=dw.t["q"].device)
    B.index_score(dw.batch, dw.ix, dw.t["q_idx"], dw.t["w"], scores)
    return scores


def topk(dw: DeviceWorkload, scores, k=None):
    k = dw.wl.topk if k is None else k
    idx = torch.empty((scores.shape[0], k), dtype=torch.int32, device=scores.device)
    B.topk(dw.batch, scores, k, idx)
    return idx


def sparse_attn(dw: DeviceWorkload, idx, ws):
    rows = dw.wl.num_queries
    out = torch.empty((rows, dw.wl.heads_q, dw.wl.dim_v), dtype=torch.bfloat16,
                      device=dw.t["q"].device)
    B.sparse_attn(dw.batch, dw.kv, dw.t["q"], idx, out, ws)
    return out


def index_select(dw: DeviceWorkload, ws, idx=None):
    wl = dw.wl
    if idx is None:
        idx = torch.empty((wl.num_seqs, wl.topk), dtype=torch.int32, device=dw.t["q"].device)
    B.index_select(dw.batch, dw.ix, dw.t["q_idx"], dw.t["w"], wl.topk, idx, ws,
                   block_k=wl.block_topk)
    return idx


def block_select(dw: DeviceWorkload, ws, blocks=None):
    wl = dw.wl
    if blocks is None:
        blocks = torch.empty((wl.num_seqs, wl.block_topk), dtype=torch.int32,
                             device=dw.t["q"].device)
    B.block_select(dw.batch, dw.ix, dw.t["q_idx"], dw.t["w"], wl.block_topk, blocks, ws)
    return blocks


def decode_step(dw: DeviceWorkload, ws, want_idx=True, out=None, idx=None):
    wl = dw.wl
    dev = dw.t["q"].device
    if out is None:
        out = torch.empty((wl.num_seqs, wl.heads_q, wl.dim_v), dtype=torch.bfloat16, device=dev)
    if want_idx and idx is None:
        idx = torch.empty((wl.num_seqs, wl.topk), dtype=torch.int32, device=dev)
    B.decode_step(dw.batch, dw.ix, dw.kv, dw.t["q_idx"], dw.t["w"], dw.t["q"], wl.topk, out, ws,
                  block_k=wl.block_topk, idx_out=idx if want_idx else None)
    return out, idx
