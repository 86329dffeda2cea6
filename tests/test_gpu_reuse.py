"""Selection reuse for requests that share a history ("How the Ascend Computing Platform
Achieves Same-Day Inference Adaptation for Ultra-Large Sparse Models" §3.1: requests sharing a
history prefix can reuse selection results).

Sequences that reuse another's selection read the same pages and carry the same indexer query
and head weights as the sequence they name (and the same attention query), so every result must
be identical with and without reuse; the reusing sequences' own workgroups are simply not
launched. Checked for the single-level and the two-level fused selection and for the decode
step on the fixed scratch, and against the oracle's index sets."""
import numpy as np
import pytest
import torch

import oracle
from indexer_top_sparse_amd import binding as B
from indexer_top_sparse_amd import device, inputs
from tests._util import check_topk_row

pytestmark = pytest.mark.gpu

# sequence -> the earlier sequence whose selection it reuses (-1: its own)
REUSE = [-1, -1, 0, -1, 1, 0]


def _say(msg):
    print(msg, flush=True)


def _shared_history(wl, reuse):
    """Make each reusing sequence read its source's pages with its source's queries."""
    for s, r in enumerate(reuse):
        if r < 0:
            continue
        assert wl.ctx_lens[s] == wl.ctx_lens[r]
        wl.page_table[s] = wl.page_table[r]
        for name in ("q_idx", "w", "q"):
            getattr(wl, name)[s] = getattr(wl, name)[r]
    return wl


def _with_reuse(dw, reuse):
    t = dw.t
    t["reuse"] = torch.tensor(reuse, dtype=torch.int32, device=t["q"].device)
    return B.Batch(t["page_table"], t["ctx_lens"], dw.wl.ctx_lens, dw.wl.page_size,
                   dw.wl.num_pages, reuse=t["reuse"], reuse_host=reuse)


@pytest.mark.parametrize("preset,ctx", [("decode32k", [3000, 5000, 3000, 700, 5000, 3000]),
                                        ("long1m", [100000, 40000, 100000, 3000, 40000, 100000])])
def test_reuse_gives_the_same_results(preset, ctx):
    torch.cuda.set_device(0)
    wl = _shared_history(inputs.make(preset, num_seqs=len(ctx), ctx=ctx, seed_offset=61), REUSE)
    _say(f"{preset} ctx={ctx} reuse={REUSE}")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out_ref, idx_ref = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert B.workspace_error(ws) == 0
    batch = _with_reuse(dw, REUSE)
    out = torch.full_like(out_ref, float("nan"))
    idx = torch.full_like(idx_ref, -7)
    B.decode_step(batch, dw.ix, dw.kv, dw.t["q_idx"], dw.t["w"], dw.t["q"], wl.topk, out, ws,
                  block_k=wl.block_topk, idx_out=idx)
    torch.cuda.synchronize()
    assert B.workspace_error(ws) == 0
    assert torch.equal(idx, idx_ref)
    assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16))
    # the fixed scratch path with the same reuse
    out2 = torch.full_like(out_ref, float("nan"))
    B.decode_step_noalloc(batch, dw.ix, dw.kv, dw.t["q_idx"], dw.t["w"], dw.t["q"], wl.topk, out2,
                          block_k=wl.block_topk)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out_ref.view(torch.int16))
    # and the index sets against the oracle (single level: every row)
    if not wl.block_topk:
        ref = oracle.decode_step(wl)
        got = idx.cpu().numpy()
        for b in range(wl.num_seqs):
            msg = check_topk_row(got[b], ref["idx"][b], ref["scores"][b], wl.ctx_lens[b], wl.topk)
            assert msg == "", f"seq {b}: {msg}"


def test_reuse_in_block_select_and_index_select():
    torch.cuda.set_device(0)
    ctx = [100000, 40000, 100000, 3000, 40000, 100000]
    wl = _shared_history(inputs.make("long1m", num_seqs=len(ctx), ctx=ctx, seed_offset=63), REUSE)
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    batch = _with_reuse(dw, REUSE)
    for bt in (dw.batch, batch):
        blocks = torch.full((wl.num_seqs, wl.block_topk), -7, dtype=torch.int32, device="cuda")
        B.block_select(bt, dw.ix, dw.t["q_idx"], dw.t["w"], wl.block_topk, blocks, ws)
        idx = torch.full((wl.num_seqs, wl.topk), -7, dtype=torch.int32, device="cuda")
        B.index_select(bt, dw.ix, dw.t["q_idx"], dw.t["w"], wl.topk, idx, ws,
                       block_k=wl.block_topk)
        torch.cuda.synchronize()
        if bt is dw.batch:
            blocks_ref, idx_ref = blocks.clone(), idx.clone()
    assert torch.equal(blocks, blocks_ref)
    assert torch.equal(idx, idx_ref)
    for s, r in enumerate(REUSE):
        if r >= 0:
            assert torch.equal(idx[s], idx[r])
