"""The failure path of the cross-workgroup waits, forced from the host.

SA_SPIN_LIMIT=0 lets every wait of the fused selection and of the latent attention's split
barrier expire after one poll; every kernel still runs to its end. Then each sequence's result
must be either the normal one or the defined failure result (every index -1, output 0; a group
of heads whose split barrier expired gets output 0), the
error word must say so, the per-sequence records must be back at zero, and the next call with
the normal limit must give the normal result on the same workspace.
"""
import os

import numpy as np
import pytest
import torch

from indexer_top_sparse_amd import binding as B
from indexer_top_sparse_amd import device, inputs

pytestmark = pytest.mark.gpu

SEL_RECORD = 256 + 3 * 2048 * 4  # counters, flag, padding and histograms of one record
SEL_BYTES = SEL_RECORD + 512 * 2 * 4 + 4096 * 8


def _say(msg):
    print(msg, flush=True)


class _SpinLimit:
    def __init__(self, v):
        self.v = v

    def __enter__(self):
        os.environ["SA_SPIN_LIMIT"] = str(self.v)

    def __exit__(self, *exc):
        os.environ.pop("SA_SPIN_LIMIT", None)


def _records_are_zero(ws, num_seqs, rows, stages=1):
    """Selection records (counters, flag, histograms; one per sequence and stage of the
    selection) and the merge records (one per row and head group, two head groups at most) are
    all zero."""
    h = ws.cpu().numpy()
    base = 256 + 2048
    for b in range(stages * num_seqs):
        rec = h[base + b * SEL_BYTES: base + b * SEL_BYTES + SEL_RECORD]
        if rec.any():
            return f"selection record {b} not zero"
    rs = (base + stages * num_seqs * SEL_BYTES + 255) // 256 * 256
    if h[rs: rs + 2 * rows * 64].any():
        return "merge records not zero"
    return ""


def test_expired_waits_give_the_defined_result_and_leave_the_workspace_clean():
    torch.cuda.set_device(0)
    wl = inputs.make("decode32k", num_seqs=8, seed_offset=41)
    _say("decode32k B=8: reference, forced failure, then normal again")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out_ref, idx_ref = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert B.workspace_error(ws) == 0
    out_ref, idx_ref = out_ref.cpu(), idx_ref.cpu()

    with _SpinLimit(0):
        out_f, idx_f = device.decode_step(dw, ws)
        torch.cuda.synchronize()
    err = B.workspace_error(ws)
    out_f, idx_f = out_f.cpu(), idx_f.cpu()
    failed = 0
    for b in range(wl.num_seqs):
        sel_failed = bool((idx_f[b] == -1).all())
        if not sel_failed:
            assert torch.equal(idx_f[b], idx_ref[b]), f"seq {b}: index set neither normal nor -1"
        zero = bool((out_f[b].float() == 0).all())
        if sel_failed:
            assert zero, f"seq {b}: selection failed but the output is not zero"
        # a row's heads merge in groups of 64 or 128: each 64-head block is zero or exact
        any_zero = False
        for h0 in range(0, wl.heads_q, 64):
            got, ref = out_f[b, h0:h0 + 64], out_ref[b, h0:h0 + 64]
            if bool((got.float() == 0).all()):
                any_zero = True
            else:
                assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), \
                    f"seq {b}, heads {h0}..: output neither normal nor zero"
        failed += sel_failed or any_zero
    _say(f"sequences with the failure result: {failed} of {wl.num_seqs}; error word {err}")
    assert failed > 0, "no wait expired with a spin limit of 0"
    assert err & 1
    msg = _records_are_zero(ws, wl.num_seqs, wl.num_seqs)
    assert msg == "", msg

    # the same workspace with the normal limit (its error word cleared by hand)
    ws[:4].zero_()
    out2, idx2 = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert B.workspace_error(ws) == 0
    assert torch.equal(idx2.cpu(), idx_ref)
    assert torch.equal(out2.cpu().view(torch.int16), out_ref.view(torch.int16))


def test_expired_split_barrier_in_attention_alone():
    """sa_sparse_attn on a given index set: head groups whose split barrier expired are all
    zero, the others exact, and the next normal call is exact again."""
    torch.cuda.set_device(0)
    wl = inputs.make("decode32k", num_seqs=8, seed_offset=43)
    _say("decode32k B=8: sparse attention with a forced barrier failure")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    idx = torch.empty((wl.num_seqs, wl.topk), dtype=torch.int32, device="cuda")
    device.index_select(dw, ws, idx=idx)
    out_ref = torch.empty((wl.num_seqs, wl.heads_q, wl.dim_v), dtype=torch.bfloat16, device="cuda")
    B.sparse_attn(dw.batch, dw.kv, dw.t["q"], idx, out_ref, ws)
    torch.cuda.synchronize()
    assert B.workspace_error(ws) == 0
    out_f = torch.full_like(out_ref, 1.0)
    with _SpinLimit(0):
        B.sparse_attn(dw.batch, dw.kv, dw.t["q"], idx, out_f, ws)
        torch.cuda.synchronize()
    err = B.workspace_error(ws)
    # a row's heads merge in groups of 64 (two head groups per row) or 128: each 64-head block
    # is either the failure result (all zero) or exact
    zero_blocks = 0
    for b in range(wl.num_seqs):
        for h0 in range(0, wl.heads_q, 64):
            got, ref = out_f[b, h0:h0 + 64], out_ref[b, h0:h0 + 64]
            if bool((got.float() == 0).all()):
                zero_blocks += 1
            else:
                assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (b, h0)
    _say(f"64-head blocks with the failure result: {zero_blocks}; error word {err}")
    assert zero_blocks > 0 and err & 1
    msg = _records_are_zero(ws, wl.num_seqs, wl.num_seqs)
    assert msg == "", msg
    ws[:4].zero_()
    out2 = torch.empty_like(out_ref)
    B.sparse_attn(dw.batch, dw.kv, dw.t["q"], idx, out2, ws)
    torch.cuda.synchronize()
    assert B.workspace_error(ws) == 0
    assert torch.equal(out2.view(torch.int16), out_ref.view(torch.int16))
    np.testing.assert_array_equal(idx.cpu().numpy()[:, :1] >= 0, True)


def test_expired_waits_in_the_two_stage_selection():
    """The fused block-then-token selection with every wait expiring: each sequence's index set
    is the normal one or all -1, the records of both stages return to zero, and the next call is
    exact."""
    torch.cuda.set_device(0)
    wl = inputs.make("long1m", num_seqs=2, ctx=[200000, 3000], seed_offset=47)
    _say("two-level B=2 block_k=512: reference, forced failure, then normal again")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out_ref, idx_ref = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert B.workspace_error(ws) == 0
    out_ref, idx_ref = out_ref.cpu(), idx_ref.cpu()
    with _SpinLimit(0):
        out_f, idx_f = device.decode_step(dw, ws)
        torch.cuda.synchronize()
    err = B.workspace_error(ws)
    out_f, idx_f = out_f.cpu(), idx_f.cpu()
    failed = 0
    for b in range(wl.num_seqs):
        sel_failed = bool((idx_f[b] == -1).all())
        if sel_failed:
            failed += 1
            assert bool((out_f[b].float() == 0).all()), f"seq {b}: failed selection, output not 0"
        else:
            assert torch.equal(idx_f[b], idx_ref[b]), f"seq {b}: index set neither normal nor -1"
    _say(f"sequences with the failure result: {failed} of {wl.num_seqs}; error word {err}")
    assert failed > 0 and err & 1
    msg = _records_are_zero(ws, wl.num_seqs, wl.num_seqs, stages=2)
    assert msg == "", msg
    ws[:4].zero_()
    out2, idx2 = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert B.workspace_error(ws) == 0
    assert torch.equal(idx2.cpu(), idx_ref)
    assert torch.equal(out2.cpu().view(torch.int16), out_ref.view(torch.int16))
