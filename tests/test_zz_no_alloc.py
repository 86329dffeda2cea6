"""sa_decode_step_noalloc (the decode step on the library's fixed scratch, for callers that
cannot allocate) against sa_decode_step on a caller's workspace.

Both run the same kernels, so every index set and every output must be identical. The calls
run back to back on one device, so each one finds the scratch as the previous call left it:
the second call is smaller than the first, and later ones grow again and change the path
(two-level selection, E4M3 rows through the other attention kernel, the 64-sequence maximum).
"""
import numpy as np
import pytest
import torch

from indexer_top_sparse_amd import binding as B
from indexer_top_sparse_amd import device, inputs

pytestmark = pytest.mark.gpu

# (name, preset, overrides): consecutive calls, in this order
CALLS = [
    ("decode32k B=32 ctx=32768", "decode32k", {}),
    ("decode32k B=5 ragged", "decode32k", dict(num_seqs=5, ctx=[5000, 1, 0, 2049, 40000])),
    ("two-level B=2 block_k=512", "long1m", dict(num_seqs=2, ctx=[200000, 3000])),
    ("E4M3 rows B=64 ragged", "fp8ragged", dict(ctx_lo=64, ctx_hi=8192)),
    ("decode32k B=3 without idx_out", "decode32k", dict(num_seqs=3, ctx=[70000, 640, 2048])),
]


def _say(msg):
    print(msg, flush=True)


def test_noalloc_matches_the_workspace_entry_point():
    torch.cuda.set_device(0)
    err = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    for i, (name, preset, over) in enumerate(CALLS):
        _say(f"call {i}: {name}")
        wl = inputs.make(preset, seed_offset=100 + i, **over)
        dw = device.to_device(wl)
        want_idx = "without idx_out" not in name
        # the ordinary entry point on a fresh workspace
        ws = device.new_workspace(dw)
        out_ref, idx_ref = device.decode_step(dw, ws, want_idx=want_idx)
        # the scratch entry point
        out = torch.full_like(out_ref, float("nan"))
        idx = torch.full_like(idx_ref, -5) if want_idx else None
        err.fill_(-7)
        B.decode_step_noalloc(dw.batch, dw.ix, dw.kv, dw.t["q_idx"], dw.t["w"], dw.t["q"],
                              wl.topk, out, block_k=wl.block_topk, idx_out=idx, error_out=err)
        torch.cuda.synchronize()
        assert B.workspace_error(ws) == 0
        assert int(err.item()) == 0, f"{name}: device error word {int(err.item())}"
        if want_idx:
            np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref.cpu().numpy(), err_msg=name)
        a = out.view(torch.int16).cpu().numpy()
        b = out_ref.view(torch.int16).cpu().numpy()
        assert np.array_equal(a, b), f"{name}: {np.count_nonzero(a != b)} output entries differ"
        del dw, ws


def test_noalloc_rejects_calls_beyond_the_scratch():
    torch.cuda.set_device(0)
    wl = inputs.make("decode32k", num_seqs=65, ctx=64)
    dw = device.to_device(wl)
    out = torch.empty((65, wl.heads_q, wl.dim_v), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.SaError) as e:
        B.decode_step_noalloc(dw.batch, dw.ix, dw.kv, dw.t["q_idx"], dw.t["w"], dw.t["q"],
                              wl.topk, out)
    assert e.value.status == B.SA_ERR_UNSUPPORTED and "64 sequences" in str(e.value)
    wl = inputs.make("decode32k", num_seqs=64, ctx=64)
    dw = device.to_device(wl)
    out = torch.empty((64, wl.heads_q, wl.dim_v), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.SaError) as e:
        B.decode_step_noalloc(dw.batch, dw.ix, dw.kv, dw.t["q_idx"], dw.t["w"], dw.t["q"],
                              65536, out)
    assert e.value.status == B.SA_ERR_UNSUPPORTED and "48 MiB" in str(e.value)
