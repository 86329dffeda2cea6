"""GPU parity of sa_cache_append against the CPU oracle: every cache byte after the append is
compared (bf16 rows, E4M3 and MXFP8 codes, fp32 scales, E8M0 exponents, bf16 block summaries
must be identical), then a decode step over the updated caches is checked against the oracle's
decode step over the oracle's updated caches.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from indexer_top_sparse_amd import binding, device, inputs
from tests._util import check_topk_row, output_error

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _new_rows(wl, seed):
    g = torch.Generator().manual_seed(seed)
    n = wl.num_queries
    k_idx = (torch.randn((n, wl.idx_dim), generator=g) * 3).to(torch.bfloat16)
    kv = torch.randn((n, wl.heads_kv, wl.dim_qk), generator=g).to(torch.bfloat16)
    v = None
    if wl.v_cache is not None:
        v = torch.randn((n, wl.heads_kv, wl.dim_v), generator=g).to(torch.bfloat16)
    return k_idx, kv, v


def _bits(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


NAMES = {"idx_keys": "idx_keys", "idx_scale": "idx_scale", "idx_mx_scale": "idx_mx_scale",
         "pooled": "pooled", "k_cache": "k_cache", "v_cache": "v_cache", "kv_scale": "kv_scale"}


def _append_on_gpu(wl, k_idx, kv, v):
    dw = device.to_device(wl)
    binding.cache_append(dw.batch, dw.ix, dw.kv, k_idx.cuda(), kv.cuda(),
                         v.cuda() if v is not None else None)
    torch.cuda.synchronize()
    return dw


@pytest.mark.parametrize("preset,over", [
    ("tiny", dict(num_seqs=3, ctx=[100, 64, 129])),
    ("decode32k", dict(num_seqs=4, ctx=[65, 300, 1, 0])),
    ("long1m", dict(num_seqs=2, ctx=[129, 4096], block_topk=4)),
    ("fp8ragged", dict(num_seqs=3, ctx=[4096, 5000, 4200])),
    ("mxfp8ragged", dict(num_seqs=2, ctx=[4100, 4500])),
    ("long1m", dict(num_seqs=1, ctx=200, q_len=70, block_topk=4)),
    ("decode32k", dict(num_seqs=2, ctx=[700, 130], q_len=[129, 3])),
])
def test_append_is_bit_exact(preset, over):
    wl = inputs.make(preset, **over)
    _say(f"cache append {preset} {over}")
    k_idx, kv, v = _new_rows(wl, 3)
    dw = _append_on_gpu(wl, k_idx, kv, v)
    want = oracle.cache_append(wl, k_idx, kv, v)
    for name, arr in want.items():
        if arr is None:
            continue
        got = _bits(dw.t[name])
        mism = int((got != arr).sum())
        assert mism == 0, f"{name}: {mism} entries differ"


def test_append_then_decode_sees_the_new_tokens():
    """Append each sequence's newest token on both sides, then decode over the updated caches:
    index sets under the near-tie rule and outputs within the fp8 bound."""
    wl = inputs.make("mxfp8ragged", num_seqs=3, ctx=[4100, 6000, 4500])
    k_idx, kv, v = _new_rows(wl, 11)
    dw = _append_on_gpu(wl, k_idx, kv, v)
    want = oracle.cache_append(wl, k_idx, kv, v)
    upd = dataclasses.replace(
        wl, idx_keys=torch.from_numpy(want["idx_keys"]),
        idx_mx_scale=torch.from_numpy(want["idx_mx_scale"]),
        k_cache=torch.from_numpy(want["k_cache"]), kv_scale=torch.from_numpy(want["kv_scale"]))
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    ref = oracle.decode_step(upd)
    got = idx.cpu().numpy()
    for b in range(upd.num_seqs):
        msg = check_topk_row(got[b], ref["idx"][b], ref["scores"][b], upd.ctx_lens[b], upd.topk)
        assert msg == "", f"seq {b}: {msg}"
    err, msg = output_error(out.float().cpu().numpy(), oracle.sparse_attn(upd, got), 5e-2)
    _say(f"  decode after append: max abs output error {err:.3e}")
    assert msg == "", msg


def test_append_rejects_summaries_over_fp8_keys():
    wl = inputs.make("fp8ragged", num_seqs=1, ctx=[4096])
    dw = device.to_device(wl)
    pooled = torch.zeros((wl.num_pages, wl.idx_dim), dtype=torch.bfloat16, device="cuda")
    ix = binding.indexer_desc(wl.idx_heads, wl.idx_dim, dw.t["idx_keys"], dw.t["idx_scale"], pooled)
    k_idx, _, _ = _new_rows(wl, 1)
    with pytest.raises(binding.SaError) as e:
        binding.cache_append(dw.batch, ix, None, k_idx.cuda())
    assert e.value.status == binding.SA_ERR_UNSUPPORTED
