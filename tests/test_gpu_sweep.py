"""A seeded sweep of decode configurations against the oracle.

Each case draws, from its own seed, a batch of 1 to 6 sequences with log-uniform context
lengths in [64, 40000) (about one in eight a stub of 1 to 8 tokens), a page size of 16, 64 or
128 tokens and K of 64, 300 or 2048. The index-key and cache format is one of four kinds: bf16
latent rows with 16, 64 or 128 query heads, the same with two-level selection (8, 32 or 64
blocks kept), E4M3 with row scales, or MXFP8 keys with 128-entry E4M3 tiles. Every case runs the fused decode step and is checked the
way the targeted tests check it: exact index sets up to near-ties at the threshold, and the
output against the oracle's attention over the GPU's own index set.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from indexer_top_sparse_amd import binding, device, inputs
from tests._util import check_topk_in, check_topk_row, output_error

pytestmark = pytest.mark.gpu

KINDS = ["bf16", "two_level", "fp8", "bf16", "mxfp8"]
PRESET = {"bf16": "decode32k", "two_level": "long1m", "fp8": "fp8ragged", "mxfp8": "mxfp8ragged"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _config(i):
    r = np.random.RandomState(5000 + i)
    kind = KINDS[i % len(KINDS)]
    B = int(r.randint(1, 7))
    # log-uniform lengths in [64, 40000); about one sequence in eight is a stub of 1 to 8 tokens
    ctx = [int(r.randint(1, 9)) if r.uniform() < 0.125 else
           int(np.exp(r.uniform(np.log(64.0), np.log(40000.0)))) for _ in range(B)]
    kw = dict(num_seqs=B, ctx=ctx, page_size=int(r.choice([16, 64, 128])),
              topk=int(r.choice([64, 300, 2048])))
    if kind in ("bf16", "two_level"):
        kw["heads_q"] = int(r.choice([16, 64, 128]))
    if kind == "two_level":
        kw["block_topk"] = int(r.choice([8, 32, 64]))
    return kind, kw


@pytest.mark.parametrize("i", range(15))
def test_decode_sweep(i):
    kind, kw = _config(i)
    wl = inputs.make(PRESET[kind], seed_offset=300 + i, **kw)
    print(f"sweep {i}: {kind} B={wl.num_seqs} ctx={wl.ctx_lens} page={wl.page_size} "
          f"K={wl.topk} heads_q={wl.heads_q} block_k={wl.block_topk}", flush=True)
    sys.stdout.flush()
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    blocks = device.block_select(dw, ws).cpu().numpy() if wl.block_topk else None
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    got = idx.cpu().numpy()
    P = wl.page_size
    if wl.block_topk:
        # blocks against the oracle's block scores; tokens against the oracle's fine stage on
        # the GPU's kept blocks (only their tokens are candidates, possibly fewer than K)
        bs = oracle.block_scores(wl)
        nblk = [-(-n // P) for n in wl.ctx_lens]
        ref_blocks = oracle.topk(bs, np.array(nblk), wl.block_topk)
        ref_tok = oracle.topk_in_blocks(wl, blocks, k=wl.topk)
        for b, n in enumerate(wl.ctx_lens):
            msg = check_topk_row(blocks[b], ref_blocks[b], bs[b], nblk[b], wl.block_topk)
            assert msg == "", f"seq {b} blocks: {msg}"
            cand = np.zeros(n, dtype=bool)
            for j in blocks[b][blocks[b] >= 0]:
                cand[j * P:min((j + 1) * P, n)] = True
            msg = check_topk_in(got[b], ref_tok[b], oracle.index_scores(wl, rows=[b])[0], cand,
                                wl.topk)
            assert msg == "", f"seq {b} tokens: {msg}"
    else:
        ref = oracle.decode_step(wl)
        for b, n in enumerate(wl.ctx_lens):
            msg = check_topk_row(got[b], ref["idx"][b], ref["scores"][b], n, wl.topk)
            assert msg == "", f"seq {b}: {msg}"
    tol = 2e-2 if kind in ("bf16", "two_level") else 5e-2
    err, msg = output_error(out.float().cpu().numpy(), oracle.sparse_attn(wl, got), tol)
    print(f"  max abs output error {err:.3e} (tol {tol})", flush=True)
    assert msg == "", msg
