"""A seeded sweep of prefill calls (scores, row Top-K, attention) against the oracle.

Each case draws, from its own seed, 1 to 3 sequences with log-uniform context lengths in
[256, 60000) and 0 to 40 new query rows each (the rows are the last positions of their
sequence), a page size of 16, 64 or 128 tokens and K of 64, 300 or 2048. The cache format is
bf16 latent rows with 16, 64 or 128 query heads, E4M3 keys and rows with row scales, or bf16
keys with E4M3 rows scaled per 128-entry tile. Scores are checked against the oracle on the
same codes, the row Top-K exactly on the GPU's own scores (rows of 8192 or more positions with
K at most an eighth of them take the one-read kernel, the rest the streaming one), and the
attention against the oracle over the GPU's index set. The score rows' stride is the longest
context, so both the 16-byte and the 4-byte loads of the one-read kernel occur.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from indexer_top_sparse_amd import binding, device, inputs
from tests._util import output_error

pytestmark = pytest.mark.gpu

DTYPES = ["bf16", "fp8", "bf16", "fp8t128"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _config(i):
    r = np.random.RandomState(7000 + i)
    dtype = DTYPES[i % len(DTYPES)]
    B = int(r.randint(1, 4))
    ctx = [int(np.exp(r.uniform(np.log(256.0), np.log(60000.0)))) for _ in range(B)]
    q_len = [int(r.randint(0, min(40, n) + 1)) for n in ctx]
    if sum(q_len) == 0:
        q_len[0] = 1
    kw = dict(num_seqs=B, ctx=ctx, q_len=q_len, page_size=int(r.choice([16, 64, 128])),
              topk=int(r.choice([64, 300, 2048])), dtype=dtype)
    if dtype == "bf16":
        kw["heads_q"] = int(r.choice([16, 64, 128]))
    return kw


@pytest.mark.parametrize("i", range(10))
def test_prefill_sweep(i):
    kw = _config(i)
    wl = inputs.make("prefill64k", seed_offset=400 + i, **kw)
    print(f"prefill sweep {i}: {kw['dtype']} ctx={wl.ctx_lens} rows={wl.q_lens} "
          f"page={wl.page_size} K={wl.topk} heads_q={wl.heads_q}", flush=True)
    sys.stdout.flush()
    dw = device.to_device(wl)
    s = device.index_score(dw).cpu().numpy()
    ref_s = oracle.index_scores(wl, ncols=s.shape[1])
    pos = wl.q_pos().numpy()
    for r in range(wl.num_queries):
        n = pos[r] + 1
        err = np.abs(s[r, :n] - ref_s[r, :n]).max()
        assert err <= 1e-4 * np.abs(ref_s[r, :n]).max(), (r, err)
        assert np.all(np.isneginf(s[r, n:])), r
    idx = device.topk(dw, torch.from_numpy(s).cuda()).cpu().numpy()
    np.testing.assert_array_equal(idx, oracle.topk(s.astype(np.float64), pos + 1, wl.topk))
    ws = device.new_workspace(dw)
    out = device.sparse_attn(dw, torch.from_numpy(idx).cuda(), ws).float().cpu().numpy()
    tol = 2e-2 if kw["dtype"] == "bf16" else 5e-2
    err, msg = output_error(out, oracle.sparse_attn(wl, idx), tol)
    print(f"  attention max abs error {err:.3e} (tol {tol})", flush=True)
    assert msg == "", msg
