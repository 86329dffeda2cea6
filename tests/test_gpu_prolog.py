"""GPU parity of sa_indexer_prolog (query, key and head-weight projections of new tokens, then
the key's LayerNorm) against the fp64 oracle.

Bounds, from the arithmetic: the GPU accumulates in fp32 (at most K * 2^-22 * sum_k |x_k W_nk|
off for a K-long contraction, a safe multiple of the unit roundoff) and rounds q_I and k_I to
bf16 (2^-9 relative, 2^-8 allowed). The key's error after the LayerNorm is its pre-norm error
scaled by |gamma| / sigma (twice, for the shift of the mean). A wrong index or a dropped term
moves entries by O(|value|), far outside these bounds.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from indexer_top_sparse_amd import binding, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _run(pi, rows, heads, dim):
    t = {k: getattr(pi, k).cuda().contiguous() for k in ("x_q", "x", "w_q", "w_k", "w_w", "gamma", "beta")}
    p = binding.prolog_desc(heads, dim, t["w_q"], t["w_k"], t["w_w"], t["gamma"], t["beta"], oracle.LN_EPS)
    q = torch.empty((rows, heads, dim), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((rows, dim), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((rows, heads), dtype=torch.float32, device="cuda")
    ws = binding.prolog_workspace(p, rows)
    binding.indexer_prolog(p, t["x_q"], t["x"], q, k, w, ws)
    torch.cuda.synchronize()
    return q.float().cpu().numpy().reshape(rows, -1), k.float().cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("rows,heads,dim,d_q,d_model", [
    (32, 64, 128, 1536, 7168),   # the decode batch of decode32k
    (5, 64, 128, 1536, 7168),    # a partial row tile
    (70, 12, 64, 256, 384),      # two row chunks, partial column tiles
    (1, 4, 64, 128, 128),
])
def test_prolog_matches_oracle(rows, heads, dim, d_q, d_model):
    print(f"prolog rows {rows} heads {heads} dim {dim} d_q {d_q} d_model {d_model}", flush=True)
    pi = inputs.make_prolog(rows, heads, dim, d_q, d_model, seed=rows)
    q, k, w = _run(pi, rows, heads, dim)
    rq, rk, rw = oracle.indexer_prolog(pi.x_q, pi.x, pi.w_q, pi.w_k, pi.w_w, pi.gamma, pi.beta)
    a = lambda t: np.abs(t.float().numpy().astype(np.float64))
    sq = a(pi.x_q) @ a(pi.w_q).T            # sum_k |x_k W_nk|
    sk = a(pi.x) @ a(pi.w_k).T
    sw = a(pi.x) @ a(pi.w_w).T
    acc = lambda K: K * 2.0 ** -22
    assert np.all(np.abs(q - rq) <= 2.0 ** -8 * np.abs(rq) + acc(d_q) * sq + 1e-30)
    assert np.all(np.abs(w - rw) <= acc(d_model) * sw + 1e-30)
    y = (a(pi.x) * np.sign(pi.x.float().numpy())) @ pi.w_k.float().numpy().T.astype(np.float64)
    sigma = np.sqrt(((y - y.mean(1, keepdims=True)) ** 2).mean(1, keepdims=True) + oracle.LN_EPS)
    gam = np.abs(pi.gamma.numpy().astype(np.float64))[None, :]
    dy = acc(d_model) * sk.max(axis=1, keepdims=True)
    bound = 2.0 ** -8 * np.abs(rk) + 2 * gam * dy / sigma + 1e-6
    err = np.abs(k - rk)
    print(f"  max err q {np.abs(q - rq).max():.2e} k {err.max():.2e} w {np.abs(w - rw).max():.2e}", flush=True)
    assert np.all(err <= bound)
