"""A seeded sweep of the row Top-K (sa_topk) over adversarial score rows, against the oracle.

Each case draws, from its own seed, 4 to 24 rows whose visible lengths mix short rows (1 to
8191 positions: the streaming selection) and long ones (8192 to 65536: the one-read kernel
while K is at most an eighth of the row), a row stride of the longest row rounded up to a
multiple of four or plus 0 to 3 (16-byte and 4-byte loads), and K from 1 to 8192 (above a
row's length the rest is -1). Every row takes one of these score patterns: N(0, 1); small
integers (heavy ties); one constant; a mix of +0 and -0; a rising or a falling ramp; a rising
trend with noise (large scores in one region); N(0, 1) with -inf at random positions; values
spread over the whole float range (subnormals to 1.7e38, both signs). Index sets are integer
results, so they must equal the oracle's exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from indexer_top_sparse_amd import binding

pytestmark = pytest.mark.gpu

KS = [1, 17, 256, 2048, 2049, 4000, 8192]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _row(r, kind, n):
    if kind == 0:
        return r.standard_normal(n)
    if kind == 1:
        return r.integers(-4, 4, n).astype(np.float64)
    if kind == 2:
        return np.full(n, 0.75)
    if kind == 3:
        return np.where(r.random(n) < 0.5, 0.0, -0.0)
    if kind == 4:
        return np.linspace(-1.0, 1.0, n)
    if kind == 5:
        return np.linspace(1.0, -1.0, n)
    if kind == 6:
        return np.linspace(0.0, 6.0, n) + r.standard_normal(n)
    if kind == 7:
        x = r.standard_normal(n)
        x[r.random(n) < 0.3] = -np.inf
        return x
    e = r.uniform(-140.0, 127.0, n)
    return np.where(r.random(n) < 0.5, 1.0, -1.0) * np.exp2(e)


def _case(i):
    r = np.random.default_rng(9000 + i)
    R = int(r.integers(4, 25))
    n = [int(r.integers(1, 8192)) if r.random() < 0.4 else int(r.integers(8192, 65537))
         for _ in range(R)]
    # even cases: a stride that is a multiple of four (16-byte loads); odd: the longest row plus
    # 0 to 3 (mostly 4-byte loads; past 65536 the whole call takes the streaming selection)
    ld = (max(n) + 3) // 4 * 4 if i % 2 == 0 else max(n) + int(r.integers(0, 4))
    k = int(r.choice(KS))
    s = np.full((R, ld), -np.inf, dtype=np.float32)
    kinds = r.integers(0, 9, R)
    for j in range(R):
        s[j, :n[j]] = _row(r, int(kinds[j]), n[j]).astype(np.float32)
    return n, ld, k, s, kinds


@pytest.mark.parametrize("i", range(12))
def test_topk_sweep(i):
    n, ld, k, s, kinds = _case(i)
    print(f"topk sweep {i}: rows {len(n)}, stride {ld}, k {k}, lengths {n}, "
          f"patterns {kinds.tolist()}", flush=True)
    R = len(n)
    P = 4096
    pages = -(-ld // P)
    dev = torch.device("cuda:0")
    pt = torch.arange(R * pages, dtype=torch.int32, device=dev).reshape(R, pages)
    ctx = torch.tensor(n, dtype=torch.int32, device=dev)
    batch = binding.Batch(pt, ctx, n, P, R * pages)
    st = torch.from_numpy(s).to(dev)
    idx = torch.empty((R, k), dtype=torch.int32, device=dev)
    binding.topk(batch, st, k, idx)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    ref = oracle.topk(s.astype(np.float64), np.array(n), k)
    for j in range(R):
        np.testing.assert_array_equal(got[j], ref[j], err_msg=f"row {j}: n {n[j]}, "
                                                              f"pattern {int(kinds[j])}")
