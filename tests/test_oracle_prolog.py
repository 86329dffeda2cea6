"""Pins of the oracle's indexer prolog ("Day0 Inference Support and Performance Optimization for
Next-Gen Large Models on Huawei Ascend CANN Architecture", §2.2: Q projection, K normalization,
head-weight projection). Test infrastructure, CPU only.

The pins are special cases with closed forms: identity-like weights that copy input columns, a
LayerNorm of a vector whose mean and variance are known by construction, the LayerNorm
invariants (zero mean and unit variance before the affine step, invariance to shifting and
scaling the input), and weights that pick one input entry per head.
"""
import numpy as np
import torch

import oracle


def _bf(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def test_identity_weights_copy_the_inputs():
    rng = np.random.default_rng(0)
    rows, H, D, dq, dm = 3, 2, 8, 20, 24
    xq = rng.integers(-8, 8, (rows, dq)).astype(np.float32)
    x = rng.integers(-8, 8, (rows, dm)).astype(np.float32)
    wq = np.zeros((H * D, dq), np.float32)
    wq[np.arange(H * D), np.arange(H * D)] = 1.0       # q_I = first H*D entries of x_q
    wk = np.zeros((D, dm), np.float32)
    wk[np.arange(D), 3 + np.arange(D)] = 1.0          # pre-norm k = x[:, 3:3+D]
    ww = np.zeros((H, dm), np.float32)
    ww[0, 5] = 2.0
    ww[1, 7] = -0.5                                    # w = (2 x5, -x7 / 2)
    q, k, w = oracle.indexer_prolog(_bf(xq), _bf(x), _bf(wq), _bf(wk), _bf(ww),
                                    torch.ones(D), torch.zeros(D))
    np.testing.assert_array_equal(q, xq[:, :H * D])
    np.testing.assert_array_equal(w, np.stack([2 * x[:, 5], -0.5 * x[:, 7]], axis=1))
    y = x[:, 3:3 + D].astype(np.float64)
    mu = y.mean(axis=1, keepdims=True)
    sd = np.sqrt(((y - mu) ** 2).mean(axis=1, keepdims=True) + oracle.LN_EPS)
    np.testing.assert_allclose(k, (y - mu) / sd, rtol=1e-14, atol=1e-14)


def test_layernorm_closed_form():
    """y = (a, -a, a, -a, ...) has mean 0 and variance a^2: k = sign * a / sqrt(a^2 + eps), then
    gamma and beta apply entrywise."""
    D, a = 8, 3.0
    y = np.array([a, -a] * (D // 2), np.float32)
    wk = np.eye(D, dtype=np.float32)
    gamma = torch.arange(1, D + 1, dtype=torch.float32)
    beta = torch.full((D,), 0.5)
    _, k, _ = oracle.indexer_prolog(_bf(np.zeros((1, 4))), _bf(y[None, :]), _bf(np.zeros((2, 4))),
                                    _bf(wk), _bf(np.zeros((1, D))), gamma, beta)
    want = np.sign(y) * a / np.sqrt(a * a + oracle.LN_EPS) * np.arange(1, D + 1) + 0.5
    np.testing.assert_allclose(k[0], want, rtol=1e-14)


def test_layernorm_invariants():
    rng = np.random.default_rng(1)
    rows, D, dm = 4, 16, 32
    x = rng.standard_normal((rows, dm)).astype(np.float32)
    wk = rng.standard_normal((D, dm)).astype(np.float32)
    args = (_bf(np.zeros((rows, 4))), _bf(x), _bf(np.zeros((2, 4))), _bf(wk), _bf(np.zeros((1, dm))))
    _, k, _ = oracle.indexer_prolog(*args, torch.ones(D), torch.zeros(D), eps=0.0)
    np.testing.assert_allclose(k.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose((k ** 2).mean(axis=1), 1.0, rtol=1e-12)
    # scaling the key weights by 4 (exact in bf16) leaves the normalized key unchanged
    wk4 = _bf(wk).float() * 4
    _, k4, _ = oracle.indexer_prolog(*args[:3], wk4.to(torch.bfloat16), args[4], torch.ones(D),
                                     torch.zeros(D), eps=0.0)
    np.testing.assert_allclose(k4, k, rtol=1e-12, atol=1e-12)


def test_projection_matches_per_head_dot_products():
    """Head h of q_I is x_q times rows h*d_I .. h*d_I + d_I - 1 of W_q: checked entry by entry
    with Python sums over small integer data (exact in fp64)."""
    rng = np.random.default_rng(2)
    rows, H, D, dq = 2, 3, 4, 6
    xq = rng.integers(-4, 5, (rows, dq)).astype(np.float32)
    wq = rng.integers(-4, 5, (H * D, dq)).astype(np.float32)
    q, _, _ = oracle.indexer_prolog(_bf(xq), _bf(np.zeros((rows, 8))), _bf(wq),
                                    _bf(np.zeros((D, 8))), _bf(np.zeros((H, 8))), torch.ones(D),
                                    torch.zeros(D))
    for r in range(rows):
        for h in range(H):
            for d in range(D):
                assert q[r, h * D + d] == sum(xq[r, i] * wq[h * D + d, i] for i in range(dq))
