"""Pins of the oracle's FP8 KV with one scale per 128 entries of each token and head
("Day0 Inference Support and Performance Optimization for Next-Gen Large Models on Huawei Ascend
CANN Architecture", §3: FP8 KV quantized per token-head-tile with a block of 128). Test
infrastructure, CPU only.

The pins: one selected row returns its own decoded value (closed form, decoded with torch's E4M3
type, not the oracle's table); a one-hot query isolates the scale of a single tile, the 64-entry
rope tile included; equal tile scales reduce to the per-row format, which has pins of its own;
and the generator's tile quantizer keeps every tile within the E4M3 rounding bound of its own
maximum.
"""
import numpy as np
import torch

import oracle
from indexer_top_sparse_amd import inputs
from tests._util import custom_workload, to_bf16

D, DV = 576, 512
NT = 5  # tiles of a 576-entry row: four of 128 and one of 64


def _decode(codes_u8: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes_u8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _workload(codes, scales, q, idx_len, kv_dtype="fp8t128"):
    """One sequence of len(codes) tokens (page size 4), latent rows [n, 1, 576] of E4M3 codes;
    scales [n, 1, 5] (fp8t128) or [n] (fp8)."""
    n = codes.shape[0]
    return custom_workload(
        ctx_lens=[n], page_size=4, q_lens=[1], q_idx=to_bf16(np.zeros((1, 1, 64))),
        w=torch.ones((1, 1)), idx_keys_logical=[to_bf16(np.zeros((n, 64)))],
        q=to_bf16(q.reshape(1, -1, D)), kv_logical=[torch.from_numpy(codes).reshape(n, 1, D)],
        topk=idx_len, softmax_scale=1.0 / 24, kv_dtype=kv_dtype,
        kv_scale_logical=[torch.from_numpy(scales.astype(np.float32))], dim_v=DV)


def _codes(rng, n):
    c = rng.integers(0, 256, (n, D), dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN patterns
    return c


def test_single_selected_row_returns_its_decoded_value():
    rng = np.random.default_rng(1)
    n = 6
    codes = _codes(rng, n)
    scales = np.ldexp(1.0, rng.integers(-6, 6, (n, 1, NT))).astype(np.float32)
    q = rng.standard_normal((2, D))
    wl = _workload(codes, scales, q, idx_len=3)
    out = oracle.sparse_attn(wl, np.array([[4, -1, -1]], dtype=np.int32))
    want = _decode(codes[4, :DV]) * np.repeat(scales[4, 0, :4], 128)
    for h in range(2):
        np.testing.assert_array_equal(out[0, h], want)


def test_one_hot_query_sees_only_its_tile_scale():
    """q = c * e_520 (inside the 64-entry rope tile): the logit of a row is
    scale * c * code[520] * sigma[tile 4]; the other tiles' scales must not enter. Two rows with
    equal codes and rope scales 2 and 1 give softmax weights proportional to
    exp(scale * c * 2) and exp(scale * c * 1)."""
    rng = np.random.default_rng(2)
    codes = _codes(rng, 2)
    codes[:, 520] = 0x38  # 1.0
    scales = np.ones((2, 1, NT), dtype=np.float32)
    scales[0, 0, 4] = 2.0
    scales[1, 0, 3] = 100.0  # a wrong tile index would pick this up
    c = 24.0
    q = np.zeros((1, D))
    q[0, 520] = c
    wl = _workload(codes, scales, q, idx_len=2)
    out = oracle.sparse_attn(wl, np.array([[0, 1]], dtype=np.int32))[0, 0]
    logit = np.array([2.0, 1.0]) * c * float(np.float32(1 / 24))  # the scale is an fp32 input
    p = np.exp(logit - logit.max())
    p /= p.sum()
    v = [_decode(codes[j, :DV]) * np.repeat(scales[j, 0, :4], 128) for j in range(2)]
    want = p[0] * v[0] + p[1] * v[1]
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)


def test_equal_tile_scales_reduce_to_the_per_row_format():
    rng = np.random.default_rng(3)
    n = 9
    codes = _codes(rng, n)
    sigma = rng.uniform(0.01, 2.0, n).astype(np.float32)
    q = rng.standard_normal((3, D))
    tiles = np.repeat(sigma[:, None, None], NT, axis=2)
    idx = np.array([[0, 3, 8, 5, -1]], dtype=np.int32)
    a = oracle.sparse_attn(_workload(codes, tiles, q, 5), idx)
    b = oracle.sparse_attn(_workload(codes, sigma, q, 5, kv_dtype="fp8"), idx)
    np.testing.assert_array_equal(a, b)


def test_tile_quantizer_keeps_each_tile_within_its_rounding_bound():
    """Tiles of one row at magnitudes 2^-20 .. 2^20 apart: every element is within half an E4M3
    step (relative 2^-4) of its value, or within 2^-10 * sigma in the subnormal range; a single
    per-row scale would flush the small tiles to zero."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, D))
    mags = np.ldexp(1.0, rng.integers(-20, 20, (8, NT)))
    x *= np.repeat(mags, 128, axis=1)[:, :D]
    codes, sigma = inputs.quantize_tiles_e4m3(torch.from_numpy(x).float(), 128)
    assert codes.shape == (8, D) and sigma.shape == (8, NT)
    xf = torch.from_numpy(x).float().double().numpy()
    dec = _decode(codes.numpy()) * np.repeat(sigma.double().numpy(), 128, axis=1)[:, :D]
    s_el = np.repeat(sigma.double().numpy(), 128, axis=1)[:, :D]
    err = np.abs(dec - xf)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, s_el * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))
    # each tile's maximum maps to 448 * sigma
    for t in range(NT):
        sl = slice(128 * t, min(D, 128 * t + 128))
        np.testing.assert_allclose(np.abs(xf[:, sl]).max(axis=1), 448 * sigma[:, t].double().numpy(),
                                   rtol=1e-6)
