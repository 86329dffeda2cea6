"""Pins of the oracle's MXFP8 indexer arithmetic (test infrastructure, CPU only).

The indexer's MXFP8 variant (E4M3 elements, one E8M0 power-of-two scale per 32 consecutive
elements; "Day0 Inference Support and Performance Optimization for Next-Gen Large Models on
Huawei Ascend CANN Architecture", §3) is pinned to hand-derived codes of the E4M3 definition,
to an exactly representable block, to the rounding bound the format implies, and to a score
example that reduces to plain arithmetic.
"""
import json
import math
import os

import numpy as np
import torch

import oracle
from indexer_top_sparse_amd import inputs
from tests._util import custom_workload, to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp8_e4m3_codes.json")


def test_e4m3_encode_hand_derived_codes():
    g = json.load(open(GOLDEN))
    for value, code, why in g["encode"]:
        got = int(oracle.e4m3_encode([value])[0])
        assert got == code, f"{value}: got {got:#04x}, want {code:#04x} ({why})"
    # -0.0 keeps its sign bit
    assert int(oracle.e4m3_encode([-0.0])[0]) == 0x80


def test_e4m3_encode_inverts_decode_on_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    back = oracle.e4m3_encode(vals)
    # +0 and -0 decode to signed zeros and come back unchanged
    np.testing.assert_array_equal(back, codes)


def test_mx_exponent_hand_derived():
    g = json.load(open(GOLDEN))
    for amax, x, why in g["mx_exponent"]:
        assert oracle.mx_exponent(amax) == x, why


def test_mx_quantize_exact_block():
    """k / 4 for k = -16..15: amax 4 gives X = -6, so every element scales to 16 k, an integer
    with at most 4 significant bits and therefore exact in E4M3 (16 = 2^4 -> code 0x58)."""
    vals = np.arange(-16, 16, dtype=np.float64) / 4
    bits = to_bf16(vals.tolist()).view(torch.int16).numpy().view(np.uint16)
    codes, e8m0 = oracle.mx_quantize_bf16(bits)
    assert e8m0.tolist() == [127 - 6]
    assert int(codes[17]) == 0x58            # 0.25 * 64 = 16
    assert int(codes[16]) == 0x00            # 0
    assert int(codes[0]) == 0xF8             # -4 * 64 = -256 = -1.0 x 2^8: exponent field 15
    np.testing.assert_array_equal(oracle.e4m3_decode(codes) * 2.0 ** -6, vals)


def test_mx_quantize_corner_block():
    """A block whose largest magnitude is 464 (X = floor(log2 464) - 8 = 0, so the elements are
    encoded as they are): 464 lies above E4M3's largest value and saturates to 448 (0x7E);
    1.0625, 17, 19 and -1.1875 sit exactly between two E4M3 neighbours and go to the one with
    the even mantissa (1.0, 16, 20, -1.25); in the subnormal range (steps of 2^-9) 1.5 steps
    rounds to 2 steps, half a step to 0, and minus half a step to -0 (0x80). Codes derived by
    hand from the E4M3 layout (sign, 4 exponent bits with bias 7, 3 mantissa bits)."""
    vals = [464.0, 1.0625, 17.0, 19.0, -1.1875, 3 * 2.0 ** -10, 2.0 ** -10, -2.0 ** -10,
            -300.0, 255.0, 0.5, -0.03125]
    want = [0x7E, 0x38, 0x58, 0x5A, 0xBA, 0x02, 0x00, 0x80,
            0xF9,         # -300: between -288 (1.125 x 2^8) and -320 (1.25 x 2^8), nearer -288
            0x78,         # 255 -> 256 = 1.0 x 2^8
            0x30,         # 0.5 = 2^-1: exponent field 6
            0x90]         # -0.03125 = -2^-5: exponent field 2
    blk = vals + [0.0] * (32 - len(vals))
    bits = to_bf16(blk).view(torch.int16).numpy().view(np.uint16)
    codes, e8m0 = oracle.mx_quantize_bf16(bits)
    assert e8m0.tolist() == [127]
    assert [int(c) for c in codes[:len(vals)]] == want
    assert not np.any(codes[len(vals):])


def test_mx_quantize_rounding_bound():
    """Random bf16 blocks: every element is within half an E4M3 step of its value (relative
    2^-4 in the normal range, 2^(X-10) absolute in the subnormal range), except elements whose
    scaled magnitude exceeds 448, which saturate to 448 * 2^X."""
    rng = np.random.default_rng(3)
    vals = rng.standard_normal((64, 128)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    bits = to_bf16(vals.tolist()).view(torch.int16).numpy().view(np.uint16)
    v = oracle.bf16_decode(bits)
    codes, e8m0 = oracle.mx_quantize_bf16(bits)
    X = e8m0.astype(np.int64) - 127
    Xe = np.repeat(X, 32, axis=1)
    deq = oracle.e4m3_decode(codes) * np.exp2(Xe.astype(np.float64))
    scaled = np.abs(v) * np.exp2(-Xe.astype(np.float64))
    err = np.abs(deq - v)
    normal = (scaled >= 2.0 ** -6) & (scaled <= 448)
    sub = scaled < 2.0 ** -6
    sat = scaled > 448
    assert np.all(err[normal] <= np.abs(v[normal]) * 2.0 ** -4 + 0)
    assert np.all(err[sub] <= np.exp2(Xe[sub] - 10.0))
    assert np.all(np.abs(deq[sat]) == 448 * np.exp2(Xe[sat].astype(np.float64)))
    # the block maximum always lands in [256, 512) before saturation
    amax = np.abs(v).reshape(64, 4, 32).max(axis=2)
    ratio = amax * np.exp2(-X.astype(np.float64))
    assert np.all((ratio >= 256) & (ratio < 512))


def test_mx_scores_reduce_to_plain_arithmetic_on_representable_values():
    """Query and key values that MXFP8 represents exactly (k / 4, k = -16..15, per block): the
    MXFP8 score equals sum_h w_h max(q_h . k_t, 0) computed directly."""
    rng = np.random.default_rng(11)
    heads, dim, n, P = 4, 128, 40, 16
    q = rng.integers(-16, 16, (heads, dim)) / 4.0
    for h in range(heads):  # every block holds -4 so that its exponent is -6
        q[h, ::32] = -4.0
    keys = rng.integers(-16, 16, (n, dim)) / 4.0
    keys[:, ::32] = -4.0
    w = rng.standard_normal(heads).astype(np.float32)
    codes, e8m0 = inputs.quantize_rows_mxfp8(torch.tensor(keys, dtype=torch.float32))
    assert torch.all(e8m0 == 121)
    wl = custom_workload(
        ctx_lens=[n], page_size=P, q_lens=[1], q_idx=to_bf16([q.tolist()]),
        w=torch.tensor([w.tolist()], dtype=torch.float32),
        idx_keys_logical=[to_bf16(keys.tolist())], q=to_bf16([[[0.0] * 128]]),
        kv_logical=[to_bf16([[[0.0] * 128]] * n)], v_logical=None, topk=8, softmax_scale=1.0)
    # same page permutation, keys replaced by their MXFP8 encoding
    phys = torch.zeros((wl.num_pages, P, dim), dtype=torch.uint8)
    phys_e = torch.zeros((wl.num_pages, P, dim // 32), dtype=torch.uint8)
    for t in range(n):
        pg = int(wl.page_table[0, t // P])
        phys[pg, t % P] = codes[t]
        phys_e[pg, t % P] = e8m0[t]
    wl.idx_keys, wl.idx_mx_scale, wl.idx_dtype, wl.idx_scale = phys, phys_e, "mxfp8", None
    got = oracle.index_scores(wl)[0]
    want = (np.maximum(q @ keys.T, 0) * w[:, None].astype(np.float64)).sum(axis=0)
    np.testing.assert_allclose(got[:n], want, rtol=1e-12, atol=1e-12)


def test_generator_mxfp8_keys_match_the_oracle_quantizer():
    """The input generator stores MXFP8 keys with torch's E4M3 conversion; on bf16-exact inputs
    its codes and exponents are the oracle's."""
    rng = np.random.default_rng(5)
    vals = rng.standard_normal((16, 128)) * np.exp(rng.uniform(-6, 6, (16, 1)))
    x = to_bf16(vals.tolist()).to(torch.float32)
    codes, e8m0 = inputs.quantize_rows_mxfp8(x)
    bits = to_bf16(vals.tolist()).view(torch.int16).numpy().view(np.uint16)
    ocodes, oe8m0 = oracle.mx_quantize_bf16(bits)
    np.testing.assert_array_equal(e8m0.numpy(), oe8m0)
    np.testing.assert_array_equal(codes.numpy(), ocodes)
