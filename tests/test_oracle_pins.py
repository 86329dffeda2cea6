"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes one part of the oracle so that a plausible mistake (a dropped ReLU, a missing
head weight, a wrong page translation, a transposed operand, a wrong tie rule, a wrong bf16
or E4M3 decode) fails at least one of them: a hand-worked example, library decoders, brute
force, dense attention computed by torch on un-paged tensors, invariances of the definition
and closed forms.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from indexer_top_sparse_amd import inputs
from tests._util import custom_workload, logical_rows, to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
REALS = ["f64", "f32"]


def _hand_workload(topk=3, c=None):
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_8token.json")))
    n, P = g["ctx"], g["page_size"]
    kI = to_bf16(g["k_idx_logical"])
    cvec = g["attn_c"] if c is None else c
    kv = to_bf16([[[ct, 0.0]] for ct in cvec])                 # [8, 1, 2]
    v = to_bf16([[[float(t), 10.0 - t]] for t in range(n)])     # [8, 1, 2]
    wl = custom_workload(
        ctx_lens=[n], page_size=P, q_lens=[1], q_idx=to_bf16([g["q_idx"]]),
        w=torch.tensor([g["w"]], dtype=torch.float32), idx_keys_logical=[kI],
        q=to_bf16([[g["attn_q"]]]), kv_logical=[kv], v_logical=[v], topk=topk,
        softmax_scale=1.0)
    return g, wl


@pytest.mark.parametrize("real", REALS)
def test_hand_worked_example(real):
    g, wl = _hand_workload()
    # the fixture's page table is [1, 0]: make sure the builder reproduced it
    wl.page_table = torch.tensor([g["page_table"]], dtype=torch.int32)
    kI = to_bf16(g["k_idx_logical"])
    keys = torch.zeros_like(wl.idx_keys)
    for t in range(8):
        keys[g["page_table"][t // 4], t % 4] = kI[t]
    wl.idx_keys = keys
    kv = torch.zeros_like(wl.k_cache)
    vv = torch.zeros_like(wl.v_cache)
    for t in range(8):
        kv[g["page_table"][t // 4], t % 4, 0] = to_bf16([g["attn_c"][t], 0.0])
        vv[g["page_table"][t // 4], t % 4, 0] = to_bf16([float(t), 10.0 - t])
    wl.k_cache, wl.v_cache = kv, vv

    s = oracle.index_scores(wl, real=real)[0]
    np.testing.assert_array_equal(s, np.array(g["scores"]))
    idx = oracle.topk(s, 8, 3, real=real)[0]
    assert list(idx) == g["top3"]
    slots = [g["page_table"][t // 4] * 4 + t % 4 for t in idx]
    assert sorted(slots) == sorted(g["top3_physical_slots"])
    out = oracle.sparse_attn(wl, idx[None, :], real=real)[0, 0]
    tol = 1e-12 if real == "f64" else 1e-5
    np.testing.assert_allclose(out, g["out_sparse"], rtol=0, atol=tol)
    assert abs(out[0] + out[1] - 10.0) < tol
    dense = oracle.sparse_attn(wl, np.arange(8, dtype=np.int32)[None, :], real=real)[0, 0]
    assert abs(dense[0] - g["out_dense_0"]) < tol
    assert abs(dense[0] + dense[1] - 10.0) < tol * 10
    # padded selection (-1 entries) is ignored
    padded = np.array([[1, -1, 4, -1, 7]], dtype=np.int32)
    np.testing.assert_allclose(oracle.sparse_attn(wl, padded, real=real)[0, 0], out, atol=tol)


def test_hand_example_rejects_missing_relu():
    """The fixture's ReLU-free ranking differs: a score without ReLU would fail the test above."""
    g, _ = _hand_workload()
    q = np.array(g["q_idx"])
    k = np.array(g["k_idx_logical"])
    w = np.array(g["w"])
    no_relu = (k @ q.T) @ w
    assert sorted(np.argsort(-no_relu, kind="stable")[:3].tolist()) == g["top3_without_relu"]
    assert g["top3_without_relu"] != g["top3"]


def test_bf16_decode_matches_torch_for_every_pattern():
    bits = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    bits = np.concatenate([bits, np.array([0x0000, 0x8000, 0x0001, 0x7F7F, 0xFF7F, 0x3F80],
                                          dtype=np.uint16)])
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    got = oracle.bf16_decode(bits)
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(got[finite], ref[finite].astype(np.float64))
    assert np.all(np.isnan(got[np.isnan(ref)]))


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    got = oracle.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.all(np.isnan(got[nan]))
    np.testing.assert_array_equal(got[~nan], ref[~nan].astype(np.float64))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def _is_valid_topk(scores, n, k, sel):
    """Property that defines the selection: exactly min(k, n) distinct positions, and every kept
    position beats every dropped one (larger score, or equal score and lower position)."""
    sel = [int(t) for t in sel if t >= 0]
    if len(sel) != min(k, n) or len(set(sel)) != len(sel):
        return False
    dropped = [t for t in range(n) if t not in set(sel)]
    for i in sel:
        for j in dropped:
            si, sj = scores[i], scores[j]
            if not (si > sj or (si == sj and i < j)):
                return False
    return True


@pytest.mark.parametrize("real", REALS)
def test_topk_brute_force_with_ties(real):
    rng = np.random.default_rng(5)
    for trial in range(200):
        n = int(rng.integers(0, 11))
        k = int(rng.integers(1, 9))
        vals = rng.choice([-1.5, -0.0, 0.0, 0.25, 1.0, 2.0, 3.5], size=n)
        got = oracle.topk(np.asarray(vals, dtype=float).reshape(1, -1) if n else
                          np.zeros((1, 1)), n, k, real=real)[0]
        assert _is_valid_topk(vals, n, k, got), (vals, k, got)
        # exhaustive: the kept set is the unique subset satisfying the property
        subsets = [c for c in itertools.combinations(range(n), min(k, n))
                   if _is_valid_topk(vals, n, k, c)]
        assert len(subsets) == 1 and sorted(subsets[0]) == [t for t in got if t >= 0]
        assert list(got[min(k, n):]) == [-1] * (k - min(k, n))
        assert list(got[:min(k, n)]) == sorted(got[:min(k, n)])


def test_negative_zero_ties_positive_zero():
    s = np.array([[0.0, -0.0, 0.0, -1.0]])
    assert list(oracle.topk(s, 4, 2)[0]) == [0, 1]
    s = np.array([[-0.0, 0.0]])
    assert list(oracle.topk(s, 2, 1)[0]) == [0]


def _mla_workload(ctx_lens, heads_q=4, P=64, seed=0, topk=2048, idx_heads=8, idx_dim=128,
                  dqk=576, dv=512, perm_seed=0, q_lens=None):
    g = torch.Generator().manual_seed(seed)
    B = len(ctx_lens)
    q_lens = q_lens or [1] * B
    nq = sum(q_lens)
    kI = [torch.randn(n, idx_dim, generator=g).to(torch.bfloat16) for n in ctx_lens]
    kv = [torch.randn(n, 1, dqk, generator=g).to(torch.bfloat16) for n in ctx_lens]
    return custom_workload(
        ctx_lens=ctx_lens, page_size=P, q_lens=q_lens,
        q_idx=torch.randn(nq, idx_heads, idx_dim, generator=g).to(torch.bfloat16),
        w=torch.randn(nq, idx_heads, generator=g) / 8, idx_keys_logical=kI,
        q=torch.randn(nq, heads_q, dqk, generator=g).to(torch.bfloat16), kv_logical=kv,
        topk=topk, softmax_scale=1 / math.sqrt(dqk), perm_seed=perm_seed, dim_v=dv)


@pytest.mark.parametrize("real", REALS)
def test_full_selection_equals_dense_attention(real):
    """K >= context: sparse attention over everything equals dense softmax(QK^T)V computed by
    torch in fp64 on un-paged rows (MLA latent rows: K = all 576, V = first 512)."""
    ctx = [200, 64, 1]
    wl = _mla_workload(ctx, topk=256)
    res = oracle.decode_step(wl, real=real)
    for b, n in enumerate(ctx):
        assert sorted(res["idx"][b][res["idx"][b] >= 0].tolist()) == list(range(n))
        rows = logical_rows(wl.k_cache, wl.page_table, b, n, wl.page_size)[:, 0].double()
        K, V = rows[:, :576], rows[:, :512]
        Q = wl.q[b].double()
        scale = float(np.float32(wl.softmax_scale))  # the scale is an fp32 argument
        att = torch.softmax((Q @ K.T) * scale, dim=-1) @ V
        tol = 1e-10 if real == "f64" else 2e-5
        np.testing.assert_allclose(res["out"][b], att.numpy(), rtol=0, atol=tol)


def test_gqa_separate_kv_dense_attention():
    """Separate K and V caches, 8 query heads over 2 KV heads (groups of 4)."""
    g = torch.Generator().manual_seed(3)
    n, d = 70, 16
    kv = [torch.randn(n, 2, d, generator=g).to(torch.bfloat16)]
    v = [torch.randn(n, 2, d, generator=g).to(torch.bfloat16)]
    wl = custom_workload(
        ctx_lens=[n], page_size=16, q_lens=[1],
        q_idx=torch.randn(1, 2, 8, generator=g).to(torch.bfloat16), w=torch.ones(1, 2),
        idx_keys_logical=[torch.randn(n, 8, generator=g).to(torch.bfloat16)],
        q=torch.randn(1, 8, d, generator=g).to(torch.bfloat16), kv_logical=kv, v_logical=v,
        topk=128, softmax_scale=0.25)
    out = oracle.sparse_attn(wl, np.arange(128, dtype=np.int32).reshape(1, -1) % 70 * 0 +
                             np.where(np.arange(128) < 70, np.arange(128), -1)[None, :])[0]
    K = logical_rows(wl.k_cache, wl.page_table, 0, n, 16).double()
    V = logical_rows(wl.v_cache, wl.page_table, 0, n, 16).double()
    for h in range(8):
        kvh = h // 4
        att = torch.softmax(wl.q[0, h].double() @ K[:, kvh].T * 0.25, -1) @ V[:, kvh]
        np.testing.assert_allclose(out[h], att.numpy(), atol=1e-12)


def test_page_permutation_invariance_bitwise():
    a = _mla_workload([300, 129], perm_seed=1, topk=64)
    b = _mla_workload([300, 129], perm_seed=2, topk=64)
    assert not torch.equal(a.page_table, b.page_table)
    ra, rb = oracle.decode_step(a), oracle.decode_step(b)
    np.testing.assert_array_equal(ra["scores"], rb["scores"])
    np.testing.assert_array_equal(ra["idx"], rb["idx"])
    np.testing.assert_array_equal(ra["out"], rb["out"])


def test_repaging_invariance_bitwise():
    a = _mla_workload([300, 129], P=64, topk=64)
    b = _mla_workload([300, 129], P=16, topk=64)
    ra, rb = oracle.decode_step(a), oracle.decode_step(b)
    np.testing.assert_array_equal(ra["scores"], rb["scores"])
    np.testing.assert_array_equal(ra["idx"], rb["idx"])
    np.testing.assert_array_equal(ra["out"], rb["out"])


def test_weight_scaling_scales_scores():
    wl = _mla_workload([500], topk=32)
    s1 = oracle.index_scores(wl)
    wl.w = wl.w * 4.0
    s4 = oracle.index_scores(wl)
    np.testing.assert_array_equal(s4, s1 * 4.0)
    np.testing.assert_array_equal(oracle.topk(s1, 500, 32), oracle.topk(s4, 500, 32))


def test_single_head_unit_weight_is_a_matmul():
    """H_I = 1, w = 1, and keys chosen so that every dot product is positive: the score is the
    plain matrix product (numpy)."""
    g = torch.Generator().manual_seed(9)
    n, d = 150, 32
    kI = torch.rand(n, d, generator=g).to(torch.bfloat16)
    q = torch.rand(1, 1, d, generator=g).to(torch.bfloat16)
    wl = custom_workload(ctx_lens=[n], page_size=16, q_lens=[1], q_idx=q,
                         w=torch.ones(1, 1), idx_keys_logical=[kI],
                         q=torch.zeros(1, 1, 8, dtype=torch.bfloat16),
                         kv_logical=[torch.zeros(n, 1, 8, dtype=torch.bfloat16)], topk=4,
                         softmax_scale=1.0)
    s = oracle.index_scores(wl)[0]
    ref = kI.double().numpy() @ q[0, 0].double().numpy()
    np.testing.assert_allclose(s, ref, rtol=1e-13)


def test_all_nonpositive_dots_give_zero_scores():
    g = torch.Generator().manual_seed(4)
    n, d = 100, 16
    kI = torch.rand(n, d, generator=g).to(torch.bfloat16)
    q = (-torch.rand(1, 3, d, generator=g)).to(torch.bfloat16)
    wl = custom_workload(ctx_lens=[n], page_size=16, q_lens=[1], q_idx=q,
                         w=torch.randn(1, 3, generator=g), idx_keys_logical=[kI],
                         q=torch.zeros(1, 1, 8, dtype=torch.bfloat16),
                         kv_logical=[torch.zeros(n, 1, 8, dtype=torch.bfloat16)], topk=4,
                         softmax_scale=1.0)
    assert np.all(oracle.index_scores(wl)[0] == 0)
    # ties everywhere: the lowest positions win
    assert list(oracle.topk(oracle.index_scores(wl), n, 4)[0]) == [0, 1, 2, 3]


def test_closed_forms_attention():
    wl = _mla_workload([130], heads_q=3, topk=16)
    idx = np.array([[3, 77, 129, 5, -1, 64, 0, 11, 12, 13, 99, 100, 101, 2, 1, 128]],
                   dtype=np.int32)
    # equal V rows -> o = v
    v = torch.randn(512).to(torch.bfloat16)
    kc = wl.k_cache.clone()
    kc[:, :, 0, :512] = v
    wl2 = custom_workload(ctx_lens=[130], page_size=64, q_lens=[1], q_idx=wl.q_idx, w=wl.w,
                          idx_keys_logical=[torch.zeros(130, 128, dtype=torch.bfloat16)],
                          q=wl.q, kv_logical=[torch.zeros(130, 1, 576, dtype=torch.bfloat16)],
                          topk=16, softmax_scale=wl.softmax_scale, dim_v=512)
    wl2.k_cache, wl2.page_table = kc, wl.page_table
    out = oracle.sparse_attn(wl2, idx)[0]
    np.testing.assert_allclose(out, np.broadcast_to(v.double().numpy(), out.shape), atol=1e-12)
    # q = 0 -> mean of the selected V rows
    wl.q = torch.zeros_like(wl.q)
    out = oracle.sparse_attn(wl, idx)[0]
    rows = logical_rows(wl.k_cache, wl.page_table, 0, 130, 64)[:, 0, :512].double()
    sel = [t for t in idx[0] if t >= 0]
    np.testing.assert_allclose(out[0], rows[sel].mean(0).numpy(), atol=1e-12)
    # empty selection -> zeros
    out = oracle.sparse_attn(wl, -np.ones((1, 16), dtype=np.int32))[0]
    assert np.all(out == 0)


def test_fp8_zero_codes_give_zero_scores():
    n = 80
    wl = custom_workload(ctx_lens=[n], page_size=16, q_lens=[1],
                         q_idx=torch.randn(1, 4, 32).to(torch.bfloat16), w=torch.randn(1, 4),
                         idx_keys_logical=[torch.zeros(n, 32, dtype=torch.uint8)],
                         idx_scale_logical=[torch.ones(n)], idx_dtype="fp8",
                         q=torch.zeros(1, 1, 8, dtype=torch.bfloat16),
                         kv_logical=[torch.zeros(n, 1, 8, dtype=torch.bfloat16)], topk=4,
                         softmax_scale=1.0)
    assert np.all(oracle.index_scores(wl)[0] == 0)


def test_fp8_scale_factors_out():
    """E4M3 keys with per-token scale sigma: the score equals the score of the decoded keys
    (code value times sigma) stored as exact bf16 (E4M3 values are exact in bf16 and sigma is a
    power of two here)."""
    g = torch.Generator().manual_seed(2)
    n = 96
    x = torch.randn(n, 64, generator=g)
    codes = x.to(torch.float8_e4m3fn)
    sigma = 2.0 ** torch.randint(-3, 4, (n,), generator=g).float()
    dec = (codes.float() * sigma[:, None]).to(torch.bfloat16)
    assert torch.equal(dec.float(), codes.float() * sigma[:, None])
    common = dict(ctx_lens=[n], page_size=32, q_lens=[1],
                  q_idx=torch.randn(1, 4, 64, generator=g).to(torch.bfloat16),
                  w=torch.randn(1, 4, generator=g), q=torch.zeros(1, 1, 8, dtype=torch.bfloat16),
                  kv_logical=[torch.zeros(n, 1, 8, dtype=torch.bfloat16)], topk=8,
                  softmax_scale=1.0)
    a = custom_workload(idx_keys_logical=[codes.view(torch.uint8)], idx_scale_logical=[sigma],
                        idx_dtype="fp8", **common)
    b = custom_workload(idx_keys_logical=[dec], **common)
    np.testing.assert_allclose(oracle.index_scores(a), oracle.index_scores(b), rtol=1e-13)


def test_prefill_row_equals_decode_at_that_length():
    """A prefill query at position p sees exactly what a decode step at context p + 1 sees."""
    ctx, ql = 700, 40
    pre = _mla_workload([ctx], q_lens=[ql], topk=128, heads_q=2)
    pos = pre.q_pos().numpy()
    s_pre = oracle.index_scores(pre)
    for r in (0, 17, ql - 1):
        p = int(pos[r])
        dec = _mla_workload([ctx], q_lens=[ql], topk=128, heads_q=2)  # same caches
        dec.ctx_lens = [p + 1]
        dec.q_lens = [1]
        dec.q_idx, dec.w, dec.q = pre.q_idx[r:r + 1], pre.w[r:r + 1], pre.q[r:r + 1]
        s_dec = oracle.index_scores(dec)[0]
        np.testing.assert_array_equal(s_dec, s_pre[r, :p + 1])
        assert np.all(np.isneginf(s_pre[r, p + 1:]))
        i_pre = oracle.topk(s_pre[r:r + 1], p + 1, 128)
        i_dec = oracle.topk(s_dec[None], p + 1, 128)
        np.testing.assert_array_equal(i_pre, i_dec)
        np.testing.assert_array_equal(oracle.sparse_attn(pre, i_pre, rows=[r]),
                                      oracle.sparse_attn(dec, i_dec))


def _two_level_workload(ctx_lens, block_topk, P=16, seed=0):
    wl = _mla_workload(ctx_lens, P=P, topk=48, seed=seed, idx_dim=32, idx_heads=4)
    wl.block_topk = block_topk
    # block summaries: mean of each block's valid key rows (the generator's definition)
    wl.pooled = inputs._pooled_keys(wl.idx_keys, wl.page_table, wl.ctx_lens, P)
    return wl


def test_two_level_with_all_blocks_equals_single_level():
    wl = _two_level_workload([300, 77], block_topk=64)
    single = oracle.index_scores(wl)
    q_pos = wl.q_pos().numpy()
    ref = oracle.topk(single, q_pos + 1, wl.topk)
    blocks, idx, _ = oracle.two_level_select(wl)
    np.testing.assert_array_equal(idx, ref)
    for r in range(2):
        nb = q_pos[r] // 16 + 1
        assert sorted(blocks[r][blocks[r] >= 0].tolist()) == list(range(nb))


def test_two_level_fine_stage_is_restricted_to_kept_blocks():
    wl = _two_level_workload([400], block_topk=5)
    blocks, idx, bs = oracle.two_level_select(wl)
    kept = set(blocks[0][blocks[0] >= 0].tolist())
    assert len(kept) == 5
    assert all((t // 16) in kept for t in idx[0] if t >= 0)
    # the kept blocks are the 5 best block scores
    order = sorted(range(25), key=lambda j: (-bs[0, j], j))[:5]
    assert kept == set(order)
    # brute force: best 48 tokens among the kept blocks' tokens
    s = oracle.index_scores(wl)[0]
    cand = sorted([t for t in range(400) if t // 16 in kept], key=lambda t: (-s[t], t))[:48]
    assert sorted(cand) == [t for t in idx[0] if t >= 0]


def test_generator_pooled_keys_are_block_means():
    wl = inputs.make("long1m", num_seqs=1, ctx=1000, page_size=64)
    kf = wl.idx_keys.double()
    for j in (0, 5, 15):  # 15 is the partial last block (1000 = 15 * 64 + 40)
        phys = int(wl.page_table[0, j])
        cnt = 64 if j < 15 else 40
        ref = kf[phys, :cnt].mean(0).to(torch.bfloat16)
        assert torch.equal(wl.pooled[phys], ref)


def test_f32_oracle_agrees_with_f64():
    """The fp32 build's own rounding stays far below the acceptance tolerances (1e-3 relative
    near-tie band for indices, 2e-2 absolute for outputs)."""
    from tests._util import check_topk_row
    wl = inputs.make("decode32k", num_seqs=2, ctx=3000)
    a = oracle.decode_step(wl, real="f64")
    b = oracle.decode_step(wl, real="f32")
    fin = np.isfinite(a["scores"])
    err = np.abs(a["scores"] - b["scores"])[fin].max()
    assert err < 1e-5 * np.abs(a["scores"][fin]).max()
    for r in range(2):
        assert check_topk_row(b["idx"][r], a["idx"][r], a["scores"][r], 3000, wl.topk) == ""
    np.testing.assert_allclose(b["out"], a["out"], atol=1e-5)


def _block_workload(ctx_lens, P=16, block_topk=6, perm_seed=0, seed=21):
    """Two-level workload whose block summaries are computed here from the logical key rows
    (fp64 mean over each block's valid tokens, rounded to bf16) and handed to the layout
    builder per logical block, so nothing on the reference side reads the page table."""
    g = torch.Generator().manual_seed(seed)
    B = len(ctx_lens)
    idx_dim, idx_heads = 32, 4
    kI = [torch.randn(n, idx_dim, generator=g).to(torch.bfloat16) for n in ctx_lens]
    pooled = []
    for n, rows in zip(ctx_lens, kI):
        nb = -(-n // P)
        pooled.append(torch.stack([rows[j * P:min(n, (j + 1) * P)].double().mean(0)
                                   for j in range(nb)]).to(torch.bfloat16))
    kv = [torch.randn(n, 1, 576, generator=g).to(torch.bfloat16) for n in ctx_lens]
    wl = custom_workload(
        ctx_lens=ctx_lens, page_size=P, q_lens=[1] * B,
        q_idx=torch.randn(B, idx_heads, idx_dim, generator=g).to(torch.bfloat16),
        w=torch.randn(B, idx_heads, generator=g) / 8, idx_keys_logical=kI,
        q=torch.randn(B, 2, 576, generator=g).to(torch.bfloat16), kv_logical=kv, topk=40,
        block_topk=block_topk, pooled_logical=pooled, softmax_scale=1 / 24, perm_seed=perm_seed,
        dim_v=512)
    return wl, pooled


def _np_block_score(q, w, kbar):
    """sum_h w_h * max(q_h . kbar, 0) in fp64 (the score formula applied to one summary row)."""
    d = q.double().numpy() @ kbar.double().numpy()
    return float(np.sum(w.double().numpy() * np.maximum(d, 0.0)))


def test_block_scores_follow_the_page_table():
    """Coarse stage ([SameDay] §3.1: blocks are ranked by their cached summaries): the score of
    logical block j is the formula applied to the summary of block j, wherever the page table
    put it. The pages are shuffled, so reading the summary table by logical index (row j
    instead of row page_table[b][j]) gives different scores; the test checks that it would."""
    ctx = [300, 77]
    wl, pooled = _block_workload(ctx)
    assert not torch.equal(wl.page_table[0, :5], torch.arange(5, dtype=torch.int32))
    got = oracle.block_scores(wl)
    wrong_gap = 0.0
    for b, n in enumerate(ctx):
        nb = -(-n // wl.page_size)
        for j in range(wl.pages_per_seq):
            if j >= nb:
                assert np.isneginf(got[b, j])
                continue
            ref = _np_block_score(wl.q_idx[b], wl.w[b], pooled[b][j])
            assert abs(got[b, j] - ref) <= 1e-12 * max(1.0, abs(ref)), (b, j, got[b, j], ref)
            # what a lookup by logical index would have scored
            wrong = _np_block_score(wl.q_idx[b], wl.w[b], wl.pooled[j])
            wrong_gap = max(wrong_gap, abs(wrong - ref))
    assert wrong_gap > 0.05 * np.abs(got[np.isfinite(got)]).max()


def test_two_level_page_permutation_invariance():
    """The same logical caches under two different page tables give the same block sets, the
    same token sets and bitwise the same outputs (selection works on logical positions)."""
    ctx = [300, 77, 150]
    a, _ = _block_workload(ctx, perm_seed=0)
    b, _ = _block_workload(ctx, perm_seed=5)
    assert not torch.equal(a.page_table, b.page_table)
    ra, rb = oracle.decode_step(a), oracle.decode_step(b)
    np.testing.assert_array_equal(ra["blocks"], rb["blocks"])
    np.testing.assert_array_equal(ra["idx"], rb["idx"])
    np.testing.assert_array_equal(ra["out"], rb["out"])
    # and the kept blocks are the best-scoring logical blocks computed from the logical rows
    _, pooled = _block_workload(ctx, perm_seed=0)
    for s, n in enumerate(ctx):
        nb = -(-n // a.page_size)
        sc = [_np_block_score(a.q_idx[s], a.w[s], pooled[s][j]) for j in range(nb)]
        best = sorted(range(nb), key=lambda j: (-sc[j], j))[:a.block_topk]
        assert sorted(best) == [j for j in ra["blocks"][s] if j >= 0]
