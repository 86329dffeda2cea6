"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

Acceptance (the contract of the library):
  * indices: exactly min(K, visible) distinct visible positions, -1 padded; every position
    in the symmetric difference with the oracle's set scores within 1e-3 * |theta| of theta,
    the oracle's K-th score (near ties). Where both sides select from the same fp32 scores
    (sa_topk) the sets must be identical.
  * attention outputs: max |out_gpu - out_oracle| <= 2e-2 (bf16 caches) or 5e-2 (E4M3), the
    oracle run on the GPU's own index set (legal near-tie swaps do not count).
  * indexer scores (sa_index_score): |s_gpu - s_oracle| <= 1e-4 * max_t |s_oracle| per row
    (fp32 accumulation of exact bf16 products; see the design notes for the bound).
"""
import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from indexer_top_sparse_amd import binding, device, inputs
from tests._util import check_topk_in, check_topk_row, custom_workload, output_error, to_bf16

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _check_decode(wl, out, idx, tol, rows=None, ref=None):
    rows = list(range(wl.num_seqs)) if rows is None else rows
    ref = ref or oracle.decode_step(wl, rows=rows)
    got_idx = idx.cpu().numpy()[rows]
    for r, b in enumerate(rows):
        n = wl.ctx_lens[b]
        if wl.block_topk:
            s_row = oracle.index_scores(wl, rows=[b])[0]
        else:
            s_row = ref["scores"][r]
        msg = check_topk_row(got_idx[r], ref["idx"][r], s_row, n, wl.topk)
        assert msg == "", f"seq {b}: {msg}"
    ref_out = oracle.sparse_attn(wl, got_idx, rows=rows)
    err, msg = output_error(out.float().cpu().numpy()[rows], ref_out, tol)
    _say(f"  max abs output error {err:.3e} (tol {tol})")
    assert msg == "", msg
    return ref


def test_hand_worked_example_on_gpu():
    """The 8-token example embedded in the smallest supported widths (d_I 64, d 128): the
    extra coordinates are zero, so scores, selection and output are the fixture's values."""
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_8token.json")))
    n = 8
    kI = torch.zeros(n, 64)
    kI[:, :2] = torch.tensor(g["k_idx_logical"])
    q_idx = torch.zeros(1, 2, 64)
    q_idx[0, :, :2] = torch.tensor(g["q_idx"])
    K = torch.zeros(n, 1, 128)
    K[:, 0, 0] = torch.tensor(g["attn_c"])
    V = torch.zeros(n, 1, 128)
    V[:, 0, 0] = torch.arange(n).float()
    V[:, 0, 1] = 10 - torch.arange(n).float()
    q = torch.zeros(1, 1, 128)
    q[0, 0, :2] = torch.tensor(g["attn_q"])
    wl = custom_workload(ctx_lens=[n], page_size=4, q_lens=[1], q_idx=q_idx.to(torch.bfloat16),
                         w=torch.tensor([g["w"]]), idx_keys_logical=[kI.to(torch.bfloat16)],
                         q=q.to(torch.bfloat16), kv_logical=[K.to(torch.bfloat16)],
                         v_logical=[V.to(torch.bfloat16)], topk=3, softmax_scale=1.0)
    _say("hand example: page table " + str(wl.page_table.tolist()))
    dw = device.to_device(wl)
    s = device.index_score(dw)
    np.testing.assert_array_equal(s.cpu().numpy()[0], np.array(g["scores"], dtype=np.float32))
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert sorted(idx.cpu().numpy()[0].tolist()) == g["top3"]
    o = out.float().cpu().numpy()[0, 0]
    np.testing.assert_allclose(o[:2], g["out_sparse"], atol=2e-2)
    assert np.all(o[2:] == 0)
    assert binding.workspace_error(ws) == 0


def test_tiny_config_decode():
    wl = inputs.make("tiny")
    _say("tiny: B=1 ctx=4096 H_I=4 d_I=64 K=256 Hq=8 d=128")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    _check_decode(wl, out, idx, 2e-2)


@pytest.mark.parametrize("ctx", [[5000, 1, 64, 3000], [0, 2048, 2049, 2047], [131, 33, 7000, 65]])
def test_decode_mla_ragged_and_edges(ctx):
    wl = inputs.make("decode32k", num_seqs=len(ctx), ctx=ctx, seed_offset=len(ctx) + ctx[0])
    _say(f"decode MLA ctx={ctx}")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    _check_decode(wl, out, idx, 2e-2)
    for b, n in enumerate(ctx):
        if n == 0:
            assert np.all(idx.cpu().numpy()[b] == -1)
            assert np.all(out.float().cpu().numpy()[b] == 0)


@pytest.mark.parametrize("heads_q", [16, 40, 100])
def test_decode_latent_head_counts(heads_q):
    # latent rows with fewer query heads than a full workgroup, or than two full head groups:
    # waves past the last head load head 0 and store nothing, and the merge leaves those
    # heads alone (40: one head group of 64 with 24 idle heads; 100: a second group of 36)
    wl = inputs.make("decode32k", num_seqs=3, ctx=[5000, 700, 2048], heads_q=heads_q,
                     seed_offset=200 + heads_q)
    _say(f"decode latent rows, {heads_q} query heads")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out = torch.full((wl.num_seqs, heads_q, wl.dim_v), 7.0, dtype=torch.bfloat16, device="cuda")
    out, idx = device.decode_step(dw, ws, out=out)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    _check_decode(wl, out, idx, 2e-2)


@pytest.mark.parametrize("topk", [1, 1000, 8192])
def test_decode_unusual_k(topk):
    # K of one, K not a multiple of the 32-row tile, and K above both the candidate list and
    # the context of two of the sequences (every visible position, then -1)
    wl = inputs.make("decode32k", num_seqs=3, ctx=[20000, 5000, 700], topk=topk,
                     seed_offset=300 + topk)
    _say(f"decode K={topk}, ctx {wl.ctx_lens}")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    _check_decode(wl, out, idx, 2e-2)


@pytest.mark.parametrize("page_size", [1, 16, 256])
def test_decode_page_sizes(page_size):
    """The fused decode step at page sizes other than 64: one token per page (every key row and
    latent row its own page), 16 (a 16-token key tile is one page) and 256 (several tiles per
    page), on permuted pages."""
    wl = inputs.make("decode32k", num_seqs=3, ctx=[3000, 700, 4097], page_size=page_size,
                     seed_offset=60 + page_size)
    _say(f"decode page_size {page_size}, ctx {wl.ctx_lens}")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    _check_decode(wl, out, idx, 2e-2)


@pytest.mark.parametrize("ctx", [32768, 1])
def test_decode_single_sequence(ctx):
    """A batch of one sequence: at 32768 tokens the whole selection grid serves one sequence
    (many workgroups meet at its barriers); at one token the step has a single candidate."""
    wl = inputs.make("decode32k", num_seqs=1, ctx=[ctx], seed_offset=90 + ctx % 7)
    _say(f"decode B=1 ctx {ctx}")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    _check_decode(wl, out, idx, 2e-2)


def test_two_level_keeping_every_block_is_single_level():
    """When block_k is at least a sequence's block count, every block is kept and the two-level
    selection must be the single-level Top-K over the whole context."""
    wl = inputs.make("long1m", num_seqs=3, ctx=[8000, 5000, 2100], block_topk=128, seed_offset=81)
    _say(f"two-level keeping every block, ctx {wl.ctx_lens}")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    blocks = device.block_select(dw, ws).cpu().numpy()
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    got = idx.cpu().numpy()
    for b, n in enumerate(wl.ctx_lens):
        nblk = -(-n // wl.page_size)
        assert nblk <= wl.block_topk
        assert sorted(blocks[b][blocks[b] >= 0].tolist()) == list(range(nblk)), f"seq {b}"
        s_row = oracle.index_scores(wl, rows=[b])[0]
        ref = oracle.topk(s_row[None, :n], np.array([n]), wl.topk)[0]
        msg = check_topk_row(got[b], ref, s_row, n, wl.topk)
        assert msg == "", f"seq {b}: {msg}"
    err, msg = output_error(out.float().cpu().numpy(), oracle.sparse_attn(wl, got), 2e-2)
    _say(f"  max abs error {err:.3e}")
    assert msg == "", msg


def test_two_level_page_size_16():
    """Hierarchical selection with blocks of 16 tokens (a block is a page): blocks against the
    oracle's block scores, then tokens against the oracle's fine stage on the GPU's blocks."""
    wl = inputs.make("long1m", num_seqs=2, ctx=[20000, 3000], block_topk=64, page_size=16,
                     seed_offset=76)
    _say(f"two-level page_size 16, ctx {wl.ctx_lens}")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    blocks = device.block_select(dw, ws).cpu().numpy()
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    bs = oracle.block_scores(wl)
    nblk = [-(-n // wl.page_size) for n in wl.ctx_lens]
    ref_blocks = oracle.topk(bs, np.array(nblk), wl.block_topk)
    got = idx.cpu().numpy()
    ref_tok = oracle.topk_in_blocks(wl, blocks, k=wl.topk)
    P = wl.page_size
    for b, n in enumerate(wl.ctx_lens):
        msg = check_topk_row(blocks[b], ref_blocks[b], bs[b], nblk[b], wl.block_topk)
        assert msg == "", f"seq {b} blocks: {msg}"
        # 64 kept blocks of 16 tokens: at most 1024 candidates, fewer than K
        cand = np.zeros(n, dtype=bool)
        for j in blocks[b][blocks[b] >= 0]:
            cand[j * P:min((j + 1) * P, n)] = True
        msg = check_topk_in(got[b], ref_tok[b], oracle.index_scores(wl, rows=[b])[0], cand, wl.topk)
        assert msg == "", f"seq {b} tokens: {msg}"
    err, msg = output_error(out.float().cpu().numpy(), oracle.sparse_attn(wl, got), 2e-2)
    _say(f"  max abs error {err:.3e}")
    assert msg == "", msg


def test_index_score_matches_oracle():
    wl = inputs.make("decode32k", num_seqs=3, ctx=[4000, 100, 1500])
    _say("index_score decode B=3")
    dw = device.to_device(wl)
    s = device.index_score(dw).cpu().numpy()
    ref = oracle.index_scores(wl, ncols=s.shape[1])
    for b, n in enumerate(wl.ctx_lens):
        err = np.abs(s[b, :n] - ref[b, :n]).max()
        assert err <= 1e-4 * np.abs(ref[b, :n]).max(), (b, err)
        assert np.all(np.isneginf(s[b, n:]))


# Row Top-K runs the one-read kernel when the row stride is at most 65536 and the streaming
# kernel above that. The exact tests below run at three strides: the scores' own width (16-byte
# loads), 20001 (not a multiple of four: 4-byte loads) and 70000 (the streaming kernel); the
# wider strides pad the rows with -inf, which no row's visible range reaches.
TOPK_STRIDES = (None, 20001, 70000)


def _at_stride(s, ld):
    if ld is None:
        return s
    wide = np.full((s.shape[0], ld), -np.inf, dtype=np.float32)
    wide[:, :s.shape[1]] = s
    return wide


@pytest.mark.parametrize("ld", TOPK_STRIDES)
def test_topk_exact_on_shared_scores(ld):
    """Both sides select from identical fp32 scores: identical sets, including ties."""
    rng = np.random.default_rng(0)
    wl = inputs.make("decode32k", num_seqs=4, ctx=[9000, 2048, 100, 3000])
    dw = device.to_device(wl)
    s = rng.standard_normal((4, 9000)).astype(np.float32)
    s[1, :2048] = np.round(s[1, :2048])         # heavy ties
    s[2, :] = 0.0
    s[2, ::3] = -0.0                             # +-0 ties
    s[3, :3000] = rng.integers(-3, 3, 3000)      # ties at the threshold
    st = torch.from_numpy(_at_stride(s, ld)).cuda()
    idx = device.topk(dw, st, k=2048).cpu().numpy()
    ref = oracle.topk(s.astype(np.float64), np.array(wl.ctx_lens), 2048)
    np.testing.assert_array_equal(idx, ref)


@pytest.mark.parametrize("ld", TOPK_STRIDES)
def test_topk_crowded_threshold_bin(ld):
    """Row Top-K when one bin of the first digit holds a whole row (row 0: 20000 distinct scores
    in [1, 1.02), so all three digits are needed), with N(0,1) scores and ties broken by position
    (row 1), and with 7168 and 7169 keys in the first threshold bin (rows 2 and 3: the streaming
    kernel's LDS list capacity and one past it, where it re-reads the row)."""
    rng = np.random.default_rng(5)
    wl = inputs.make("decode32k", num_seqs=4, ctx=[20000, 12000, 9000, 9000])
    dw = device.to_device(wl)
    s = np.full((4, 20000), -np.inf, dtype=np.float32)
    s[0] = (1.0 + 0.02 * rng.permutation(20000) / 20000).astype(np.float32)
    s[1, :12000] = rng.standard_normal(12000).astype(np.float32)
    s[1, 100:600] = s[1, 50]                     # ties around a typical value
    for r, m in ((2, 7168), (3, 7169)):
        s[r, :9000] = (0.5 * rng.random(9000)).astype(np.float32)          # bins below [2, 2.5)
        sel = rng.permutation(9000)[:m]
        s[r, sel] = (2.0 + 0.4 * rng.permutation(m) / m).astype(np.float32)  # one first-digit bin
    st = torch.from_numpy(_at_stride(s, ld)).cuda()
    idx = device.topk(dw, st, k=2048).cpu().numpy()
    ref = oracle.topk(s.astype(np.float64), np.array(wl.ctx_lens), 2048)
    np.testing.assert_array_equal(idx, ref)


def test_topk_rows_at_the_register_kernel_limit():
    """Rows of exactly 65536 visible scores (the one-read kernel's limit), one of them with a
    crowded threshold bin and ties, one short row, and the same rows through the streaming kernel
    (stride 65537)."""
    rng = np.random.default_rng(9)
    wl = inputs.make("decode32k", num_seqs=3, ctx=[65536, 65536, 5], seed_offset=9)
    dw = device.to_device(wl)
    s = np.full((3, 65536), -np.inf, dtype=np.float32)
    s[0] = rng.standard_normal(65536).astype(np.float32)
    s[1] = np.round(rng.standard_normal(65536) * 4).astype(np.float32)  # few distinct values
    s[1, -3000:] = 1.0 + 1e-3 * rng.random(3000).astype(np.float32)     # the top bins, at the end
    s[2, :5] = rng.standard_normal(5).astype(np.float32)
    ref = oracle.topk(s.astype(np.float64), np.array(wl.ctx_lens), 2048)
    for ld in (65536, 65537):
        st = torch.from_numpy(_at_stride(s, ld if ld > 65536 else None)).cuda()
        idx = device.topk(dw, st, k=2048).cpu().numpy()
        np.testing.assert_array_equal(idx, ref, err_msg=f"stride {ld}")


@pytest.mark.parametrize("k", [2048, 2049, 4096, 8192])
def test_topk_full_rows_large_k(k):
    """Rows of 65536 scores on both sides of the one-read kernel's switch at k = 2048 (four
    workgroups per CU up to it, two above), and rows whose candidate list overflows the larger
    list, which take the streaming selection (k = 8192); with 16-byte and 4-byte loads."""
    rng = np.random.default_rng(40 + k)
    wl = inputs.make("decode32k", num_seqs=3, ctx=[65536, 65536, 40000], seed_offset=40)
    dw = device.to_device(wl)
    s = np.full((3, 65536), -np.inf, dtype=np.float32)
    s[0] = rng.standard_normal(65536).astype(np.float32)
    s[1] = (rng.standard_normal(65536) * np.linspace(0.5, 2.0, 65536)).astype(np.float32)
    s[2, :40000] = np.round(rng.standard_normal(40000) * 8).astype(np.float32)  # ties
    # stride 65536: 16-byte loads; 65533 (not a multiple of four; the rows cut there): 4-byte loads
    for ld in (65536, 65533):
        sl = np.ascontiguousarray(s[:, :ld])
        ref = oracle.topk(sl.astype(np.float64), np.minimum(np.array(wl.ctx_lens), ld), k)
        idx = device.topk(dw, torch.from_numpy(sl).cuda(), k=k).cpu().numpy()
        np.testing.assert_array_equal(idx, ref, err_msg=f"stride {ld}")


def test_topk_rows_with_large_scores_in_one_region():
    """Rows of 65536 whose largest scores gather in one region, as recent positions may: a rising
    trend with noise, a strictly increasing row, and a row whose Top-2048 lie in its last 2500
    positions (the sample must see the region for the one-read path; the result is exact on
    either path)."""
    rng = np.random.default_rng(77)
    n = 65536
    wl = inputs.make("decode32k", num_seqs=3, ctx=[n, n, n], seed_offset=77)
    dw = device.to_device(wl)
    s = np.empty((3, n), dtype=np.float32)
    s[0] = (np.linspace(0.0, 6.0, n) + rng.standard_normal(n)).astype(np.float32)
    s[1] = np.linspace(-1.0, 1.0, n).astype(np.float32)
    s[2] = rng.standard_normal(n).astype(np.float32)
    s[2, -2500:] = (5.0 + rng.random(2500)).astype(np.float32)
    ref = oracle.topk(s.astype(np.float64), np.array(wl.ctx_lens), 2048)
    idx = device.topk(dw, torch.from_numpy(s).cuda(), k=2048).cpu().numpy()
    np.testing.assert_array_equal(idx, ref)


def test_sparse_attn_on_oracle_indices():
    wl = inputs.make("decode32k", num_seqs=3, ctx=[3000, 40, 2100])
    dw = device.to_device(wl)
    ref = oracle.decode_step(wl)
    idx = torch.from_numpy(ref["idx"]).cuda()
    ws = device.new_workspace(dw)
    out = device.sparse_attn(dw, idx, ws).float().cpu().numpy()
    err, msg = output_error(out, ref["out"], 2e-2)
    _say(f"  sparse_attn max abs error {err:.3e}")
    assert msg == "", msg


def test_prefill_path_small():
    wl = inputs.make("prefill64k", ctx=3000, q_len=48)
    _say("prefill: ctx 3000, 48 query rows")
    dw = device.to_device(wl)
    s = device.index_score(dw).cpu().numpy()
    ref_s = oracle.index_scores(wl, ncols=s.shape[1])
    pos = wl.q_pos().numpy()
    for r in range(wl.num_queries):
        n = pos[r] + 1
        err = np.abs(s[r, :n] - ref_s[r, :n]).max()
        assert err <= 1e-4 * np.abs(ref_s[r, :n]).max()
    idx = device.topk(dw, torch.from_numpy(s).cuda()).cpu().numpy()
    ref_idx = oracle.topk(s.astype(np.float64), pos + 1, wl.topk)
    np.testing.assert_array_equal(idx, ref_idx)
    ws = device.new_workspace(dw)
    out = device.sparse_attn(dw, torch.from_numpy(idx).cuda(), ws).float().cpu().numpy()
    ref_out = oracle.sparse_attn(wl, idx)
    err, msg = output_error(out, ref_out, 2e-2)
    _say(f"  prefill attention max abs error {err:.3e}")
    assert msg == "", msg


@pytest.mark.parametrize("dtype", ["fp8", "fp8t128"])
def test_prefill_path_fp8(dtype):
    """Prefill rows over E4M3 caches: E4M3 indexer keys with row scales and E4M3 latent rows
    with row scales (fp8), or bf16 keys and latent rows with a scale per 128-entry tile
    (fp8t128). Scores against the oracle on the same codes, the row Top-K exact on the GPU's
    scores, the attention within the fp8 tolerance."""
    wl = inputs.make("prefill64k", ctx=2500, q_len=40, dtype=dtype, seed_offset=21)
    _say(f"prefill {dtype}: ctx 2500, 40 query rows")
    dw = device.to_device(wl)
    s = device.index_score(dw).cpu().numpy()
    ref_s = oracle.index_scores(wl, ncols=s.shape[1])
    pos = wl.q_pos().numpy()
    for r in range(wl.num_queries):
        n = pos[r] + 1
        err = np.abs(s[r, :n] - ref_s[r, :n]).max()
        assert err <= 1e-4 * np.abs(ref_s[r, :n]).max(), (r, err)
    idx = device.topk(dw, torch.from_numpy(s).cuda()).cpu().numpy()
    np.testing.assert_array_equal(idx, oracle.topk(s.astype(np.float64), pos + 1, wl.topk))
    ws = device.new_workspace(dw)
    out = device.sparse_attn(dw, torch.from_numpy(idx).cuda(), ws).float().cpu().numpy()
    err, msg = output_error(out, oracle.sparse_attn(wl, idx), 5e-2)
    _say(f"  attention max abs error {err:.3e}")
    assert msg == "", msg


def test_prefill_batch_of_sequences():
    # several sequences in one prefill call: a short one, one with no new rows, a long one,
    # and one made only of new rows (no prefix); row blocks of the indexer GEMM never span two
    # sequences, and every row sees its own sequence's history only
    wl = inputs.make("prefill64k", num_seqs=4, ctx=[700, 500, 3000, 129], q_len=[5, 0, 40, 129],
                     seed_offset=21)
    _say(f"prefill batch: ctx {wl.ctx_lens}, rows {wl.q_lens}")
    dw = device.to_device(wl)
    s = device.index_score(dw).cpu().numpy()
    ref_s = oracle.index_scores(wl, ncols=s.shape[1])
    pos = wl.q_pos().numpy()
    assert s.shape[0] == wl.num_queries == 174
    for r in range(wl.num_queries):
        n = pos[r] + 1
        err = np.abs(s[r, :n] - ref_s[r, :n]).max()
        assert err <= 1e-4 * np.abs(ref_s[r, :n]).max(), r
        assert np.all(np.isneginf(s[r, n:])), r  # past the row's own position
    idx = device.topk(dw, torch.from_numpy(s).cuda()).cpu().numpy()
    ref_idx = oracle.topk(s.astype(np.float64), pos + 1, wl.topk)
    np.testing.assert_array_equal(idx, ref_idx)
    ws = device.new_workspace(dw)
    out = device.sparse_attn(dw, torch.from_numpy(idx).cuda(), ws).float().cpu().numpy()
    ref_out = oracle.sparse_attn(wl, idx)
    err, msg = output_error(out, ref_out, 2e-2)
    _say(f"  prefill batch attention max abs error {err:.3e}")
    assert msg == "", msg


def test_fp8_ragged_small():
    wl = inputs.make("fp8ragged", num_seqs=5, ctx=[4096, 9000, 300, 2048, 5000])
    _say("fp8 ragged B=5")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    _check_decode(wl, out, idx, 5e-2)


def test_two_level_small():
    """Blocks first (near-tie rule at block level), then tokens against the oracle's fine stage
    on the GPU's kept blocks; a partial last block and a sequence with fewer blocks than
    block_k are included."""
    wl = inputs.make("long1m", num_seqs=3, ctx=[40000, 9000, 3000], block_topk=64)
    _say("two-level B=3 ctx 40000/9000/3000, 64 blocks")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    blocks = device.block_select(dw, ws).cpu().numpy()
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    bs = oracle.block_scores(wl)
    nblk = [-(-n // wl.page_size) for n in wl.ctx_lens]
    ref_blocks = oracle.topk(bs, np.array(nblk), wl.block_topk)
    got = idx.cpu().numpy()
    ref_tok = oracle.topk_in_blocks(wl, blocks, k=wl.topk)
    for b, n in enumerate(wl.ctx_lens):
        msg = check_topk_row(blocks[b], ref_blocks[b], bs[b], nblk[b], wl.block_topk)
        assert msg == "", f"seq {b} blocks: {msg}"
        s_row = oracle.index_scores(wl, rows=[b])[0]
        msg = check_topk_row(got[b], ref_tok[b], s_row, n, wl.topk)
        assert msg == "", f"seq {b} tokens: {msg}"
    assert np.all(blocks[2, nblk[2]:] == -1)
    err, msg = output_error(out.float().cpu().numpy(), oracle.sparse_attn(wl, got), 2e-2)
    _say(f"  two-level max abs error {err:.3e}")
    assert msg == "", msg


def test_decode_is_deterministic():
    wl = inputs.make("decode32k", num_seqs=4, ctx=[6000, 3000, 2049, 100])
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    o1, i1 = device.decode_step(dw, ws)
    o2, i2 = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(o1, o2)


def test_page_permutation_invariance_gpu():
    a = inputs.make("decode32k", num_seqs=2, ctx=[3000, 1000])
    # same logical content under another page table: permute physical pages
    perm = torch.randperm(a.num_pages, generator=torch.Generator().manual_seed(7))
    inv = torch.argsort(perm)
    b = inputs.make("decode32k", num_seqs=2, ctx=[3000, 1000])
    b.page_table = perm[a.page_table.long()].to(torch.int32)
    b.idx_keys = a.idx_keys[inv]
    b.k_cache = a.k_cache[inv]
    outs = []
    for wl in (a, b):
        dw = device.to_device(wl)
        ws = device.new_workspace(dw)
        outs.append(device.decode_step(dw, ws))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][0], outs[1][0])


def test_decode_all_scores_equal():
    """Zero indexer queries: every score is 0, so the selection is the lowest positions. The
    long sequence's threshold bin overflows the candidate list (radix passes); the others are
    resolved through the list."""
    wl = inputs.make("decode32k", num_seqs=3, ctx=[9000, 3000, 2053], seed_offset=11)
    wl.q_idx = torch.zeros_like(wl.q_idx)
    _say("decode: all scores equal, ctx 9000/3000/2053")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    got = idx.cpu().numpy()
    for b in range(3):
        np.testing.assert_array_equal(got[b], np.arange(wl.topk, dtype=np.int32))
    err, msg = output_error(out.float().cpu().numpy(), oracle.sparse_attn(wl, got), 2e-2)
    assert msg == "", msg


def test_decode_exact_integer_scores_with_ties():
    """Keys and queries in {-1, 0, 1} and w = 1/4: every score is exact in fp32 and fp64, with
    many ties at the threshold, so the index sets must equal the oracle's exactly (lower
    positions win ties) on both the list path and the radix-pass path."""
    wl = inputs.make("decode32k", num_seqs=4, ctx=[70000, 20000, 5000, 3001], seed_offset=12)
    g = torch.Generator().manual_seed(99)
    wl.idx_keys = torch.randint(-1, 2, wl.idx_keys.shape, generator=g).to(torch.bfloat16)
    wl.q_idx = torch.randint(-1, 2, wl.q_idx.shape, generator=g).to(torch.bfloat16)
    wl.w = torch.full_like(wl.w, 0.25)
    _say("decode: integer scores with ties, ctx 70000/20000/5000/3001")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    ref = oracle.decode_step(wl)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"])
    err, msg = output_error(out.float().cpu().numpy(), ref["out"], 2e-2)
    assert msg == "", msg


def test_decode_batch_larger_than_one_selection_launch():
    """300 sequences (more than half the resident capacity of the selection kernel, so the
    batch runs as several launches) with mixed short lengths, including empty ones."""
    rng = np.random.default_rng(5)
    ctx = [int(x) for x in rng.integers(1, 3000, 300)]
    ctx[7] = 0
    ctx[150] = 2048
    wl = inputs.make("decode32k", num_seqs=300, ctx=ctx, seed_offset=13)
    _say("decode: B=300, ctx 0..3000")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    _check_decode(wl, out, idx, 2e-2)


def test_prefill_large_k_splits_rows():
    """K = 4096 over 300 prefill rows: many rows fill the device, yet each row's index set is
    split (at most 2048 selected rows per attention workgroup), exercising the merge."""
    wl = inputs.make("prefill64k", ctx=6000, q_len=300, topk=4096, seed_offset=14)
    _say("prefill: ctx 6000, 300 rows, K=4096")
    dw = device.to_device(wl)
    s = device.index_score(dw)
    idx = device.topk(dw, s)
    ws = device.new_workspace(dw)
    out = device.sparse_attn(dw, idx, ws).float().cpu().numpy()
    got = idx.cpu().numpy()
    pos = wl.q_pos().numpy()
    ref_idx = oracle.topk(s.cpu().numpy().astype(np.float64), pos + 1, wl.topk)
    np.testing.assert_array_equal(got, ref_idx)
    err, msg = output_error(out, oracle.sparse_attn(wl, got), 2e-2)
    _say(f"  max abs output error {err:.3e}")
    assert msg == "", msg


def test_decode_long_contexts_fill_a_selection_launch():
    """128 sequences of 64000 tokens: with one workgroup per sequence plus the spare ones, a
    workgroup's share would not fit the LDS of a CU, so the batch runs as smaller launches
    with more workgroups per sequence. Small head shapes keep the inputs at a few GB."""
    _say("decode: B=128, ctx 64000, 4 indexer heads, 8 query heads, K=256")
    wl = inputs.make("decode32k", num_seqs=128, ctx=64000, idx_heads=4, idx_dim=64, topk=256,
                     heads_q=8, dim_qk=128, dim_v=128, seed_offset=15)
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    _check_decode(wl, out, idx, 2e-2, rows=[0, 1, 63, 64, 127])
