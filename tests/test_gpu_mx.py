"""GPU parity of the MXFP8 indexer (E4M3 key codes with one E8M0 exponent per 32 entries; the
library quantizes the bf16 query per 32 entries itself) against the CPU oracle.

Scores: |s_gpu - s_oracle| <= 1e-4 * max_t |s_oracle| per row. Both sides use the same key codes
(the generator's), the oracle quantizes the query in its own code; one query entry rounded to a
different E4M3 code moves a score by far more than the tolerance, so the bound also checks that
the two quantizations agree. Index sets and attention outputs: the acceptance rules of the
other decode tests (near ties at the K-th score; 5e-2 on outputs over E4M3 KV).
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


def _check_scores(wl, s):
    ref = oracle.index_scores(wl, ncols=s.shape[1])
    pos = wl.q_pos().numpy()
    for r in range(wl.num_queries):
        n = int(pos[r]) + 1  # positions 0 .. the row's own (none when the sequence is empty)
        if n == 0:
            assert np.all(np.isneginf(s[r])), r
            continue
        err = np.abs(s[r, :n] - ref[r, :n]).max()
        scale = np.abs(ref[r, :n]).max()
        assert err <= 1e-4 * scale, (r, err, scale)
        assert np.all(np.isneginf(s[r, n:])), r


def _scores(wl):
    dw = device.to_device(wl)
    return device.index_score(dw).cpu().numpy()


def test_mx_index_score_matches_oracle():
    wl = inputs.make("mxfp8ragged", num_seqs=5, ctx=[4096, 300, 9000, 17, 0])
    _say("MXFP8 index_score B=5 (64 heads, d_I 128), ctx 4096/300/9000/17/0")
    _check_scores(wl, _scores(wl))


@pytest.mark.parametrize("heads,dim", [(12, 64), (64, 64), (5, 128)])
def test_mx_index_score_heads_and_dims(heads, dim):
    wl = inputs.make("mxfp8ragged", num_seqs=3, ctx=[2000, 65, 1025], idx_heads=heads,
                     idx_dim=dim)
    _say(f"MXFP8 index_score heads {heads} d_I {dim}")
    _check_scores(wl, _scores(wl))


def _edge_queries(wl):
    """Query rows whose quantization hits the rounding and range corners: an all-zero block,
    saturation, ties between E4M3 neighbours (normal and subnormal, both signs), a whole row
    near the bottom and one near the top of the exponent range."""
    q = wl.q_idx.float().clone()
    row = q[0, 0]
    row[0:32] = 0.0                                 # all-zero block: E8M0 0, codes 0
    blk = torch.zeros(32)
    # amax 464 -> X = 0: 464 saturates to 448; 1.0625 ties to 1.0, 17 to 16, 19 to 20,
    # -1.1875 to -1.25; 3 * 2^-10 ties to 2 * 2^-9 (subnormal), 2^-10 to 0, -2^-10 to -0
    vals = [464.0, 1.0625, 17.0, 19.0, -1.1875, 3 * 2.0 ** -10, 2.0 ** -10, -2.0 ** -10,
            -300.0, 255.0, 0.5, -0.03125]
    blk[:len(vals)] = torch.tensor(vals)
    row[32:64] = blk
    q[0, 1] = 0.0                                    # a head of zeros
    q[1] = q[1] * 2.0 ** -100                        # exponents near the bottom of the range
    q[2] = q[2] * 2.0 ** 60                          # and far above the keys'
    return dataclasses.replace(wl, q_idx=q.to(torch.bfloat16))


def test_mx_query_quantization_edges():
    wl = _edge_queries(inputs.make("mxfp8ragged", num_seqs=3, ctx=[3000, 1500, 700]))
    _say("MXFP8 index_score: query quantization corners")
    _check_scores(wl, _scores(wl))


def test_mx_prefill_rows():
    wl = inputs.make("mxfp8ragged", num_seqs=1, ctx=2500, q_len=40)
    _say("MXFP8 index_score: 40 prefill rows over ctx 2500")
    _check_scores(wl, _scores(wl))


def _check_decode(wl, out, idx, tol):
    ref = oracle.decode_step(wl)
    got = idx.cpu().numpy()
    for b in range(wl.num_seqs):
        msg = check_topk_row(got[b], ref["idx"][b], ref["scores"][b], wl.ctx_lens[b], wl.topk)
        assert msg == "", f"seq {b}: {msg}"
    ref_out = oracle.sparse_attn(wl, got)
    err, msg = output_error(out.float().cpu().numpy(), ref_out, tol)
    _say(f"  max abs output error {err:.3e} (tol {tol})")
    assert msg == "", msg


@pytest.mark.parametrize("ctx,heads,dim", [([4096, 9000, 300, 2048, 5000], 64, 128),
                                           ([1, 2048, 2049, 2047, 7000], 12, 64)])
def test_mx_decode_small(ctx, heads, dim):
    wl = inputs.make("mxfp8ragged", num_seqs=len(ctx), ctx=ctx, idx_heads=heads, idx_dim=dim)
    _say(f"MXFP8 decode B={len(ctx)} heads {heads} d_I {dim}")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    _check_decode(wl, out, idx, 5e-2)


def test_mx_decode_query_edges():
    wl = _edge_queries(inputs.make("mxfp8ragged", num_seqs=3, ctx=[6000, 2100, 2600]))
    _say("MXFP8 decode: query quantization corners")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    _check_decode(wl, out, idx, 5e-2)


def test_mx_full_size_sampled_rows():
    """The full ragged batch (64 sequences, 4K-128K) in the benchmark's launch configuration;
    the oracle checks a sample of rows (the shortest, the longest and a few between)."""
    wl = inputs.make("mxfp8ragged")
    _say(f"MXFP8 decode full size: B={wl.num_seqs}, ctx {min(wl.ctx_lens)}..{max(wl.ctx_lens)}")
    dw = device.to_device(wl)
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    assert binding.workspace_error(ws) == 0
    order = np.argsort(wl.ctx_lens)
    rows = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2]), 7, 33})
    ref = oracle.decode_step(wl, rows=rows)
    got = idx.cpu().numpy()[rows]
    for r, b in enumerate(rows):
        msg = check_topk_row(got[r], ref["idx"][r], ref["scores"][r], wl.ctx_lens[b], wl.topk)
        assert msg == "", f"seq {b}: {msg}"
    ref_out = oracle.sparse_attn(wl, got, rows=rows)
    err, msg = output_error(out.float().cpu().numpy()[rows], ref_out, 5e-2)
    _say(f"  sampled rows {rows}: max abs output error {err:.3e}")
    assert msg == "", msg


@pytest.mark.parametrize("spread", [0, 6])
def test_fp8_tile_kv_attention_on_oracle_indices(spread):
    """sa_sparse_attn over E4M3 latent rows with one scale per 128 entries, on the oracle's own
    index sets. spread > 0 multiplies every (row, tile) scale by 2^U[-spread, spread], so that
    neighbouring tiles of a row differ by up to 2^(2 spread): a wrong tile index or a scale
    applied to the wrong partial sum moves the output by far more than the bound, which is
    relative to the largest output (bf16 rounding of P and of the output)."""
    wl = inputs.make("mxfp8ragged", num_seqs=3, ctx=[3000, 40, 2100])
    if spread:
        g = torch.Generator().manual_seed(17)
        e = torch.randint(-spread, spread + 1, wl.kv_scale.shape, generator=g)
        wl = dataclasses.replace(wl, kv_scale=(wl.kv_scale * torch.pow(2.0, e.float())).contiguous())
    _say(f"E4M3 tile-128 KV attention, scale spread 2^+-{spread}")
    dw = device.to_device(wl)
    ref = oracle.decode_step(wl)
    idx = torch.from_numpy(ref["idx"]).cuda()
    ws = device.new_workspace(dw)
    out = device.sparse_attn(dw, idx, ws).float().cpu().numpy()
    want = oracle.sparse_attn(wl, ref["idx"])
    err = np.abs(out - want).max()
    bound = 1e-2 * np.abs(want).max()
    _say(f"  max abs error {err:.3e} (bound {bound:.3e})")
    assert err <= bound


def test_mx_two_level_is_rejected():
    wl = inputs.make("mxfp8ragged", num_seqs=2, ctx=[3000, 4000])
    dw = device.to_device(wl)
    ws = binding.new_workspace(dw.batch, dw.kv, wl.topk, 16, device=dw.t["q"].device)
    with pytest.raises(binding.SaError) as e:
        binding.decode_step(dw.batch, dw.ix, dw.kv, dw.t["q_idx"], dw.t["w"], dw.t["q"],
                            wl.topk, torch.empty((2, wl.heads_q, wl.dim_v), dtype=torch.bfloat16,
                                                 device="cuda"), ws, block_k=16)
    assert e.value.status == binding.SA_ERR_UNSUPPORTED
