"""GPU side of the paged cache allocator: whole-page copies (sa_copy_pages) are bit-exact in
every cache table, and a decode step over page tables made by the pool (a forked sequence whose
shared last page was copied on write, then one new token appended to each) matches the oracle
run on the same caches; the forked sequence still reads its parent's prefix.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from indexer_top_sparse_amd import binding, device, inputs
from tests._util import check_topk_row, output_error

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()


@pytest.mark.parametrize("preset,over", [
    ("mxfp8ragged", dict(num_seqs=2, ctx=[4100, 4500])),
    ("fp8ragged", dict(num_seqs=2, ctx=[4100, 4500])),
    ("long1m", dict(num_seqs=2, ctx=[3000, 5000], block_topk=4)),
    ("tiny", dict(num_seqs=2, ctx=[300, 200])),
])
def test_copy_pages_is_bit_exact(preset, over):
    wl = inputs.make(preset, **over)
    dw = device.to_device(wl)
    rng = np.random.default_rng(3)
    pages = rng.permutation(wl.num_pages)[:2 * min(8, wl.num_pages // 2)].reshape(-1, 2)
    before = {k: v.clone() for k, v in dw.t.items()}
    pairs = torch.from_numpy(pages.astype(np.int32)).cuda()
    binding.copy_pages(dw.ix, dw.kv, wl.page_size, pairs)
    torch.cuda.synchronize()
    for name in ("idx_keys", "idx_scale", "idx_mx_scale", "pooled", "k_cache", "v_cache", "kv_scale"):
        if name not in dw.t:
            continue
        want = before[name].clone()
        for s, d in pages:
            want[d] = before[name][s]
        assert np.array_equal(_bits(dw.t[name]), _bits(want)), name


def test_decode_over_pool_page_tables_with_copy_on_write():
    P, n0 = 64, 300
    base = inputs.make("decode32k", num_seqs=2, ctx=[n0 + 1, n0 + 1])
    pool = binding.Pool(base.num_pages, P)
    a = pool.new()
    pool.reserve(a, n0)
    g = torch.Generator().manual_seed(5)
    # the prefix: n0 tokens of sequence a, written through the pool's page table
    keys = torch.zeros_like(base.idx_keys)
    kvc = torch.zeros_like(base.k_cache)
    pa = pool.page_table(a)
    pref_k = torch.randn((n0, base.idx_dim), generator=g).to(torch.bfloat16)
    pref_kv = torch.randn((n0, 1, base.dim_qk), generator=g).to(torch.bfloat16)
    for t in range(n0):
        keys[pa[t // P], t % P] = pref_k[t]
        kvc[pa[t // P], t % P] = pref_kv[t]
    b = pool.fork(a)
    cow_b = pool.reserve(b, n0 + 1)          # b's next token lands in the shared last page
    cow_a = pool.reserve(a, n0 + 1)          # a's copy of that page is no longer shared
    assert len(cow_b) == 1 and not cow_a
    pt = torch.zeros((2, base.pages_per_seq), dtype=torch.int32)
    for i, s in enumerate((a, b)):
        tbl = pool.page_table(s)
        pt[i, :len(tbl)] = torch.tensor(tbl, dtype=torch.int32)
    wl = dataclasses.replace(base, page_table=pt, idx_keys=keys, k_cache=kvc)
    dw = device.to_device(wl)
    binding.copy_pages(dw.ix, dw.kv, P, torch.tensor(cow_b, dtype=torch.int32).cuda())
    new_k = torch.randn((2, base.idx_dim), generator=g).to(torch.bfloat16)
    new_kv = torch.randn((2, 1, base.dim_qk), generator=g).to(torch.bfloat16)
    binding.cache_append(dw.batch, dw.ix, dw.kv, new_k.cuda(), new_kv.cuda())
    ws = device.new_workspace(dw)
    out, idx = device.decode_step(dw, ws)
    torch.cuda.synchronize()
    fin = dataclasses.replace(wl, idx_keys=dw.t["idx_keys"].cpu(), k_cache=dw.t["k_cache"].cpu())
    # both sequences read the prefix, then their own token
    for i in range(2):
        tbl = pt[i].tolist()
        got = torch.stack([fin.idx_keys[tbl[t // P], t % P] for t in range(n0 + 1)])
        assert torch.equal(got[:n0], pref_k) and torch.equal(got[n0], new_k[i])
    ref = oracle.decode_step(fin)
    gi = idx.cpu().numpy()
    for i in range(2):
        assert check_topk_row(gi[i], ref["idx"][i], ref["scores"][i], n0 + 1, fin.topk) == ""
    err, msg = output_error(out.float().cpu().numpy(), oracle.sparse_attn(fin, gi), 2e-2)
    print(f"  decode over pool page tables: max abs output error {err:.3e}", flush=True)
    assert msg == "", msg
