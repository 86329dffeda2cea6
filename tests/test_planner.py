"""Host-only launch planning (no GPU): the capacity arithmetic of the kernels whose workgroups
wait for each other. A merging or selecting grid larger than what the device holds at once
could wait forever (until the spin limit), so these properties are what keeps those launches
correct: every workgroup fits, every sequence stays within its record, and the plan is the
tightest one that does."""
import os
import random

import pytest

from indexer_top_sparse_amd import binding as B


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return B.load()


def _groups(nc, chunk):
    return -(-nc // chunk) if nc > 0 else 1


def _check_selection(ncand, cap):
    chunk, groups = B.plan_selection(ncand, cap)
    assert chunk >= 64 and chunk % 64 == 0
    per_seq = [_groups(n, chunk) for n in ncand]
    assert groups == sum(per_seq)
    assert groups <= cap, (chunk, groups, cap)
    assert max(per_seq) <= 512
    # the smallest such chunk: 64 less breaks one of the two limits
    if chunk > 64:
        smaller = [_groups(n, chunk - 64) for n in ncand]
        assert sum(smaller) > cap or max(smaller) > 512
    return chunk, groups


def test_selection_plan_for_the_decode_workload(lib):
    # 32 sequences of 32768 tokens on 256 CUs holding 2 selection workgroups each
    assert _check_selection([32768] * 32, 512) == (2048, 512)
    # one workgroup per CU: twice the chunk
    assert _check_selection([32768] * 32, 256) == (4096, 256)


def test_selection_plan_properties(lib):
    rng = random.Random(5)
    cases = [([0] * 7, 7), ([1], 1), ([1048576], 512), ([1048576] * 4, 512),
             ([1048576] * 4, 2048), ([16384] * 64, 64), ([16] * 100, 100)]
    for _ in range(200):
        n = rng.randint(1, 128)
        ncand = [int(rng.choice([0, 1, 63, 64, 65]) if rng.random() < 0.2
                     else int(2 ** rng.uniform(0, 20))) for _ in range(n)]
        cases.append((ncand, rng.randint(n, 1024)))
    for ncand, cap in cases:
        _check_selection(ncand, cap)


def test_selection_plan_rejects_what_cannot_fit(lib):
    with pytest.raises(B.SaError):
        B.plan_selection([100] * 9, 8)  # fewer resident workgroups than sequences
    with pytest.raises(B.SaError):
        B.plan_selection([-1], 8)


def _check_latent(rows, k, cap, recs, heads=128):
    splits, slen, hg, merge, grid = B.plan_latent_attention(rows, k, heads, cap, recs)
    if splits == 0:
        return None
    assert hg in (1, 2) and (hg == 1 or heads > 64)
    # 64 heads per workgroup (a row of at most 64 heads, or two head groups) hold at most 1024
    # rows per split in LDS, 128 heads per workgroup 2048
    two_phase = heads <= 64 or hg == 2
    assert slen % 32 == 0 and 32 <= slen <= (1024 if two_phase else 2048)
    assert splits * slen >= k
    assert (merge == 0) == (splits == 1)
    units = hg * splits
    if units > 1:  # the workgroups of a row share an XCD: row r's indices are r mod 8
        assert grid == 8 * units * -(-rows // 8)
    else:
        assert grid == rows
    if merge:
        assert grid <= cap and rows * hg <= recs
    return splits, slen, hg, merge, grid


def test_latent_attention_plan_for_the_workloads(lib):
    # decode: 32 rows x 2048 selected rows, 128 heads, 256 CUs: two head groups of 64 and 4
    # splits of 512 rows per row, the 8 workgroups of a row on one XCD
    assert _check_latent(32, 2048, 256, 64) == (4, 512, 2, 1, 256)
    # prefill: 4096 rows, one workgroup of 128 heads each, no merge
    assert _check_latent(4096, 2048, 256, 8192) == (1, 2048, 1, 0, 4096)
    # more selected rows than one split holds, and too many rows to merge resident: the other
    # kernel runs
    assert _check_latent(300, 4096, 256, 8192) is None
    # no merge records: only an unsplit launch qualifies, and 2048 rows need two splits of 64
    # heads, so the other kernel runs; 1024 rows fit one split
    assert _check_latent(32, 2048, 256, 0) is None
    assert _check_latent(32, 1024, 256, 0) == (1, 1024, 2, 0, 64)
    # at most 64 heads: one head group, all waves busy in two tile phases
    assert _check_latent(32, 2048, 256, 64, heads=64) == (8, 256, 1, 1, 256)


def test_latent_attention_plan_properties(lib):
    for rows in list(range(1, 40)) + [64, 100, 128, 255, 256, 257, 4096]:
        for k in (1, 31, 100, 128, 129, 1025, 2047, 2048, 2049, 4096, 65536):
            for cap in (0, 100, 256, 512):
                for recs in (0, rows, 2 * rows, 8192):
                    for heads in (16, 64, 65, 128):
                        _check_latent(rows, k, cap, recs, heads)
