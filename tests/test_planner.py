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


def _check_latent(rows, k, cap, recs):
    splits, slen, merge, grid = B.plan_latent_attention(rows, k, cap, recs)
    if splits == 0:
        return None
    assert slen % 32 == 0 and 32 <= slen <= 2048
    assert splits * slen >= k
    assert (merge == 0) == (splits == 1)
    if merge == 2:
        assert rows % 8 == 0
        assert grid == 8 * splits * (rows // 8)
    else:
        assert grid == rows * splits
    if merge:
        assert grid <= cap and rows <= recs
    return splits, slen, merge, grid


def test_latent_attention_plan_for_the_workloads(lib):
    # decode: 32 rows x 2048 selected rows, 256 CUs: 8 splits of 256 rows, on one XCD per row
    assert _check_latent(32, 2048, 256, 32) == (8, 256, 2, 256)
    # prefill: 4096 rows, one split each, no merge
    assert _check_latent(4096, 2048, 256, 4096) == (1, 2048, 0, 4096)
    # more selected rows than one split holds, and too many rows to merge resident: the other
    # kernel runs
    assert _check_latent(300, 4096, 256, 4096) is None
    # no merge records: only an unsplit launch qualifies
    assert _check_latent(32, 2048, 256, 0) == (1, 2048, 0, 32)


def test_latent_attention_plan_properties(lib):
    for rows in list(range(1, 40)) + [64, 100, 128, 255, 256, 257, 4096]:
        for k in (1, 31, 100, 128, 129, 2047, 2048, 2049, 4096, 65536):
            for cap in (0, 100, 256, 512):
                for recs in (0, rows, 4096):
                    _check_latent(rows, k, cap, recs)
