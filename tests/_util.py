"""Helpers shared by the tests: hand-built workloads and the acceptance comparators."""
from __future__ import annotations

import math

import numpy as np
import torch

from indexer_top_sparse_amd.inputs import Workload


def to_bf16(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def paged_from_logical(per_seq_rows, page_size, perm_seed=0):
    """Scatter per-sequence logical rows [n_b, ...] into a paged cache [pages, P, ...].

    Logical page j of sequence b is stored at physical page perm[k] (k counts pages over
    sequences in order). Returns (cache, page_table int32 [B, max_pages], num_pages)."""
    B = len(per_seq_rows)
    npg = [math.ceil(r.shape[0] / page_size) for r in per_seq_rows]
    num_pages = max(1, sum(npg))
    g = torch.Generator().manual_seed(perm_seed)
    perm = torch.randperm(num_pages, generator=g)
    tail = per_seq_rows[0].shape[1:]
    cache = torch.zeros((num_pages, page_size) + tuple(tail), dtype=per_seq_rows[0].dtype)
    pt = torch.zeros((B, max(1, max(npg))), dtype=torch.int32)
    k = 0
    for b, rows in enumerate(per_seq_rows):
        for j in range(npg[b]):
            blk = rows[j * page_size:(j + 1) * page_size]
            cache[perm[k], :blk.shape[0]] = blk
            pt[b, j] = int(perm[k])
            k += 1
    return cache, pt, num_pages


def custom_workload(*, ctx_lens, page_size, q_lens, q_idx, w, idx_keys_logical, q,
                    kv_logical, v_logical=None, topk, block_topk=0, pooled_logical=None,
                    softmax_scale, perm_seed=0, idx_dtype="bf16", idx_scale_logical=None,
                    kv_dtype="bf16", kv_scale_logical=None, dim_v=None) -> Workload:
    """Build a Workload from per-sequence logical tensors (lists indexed by sequence).

    idx_keys_logical[b]: [n_b, d_I]; kv_logical[b]: [n_b, H_kv, k_row]; v_logical[b]:
    [n_b, H_kv, d_v] or None when V aliases the first dim_v entries of each K row."""
    keys, pt, num_pages = paged_from_logical(idx_keys_logical, page_size, perm_seed)
    kc, pt2, _ = paged_from_logical(kv_logical, page_size, perm_seed)
    assert torch.equal(pt, pt2)
    vc = None
    if v_logical is not None:
        vc, _, _ = paged_from_logical(v_logical, page_size, perm_seed)
    iscale = None
    if idx_scale_logical is not None:
        iscale, _, _ = paged_from_logical([s.unsqueeze(-1) for s in idx_scale_logical],
                                          page_size, perm_seed)
        iscale = iscale.squeeze(-1).contiguous()
    kvscale = None
    if kv_scale_logical is not None:
        kvscale, _, _ = paged_from_logical([s.unsqueeze(-1) for s in kv_scale_logical],
                                           page_size, perm_seed)
        kvscale = kvscale.squeeze(-1).contiguous()
    pooled = None
    if pooled_logical is not None:
        # one summary row per block, stored at the block's physical page
        pooled = torch.zeros((num_pages, pooled_logical[0].shape[-1]), dtype=torch.bfloat16)
        for b, prow in enumerate(pooled_logical):
            for j in range(prow.shape[0]):
                pooled[pt[b, j]] = prow[j]
    H_kv = kv_logical[0].shape[1]
    k_row = kv_logical[0].shape[2]
    dv = dim_v if dim_v is not None else (v_logical[0].shape[2] if v_logical is not None
                                          else k_row)
    return Workload(
        name="custom", config_id=0, num_seqs=len(ctx_lens), ctx_lens=list(ctx_lens),
        page_size=page_size, pages_per_seq=pt.shape[1], num_pages=num_pages, page_table=pt,
        q_lens=list(q_lens), idx_heads=q_idx.shape[1], idx_dim=q_idx.shape[2],
        idx_dtype=idx_dtype, q_idx=q_idx, w=w, idx_keys=keys, idx_scale=iscale, pooled=pooled,
        topk=topk, block_topk=block_topk, heads_q=q.shape[1], heads_kv=H_kv,
        dim_qk=q.shape[2], dim_v=dv, kv_dtype=kv_dtype, q=q, k_cache=kc, v_cache=vc,
        kv_scale=kvscale, softmax_scale=float(softmax_scale))


def logical_rows(cache: torch.Tensor, page_table: torch.Tensor, b: int, n: int,
                 page_size: int) -> torch.Tensor:
    """Inverse of paged_from_logical for one sequence (test-side view, used for brute force)."""
    rows = []
    for j in range(math.ceil(n / page_size)):
        rows.append(cache[int(page_table[b, j])])
    if not rows:
        return cache[:0].reshape((0,) + tuple(cache.shape[2:]))
    return torch.cat(rows, 0)[:n]


# ---------------------------------------------------------------------------- comparators

def check_topk_row(got, ref, ref_scores_row, n_visible, k, rel=1e-3):
    """Acceptance of one GPU index row against the oracle's.

    got/ref: int arrays [k] (ascending positions then -1 padding, any order accepted for got).
    The GPU set must hold exactly k_eff = min(k, n_visible) distinct visible positions and then
    -1s; every position in the symmetric difference with the oracle's set must score within
    rel * |theta| of theta, the oracle's k_eff-th largest score. Returns an error string or ''.
    """
    got = np.asarray(got)
    ref = np.asarray(ref)
    k_eff = min(k, n_visible)
    g = got[got >= 0]
    if len(g) != k_eff:
        return f"expected {k_eff} valid indices, got {len(g)}"
    if np.any(got[got < 0] != -1):
        return "negative index other than -1"
    if np.sum(got == -1) != k - k_eff:
        return "padding is not -1"
    if len(np.unique(g)) != len(g):
        return "duplicate indices"
    if np.any(g >= n_visible):
        return "index outside the visible range"
    r = ref[ref >= 0]
    if k_eff == 0:
        return ""
    theta = float(np.min(ref_scores_row[r]))
    tol = rel * abs(theta)
    diff = np.setxor1d(g, r)
    bad = [int(t) for t in diff if abs(float(ref_scores_row[t]) - theta) > tol]
    if bad:
        return (f"{len(diff)} differing positions, {len(bad)} outside the near-tie band "
                f"(theta={theta:.6g}, e.g. pos {bad[0]} score {float(ref_scores_row[bad[0]]):.6g})")
    return ""


def check_topk_in(got, ref, ref_scores_row, candidates, k, rel=1e-3):
    """check_topk_row when only some positions are candidates (the tokens of the kept blocks of a
    hierarchical selection): candidates is a bool array over the sequence's positions; the GPU
    set must hold exactly k_eff = min(k, number of candidates) distinct candidates and then -1s,
    and the near-tie rule applies as in check_topk_row. Returns an error string or ''."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    cand = np.asarray(candidates, dtype=bool)
    k_eff = min(k, int(cand.sum()))
    g = got[got >= 0]
    if len(g) != k_eff:
        return f"expected {k_eff} valid indices, got {len(g)}"
    if np.any(got[got < 0] != -1):
        return "negative index other than -1"
    if np.sum(got == -1) != k - k_eff:
        return "padding is not -1"
    if len(np.unique(g)) != len(g):
        return "duplicate indices"
    if np.any(g >= len(cand)) or not np.all(cand[g]):
        return "index outside the candidates"
    r = ref[ref >= 0]
    if k_eff == 0:
        return ""
    theta = float(np.min(ref_scores_row[r]))
    tol = rel * abs(theta)
    diff = np.setxor1d(g, r)
    bad = [int(t) for t in diff if abs(float(ref_scores_row[t]) - theta) > tol]
    if bad:
        return (f"{len(diff)} differing positions, {len(bad)} outside the near-tie band "
                f"(theta={theta:.6g}, e.g. pos {bad[0]} score {float(ref_scores_row[bad[0]]):.6g})")
    return ""


# Attention outputs pass two gates. ABS: the acceptance tolerance against the fp32/fp64
# definition (2e-2 for bf16 caches, 5e-2 for E4M3 caches). REL: a regression gate relative to
# the largest reference output. Outputs here are small (at the 576-wide latent shapes the
# largest |o| is about 0.25), so a 3 % error in the softmax scale moves them by less than the
# absolute tolerance; the kernel's own error (bf16 rounding of the probabilities and of the
# output, fp32 accumulation) stays below a few parts per thousand of max |o|.
REL_GATE = 2e-2


def output_error(got, ref, abs_tol, rel=REL_GATE):
    """(max-abs error, message): message is '' when both gates pass."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    if err > abs_tol:
        return err, f"max abs error {err:.3e} above the acceptance tolerance {abs_tol}"
    if err > rel * scale:
        return err, (f"max abs error {err:.3e} above the regression gate {rel} * max|ref| "
                     f"= {rel * scale:.3e}")
    return err, ""
