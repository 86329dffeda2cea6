"""The acceptance comparators themselves, on the CPU: they must reject the mistakes they exist
to catch. The gates are applied by every GPU parity test and by smoke()."""
import dataclasses

import numpy as np
import torch

import oracle
from indexer_top_sparse_amd import inputs
from tests._util import check_topk_in, check_topk_row, output_error


def test_output_gate_rejects_a_three_percent_softmax_scale_error():
    """At the headline shape (128 heads over 576-wide latent rows, K = 2048 of 32768 tokens)
    the outputs are small, so the absolute tolerance alone (2e-2) passes an attention whose
    logits are scaled 3 % too much; the relative gate does not. The oracle's own output,
    rounded to bf16 as the library returns it, passes both."""
    wl = inputs.make("decode32k", num_seqs=2)
    ref = oracle.decode_step(wl)
    idx = ref["idx"]
    want = ref["out"]
    as_bf16 = torch.from_numpy(want).to(torch.bfloat16).double().numpy()
    err, msg = output_error(as_bf16, want, 2e-2)
    assert msg == "", msg
    bad = oracle.sparse_attn(dataclasses.replace(wl, softmax_scale=wl.softmax_scale * 1.03), idx)
    err, msg = output_error(bad, want, 2e-2)
    assert err <= 2e-2, "the absolute tolerance alone would have accepted this output"
    assert "regression gate" in msg, msg
    assert err > 0.04 * np.abs(want).max()


def test_output_gate_on_empty_outputs():
    z = np.zeros((2, 3, 4))
    assert output_error(z, z, 2e-2)[1] == ""
    assert output_error(z + 1e-6, z, 2e-2)[1] != ""


def test_index_gate():
    s = np.array([5.0, 4.0, 3.0, 3.0005, 1.0, 0.0])
    ref = np.array([0, 1, 3])
    # the exact set, in any order
    assert check_topk_row(np.array([3, 0, 1]), ref, s, 6, 3) == ""
    # a near tie (3.0 against theta = 3.0005, within 1e-3 * theta) is accepted
    assert check_topk_row(np.array([0, 1, 2]), ref, s, 6, 3) == ""
    # a clear miss is not, nor a duplicate, nor a position past the visible range
    assert check_topk_row(np.array([0, 1, 4]), ref, s, 6, 3) != ""
    assert check_topk_row(np.array([0, 1, 1]), ref, s, 6, 3) != ""
    assert check_topk_row(np.array([0, 1, 3]), ref, s, 3, 3) != ""
    # K above the visible count: the visible positions, then exactly -1
    ref4 = np.array([0, 1, 2, -1])
    assert check_topk_row(np.array([0, 1, 2, -1]), ref4, s, 3, 4) == ""
    assert check_topk_row(np.array([0, 1, 2, -2]), ref4, s, 3, 4) != ""
    assert check_topk_row(np.array([0, 1, -1, -1]), ref4, s, 3, 4) != ""


def test_index_gate_over_candidates():
    """Hierarchical selection: only the tokens of the kept blocks are candidates, and there may
    be fewer of them than K."""
    s = np.array([9.0, 8.0, 5.0, 4.0, 3.0, 3.0005, 1.0, 0.0])
    cand = np.array([False, False, True, True, True, True, False, True])  # 0, 1, 6 not kept
    ref = np.array([2, 3, 5])
    assert check_topk_in(np.array([2, 3, 5]), ref, s, cand, 3) == ""
    assert check_topk_in(np.array([2, 3, 4]), ref, s, cand, 3) == ""   # near tie at theta
    # a larger score outside the candidates, or a clear miss, is rejected
    assert check_topk_in(np.array([0, 2, 3]), ref, s, cand, 3) != ""
    assert check_topk_in(np.array([2, 3, 7]), ref, s, cand, 3) != ""
    # K above the candidate count (5): the candidates, then exactly -1
    ref7 = np.array([2, 3, 4, 5, 7, -1, -1])
    assert check_topk_in(np.array([2, 3, 4, 5, 7, -1, -1]), ref7, s, cand, 7) == ""
    assert check_topk_in(np.array([2, 3, 4, 5, 6, -1, -1]), ref7, s, cand, 7) != ""
    assert check_topk_in(np.array([2, 3, 4, 5, -1, -1, -1]), ref7, s, cand, 7) != ""
    assert check_topk_in(np.array([2, 3, 4, 5, 7, -1, -2]), ref7, s, cand, 7) != ""
