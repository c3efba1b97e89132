"""Pins for the document-id helpers of the oracle.

``cu_seqlens_from_ids`` is checked on a worked example, against numpy's run
detection and on edge cases; ``document_masked_attention`` (one packed
sequence, sample-id mask over the whole [T, T] score matrix) is checked
against torch SDPA with the same boolean mask in float64, and against the
oracle's varlen attention on the runs, which is the identity the GPU path
relies on.
"""

import numpy as np
import pytest
import torch

import oracle


def test_worked_example_and_capacity_tail():
    ids = [7, 7, 7, 2, 5, 5]
    cu, n = oracle.cu_seqlens_from_ids(ids, 5)
    assert n == 3 and cu.tolist() == [0, 3, 4, 6, 6, 6]
    with pytest.raises(ValueError):
        oracle.cu_seqlens_from_ids(ids, 2)
    cu, n = oracle.cu_seqlens_from_ids([4], 1)
    assert n == 1 and cu.tolist() == [0, 1]
    # a repeated id after another document starts a new run
    cu, n = oracle.cu_seqlens_from_ids([1, 1, 2, 1], 4)
    assert n == 3 and cu.tolist() == [0, 2, 3, 4, 4]


@pytest.mark.parametrize("seed", range(4))
def test_matches_numpy_run_detection(seed):
    rng = np.random.default_rng(seed)
    ids = np.repeat(rng.integers(0, 5, size=40), rng.integers(1, 9, size=40))
    cu, n = oracle.cu_seqlens_from_ids(ids, 200)
    starts = np.flatnonzero(np.r_[True, ids[1:] != ids[:-1]])
    assert n == len(starts)
    assert np.array_equal(cu[:n], starts) and np.all(cu[n:] == len(ids))
    lengths = np.diff(cu[: n + 1])
    assert lengths.min() >= 1 and lengths.sum() == len(ids)


@pytest.mark.parametrize("causal", [False, True])
def test_document_mask_matches_sdpa_and_varlen(causal):
    rng = np.random.default_rng(11 + causal)
    ids = np.repeat([3, 1, 4, 9, 2], [5, 1, 7, 4, 9])  # each document one contiguous run
    t, h, d = len(ids), 2, 8
    q, k, v = (rng.standard_normal((t, h, d)) for _ in range(3))
    out, lse = oracle.document_masked_attention(q, k, v, ids, 0.3, causal)
    mask = torch.from_numpy(ids[:, None] == ids[None, :])
    if causal:
        mask = mask & torch.ones(t, t, dtype=torch.bool).tril()
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).transpose(0, 1), torch.from_numpy(k).transpose(0, 1),
        torch.from_numpy(v).transpose(0, 1), attn_mask=mask, scale=0.3).transpose(0, 1).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12
    cu, n = oracle.cu_seqlens_from_ids(ids, 8)
    vout, vlse = oracle.varlen_attention(q, k, v, cu, cu, 0.3, causal)
    assert np.max(np.abs(out - vout)) < 1e-12 and np.max(np.abs(lse - vlse)) < 1e-12


def test_repeated_id_in_separate_runs_is_not_one_document():
    """A packed buffer keeps a document's tokens together; if an id came back
    after another document, the dense mask would join the two runs while the
    run boundaries split them.  The helpers follow the runs."""
    rng = np.random.default_rng(13)
    ids = np.repeat([3, 1, 3], [4, 2, 5])
    t, h, d = len(ids), 1, 4
    q, k, v = (rng.standard_normal((t, h, d)) for _ in range(3))
    cu, n = oracle.cu_seqlens_from_ids(ids, 4)
    assert n == 3
    dense, _ = oracle.document_masked_attention(q, k, v, ids, 0.5)
    runs, _ = oracle.varlen_attention(q, k, v, cu, cu, 0.5)
    assert np.max(np.abs(dense[4:6] - runs[4:6])) < 1e-12   # the middle document is alone either way
    assert np.max(np.abs(dense[:4] - runs[:4])) > 1e-3       # the two runs of id 3 differ
