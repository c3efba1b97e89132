"""Pins for the oracle's ragged matrix multiplication (``oracle.ragged_matmul``).

"PyCoRa", "Ragged Matrix Multiplication": every sequence of the packed batch
is multiplied by its own weight matrix.  The pins check the oracle against
torch's batched matmul over the padded envelope (float64), a pure-Python
brute force, closed forms (identity and zero weights, one-hot inputs) and
invariants (sequence independence, linearity, the shared-weight case equals
one plain product of all rows); planted mistakes are caught.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import varlen_oracle


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _case(seed, lengths, k, n):
    rng = np.random.default_rng(seed)
    t = int(sum(lengths))
    x = rng.standard_normal((t, k))
    w = rng.standard_normal((len(lengths), n, k))
    b = rng.standard_normal((len(lengths), n))
    return x, w, b, _cu(lengths)


@pytest.mark.parametrize("seed", range(3))
def test_matches_padded_bmm(seed):
    lengths = [5, 1, 17, 0, 9]
    x, w, b, cu = _case(seed, lengths, 12, 7)
    y = oracle.ragged_matmul(x, w, cu, b)
    lmax = max(lengths)
    xp = torch.zeros(len(lengths), lmax, 12, dtype=torch.float64)
    for i, n in enumerate(lengths):
        xp[i, :n] = torch.from_numpy(x[cu[i]:cu[i + 1]])
    yp = torch.bmm(xp, torch.from_numpy(w).transpose(1, 2).contiguous()) + torch.from_numpy(b)[:, None, :]
    for i, n in enumerate(lengths):
        assert np.max(np.abs(y[cu[i]:cu[i + 1]] - yp[i, :n].numpy()), initial=0.0) < 1e-12


def test_pure_python_brute_force():
    lengths = [2, 3]
    x, w, b, cu = _case(7, lengths, 4, 3)
    y = oracle.ragged_matmul(x, w, cu, b)
    for i in range(2):
        for r in range(cu[i], cu[i + 1]):
            for j in range(3):
                ref = b[i, j] + sum(x[r, kk] * w[i, j, kk] for kk in range(4))
                assert abs(y[r, j] - ref) < 1e-12


def test_identity_zero_and_one_hot():
    lengths = [4, 6]
    x, _, _, cu = _case(8, lengths, 5, 5)
    eye = np.stack([np.eye(5), 2 * np.eye(5)])
    y = oracle.ragged_matmul(x, eye, cu)
    assert np.array_equal(y[:4], x[:4]) and np.array_equal(y[4:], 2 * x[4:])
    bias = np.array([[1.0, 2, 3, 4, 5], [-1, -2, -3, -4, -5]])
    y0 = oracle.ragged_matmul(x, np.zeros((2, 5, 5)), cu, bias)
    assert np.array_equal(y0[:4], np.broadcast_to(bias[0], (4, 5)))
    # a one-hot row picks one input column of each weight row
    xo = np.zeros((10, 5))
    xo[:, 2] = 1.0
    w = np.arange(2 * 5 * 5, dtype=np.float64).reshape(2, 5, 5)
    yo = oracle.ragged_matmul(xo, w, cu)
    assert np.array_equal(yo[0], w[0, :, 2]) and np.array_equal(yo[9], w[1, :, 2])


def test_shared_weight_is_one_plain_product():
    lengths = [3, 0, 8, 1]
    x, w, b, cu = _case(9, lengths, 6, 4)
    y = oracle.ragged_matmul(x, w[0], cu, b[0], shared_weight=True, shared_bias=True)
    assert np.max(np.abs(y - (x @ w[0].T + b[0]))) < 1e-12


def test_sequence_independence_linearity_and_unowned_rows():
    lengths = [4, 7, 2]
    x, w, b, cu = _case(10, lengths, 6, 5)
    xx = np.concatenate([x, np.full((3, 6), np.nan)])  # capacity rows past cu[B]
    y = oracle.ragged_matmul(xx, w, cu, b)
    assert np.array_equal(y[cu[-1]:], np.zeros((3, 5)))
    w2 = w.copy()
    w2[1] *= -3.0
    y2 = oracle.ragged_matmul(xx, w2, cu, b)
    assert np.array_equal(y[:4], y2[:4]) and np.array_equal(y[11:13], y2[11:13])
    ya = oracle.ragged_matmul(x, w, cu)
    yb = oracle.ragged_matmul(2.5 * x, w, cu)
    assert np.max(np.abs(yb - 2.5 * ya)) < 1e-12


def test_planted_weight_transpose_is_caught(monkeypatch):
    real = varlen_oracle.ragged_matmul

    def wrong(x, weight, cu_seqlens, bias=None, shared_weight=False, shared_bias=False):
        w = np.asarray(weight)
        wt = np.swapaxes(w, -1, -2)  # uses weight instead of weight^T
        return real(x, wt, cu_seqlens, bias, shared_weight, shared_bias)
    monkeypatch.setattr(oracle, "ragged_matmul", wrong)
    with pytest.raises(Exception):
        test_identity_zero_and_one_hot()
        test_pure_python_brute_force()


def test_planted_wrong_sequence_weight_is_caught(monkeypatch):
    real = varlen_oracle.ragged_matmul

    def shifted(x, weight, cu_seqlens, bias=None, shared_weight=False, shared_bias=False):
        return real(x, np.roll(np.asarray(weight), 1, axis=0), cu_seqlens, bias, shared_weight, shared_bias)
    monkeypatch.setattr(oracle, "ragged_matmul", shifted)
    with pytest.raises(AssertionError):
        test_matches_padded_bmm(0)
