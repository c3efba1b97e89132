"""Pins for the oracle's attention gradients (``oracle.varlen_attention_bwd``).

The pages train through packed attention but print no backward algorithm, so
the oracle writes out the derivative of its own forward.  Nothing here
re-derives that formula: each test checks the gradients against central
finite differences of the (separately pinned) forward oracle, against torch
autograd through the padded float64 SDPA reference of
"gigl.nn.packed_attention", against closed forms, or against invariants that
follow from the shape of the softmax.  The planted mistakes at the end check
that plausible errors in the formula are caught.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import varlen_oracle


def _cu(lengths):
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return np.asarray(out, dtype=np.int32)


def _rand(rng, t, h, d):
    return rng.standard_normal((t, h, d))


def _loss(q, k, v, dout, cu_q, cu_k, scale, causal):
    out, _ = oracle.varlen_attention(q, k, v, cu_q, cu_k, scale, causal)
    return float(np.sum(out * dout))


def _finite_difference(q, k, v, dout, cu_q, cu_k, scale, causal, eps=1e-5):
    """Central differences of sum(dout * out) for every entry of q, k and v."""
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        for idx in np.ndindex(*g.shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            g[idx] = (_loss(*plus, dout, cu_q, cu_k, scale, causal)
                      - _loss(*minus, dout, cu_q, cu_k, scale, causal)) / (2 * eps)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lq,lk", [([1, 4, 6], [1, 4, 6]), ([2, 5, 3], [4, 5, 1])])
def test_bwd_matches_finite_differences(lq, lk, causal):
    rng = np.random.default_rng(31 + 2 * causal + len(set(lq) ^ set(lk)))
    h, d = 2, 3
    q = _rand(rng, sum(lq), h, d)
    k = _rand(rng, sum(lk), h, d)
    v = _rand(rng, sum(lk), h, d)
    dout = _rand(rng, sum(lq), h, d)
    cq, ck = _cu(lq), _cu(lk)
    scale = 0.6
    dq, dk, dv = oracle.varlen_attention_bwd(q, k, v, dout, cq, ck, scale, causal)
    fq, fk, fv = _finite_difference(q, k, v, dout, cq, ck, scale, causal)
    assert np.max(np.abs(dq - fq)) < 1e-7
    assert np.max(np.abs(dk - fk)) < 1e-7
    assert np.max(np.abs(dv - fv)) < 1e-7
    assert np.max(np.abs(dq)) > 1e-2 and np.max(np.abs(dk)) > 1e-2  # not trivially zero


def _autograd_padded(q, k, v, dout, lengths, scale, causal):
    """Gradients from torch autograd through SDPA on a padded float64 grid."""
    b = len(lengths)
    lmax = int(max(lengths))
    h, d = q.shape[1], q.shape[2]
    cu = _cu(lengths)

    def pad(x):
        p = torch.zeros(b, h, lmax, d, dtype=torch.float64)
        for i in range(b):
            p[i, :, :lengths[i]] = torch.from_numpy(x[cu[i]:cu[i + 1]]).transpose(0, 1)
        return p

    qp, kp, vp, dop = pad(q), pad(k), pad(v), pad(dout)
    for t in (qp, kp, vp):
        t.requires_grad_(True)
    key_valid = torch.arange(lmax)[None, :] < torch.as_tensor(lengths)[:, None]
    mask = key_valid[:, None, None, :].expand(b, 1, lmax, lmax)
    if causal:
        mask = mask & torch.ones(lmax, lmax, dtype=torch.bool).tril()
    mask = mask | (~key_valid[:, None, :, None] & torch.eye(lmax, dtype=torch.bool))
    out = torch.nn.functional.scaled_dot_product_attention(qp, kp, vp, attn_mask=mask, scale=scale)
    out.backward(dop)  # padded rows of dout are zero, so padding feeds no gradient

    def unpad(g):
        r = np.zeros_like(q)
        for i in range(b):
            r[cu[i]:cu[i + 1]] = g[i, :, :lengths[i]].transpose(0, 1).numpy()
        return r

    return unpad(qp.grad), unpad(kp.grad), unpad(vp.grad)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", range(2))
def test_bwd_matches_autograd_of_padded_sdpa(seed, causal):
    rng = np.random.default_rng(40 + seed)
    lengths = np.asarray([1, 7, 64, 3, 33, 1, 20])
    rng.shuffle(lengths)
    h, d = 2, 16
    t = int(lengths.sum())
    q, k, v, dout = (_rand(rng, t, h, d) for _ in range(4))
    scale = float(np.float32(0.25))
    cu = _cu(lengths)
    dq, dk, dv = oracle.varlen_attention_bwd(q, k, v, dout, cu, cu, scale, causal)
    rq, rk, rv = _autograd_padded(q, k, v, dout, lengths, scale, causal)
    assert np.max(np.abs(dq - rq)) < 1e-11
    assert np.max(np.abs(dk - rk)) < 1e-11
    assert np.max(np.abs(dv - rv)) < 1e-11


def test_bwd_length_one_sequences():
    """A one-token sequence: out = v whatever q and k are, so dv = dout and
    dq = dk = 0."""
    rng = np.random.default_rng(50)
    h, d = 3, 8
    q, k, v, dout = (_rand(rng, 4, h, d) for _ in range(4))
    cu = _cu([1, 1, 1, 1])
    for causal in (False, True):
        dq, dk, dv = oracle.varlen_attention_bwd(q, k, v, dout, cu, cu, 0.5, causal)
        assert np.array_equal(dq, np.zeros_like(dq)) and np.array_equal(dk, np.zeros_like(dk))
        assert np.max(np.abs(dv - dout)) < 1e-15


def test_bwd_zero_queries():
    """q = 0 gives uniform weights 1/L: dk = 0 (dk is a sum of q rows) and
    every dv row is the mean of the output gradients."""
    rng = np.random.default_rng(51)
    lengths = [5, 9]
    h, d = 2, 6
    t = sum(lengths)
    q = np.zeros((t, h, d))
    k, v, dout = (_rand(rng, t, h, d) for _ in range(3))
    cu = _cu(lengths)
    dq, dk, dv = oracle.varlen_attention_bwd(q, k, v, dout, cu, cu, 0.4, False)
    assert np.max(np.abs(dk)) < 1e-15
    for i in range(2):
        mean = dout[cu[i]:cu[i + 1]].mean(axis=0)
        assert np.max(np.abs(dv[cu[i]:cu[i + 1]] - mean[None])) < 1e-14
    assert np.max(np.abs(dq)) > 1e-2


def test_bwd_constant_values():
    """Equal value rows make out independent of q and k: dq = dk = 0."""
    rng = np.random.default_rng(52)
    lengths = [6, 3]
    h, d = 2, 5
    t = sum(lengths)
    q, k, dout = (_rand(rng, t, h, d) for _ in range(3))
    v = np.broadcast_to(rng.standard_normal((1, h, d)), (t, h, d)).copy()
    cu = _cu(lengths)
    for causal in (False, True):
        dq, dk, dv = oracle.varlen_attention_bwd(q, k, v, dout, cu, cu, 0.7, causal)
        assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13


def test_bwd_causal_first_row_has_no_query_gradient():
    """Causal query 0 sees key 0 only: its softmax is the constant 1."""
    rng = np.random.default_rng(53)
    lengths = [4, 7, 2]
    h, d = 2, 4
    t = sum(lengths)
    q, k, v, dout = (_rand(rng, t, h, d) for _ in range(4))
    cu = _cu(lengths)
    dq, _, _ = oracle.varlen_attention_bwd(q, k, v, dout, cu, cu, 0.5, True)
    for i in range(3):
        assert np.max(np.abs(dq[cu[i]])) < 1e-15
        assert np.max(np.abs(dq[cu[i] + 1])) > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_invariants(causal):
    """Per (sequence, head):
    * shifting every key by one vector adds a per-row constant to the scores,
      so sum_j dk_j = 0;
    * every query that sees a key spreads weights summing to one, so
      sum_j dv_j = sum_p dout_p;
    * scaling all queries by t equals scaling all keys by t, so
      sum_p dq_p . q_p = sum_j dk_j . k_j."""
    rng = np.random.default_rng(54 + causal)
    lengths = [1, 12, 30, 5]
    h, d = 3, 8
    t = sum(lengths)
    q, k, v, dout = (_rand(rng, t, h, d) for _ in range(4))
    cu = _cu(lengths)
    dq, dk, dv = oracle.varlen_attention_bwd(q, k, v, dout, cu, cu, 0.35, causal)
    for i in range(len(lengths)):
        s = slice(cu[i], cu[i + 1])
        for hh in range(h):
            assert np.max(np.abs(dk[s, hh].sum(axis=0))) < 1e-12
            assert np.max(np.abs(dv[s, hh].sum(axis=0) - dout[s, hh].sum(axis=0))) < 1e-12
            lhs = np.sum(dq[s, hh] * q[s, hh])
            rhs = np.sum(dk[s, hh] * k[s, hh])
            assert abs(lhs - rhs) < 1e-12


def test_bwd_keyless_queries_and_unowned_rows():
    """Causal with Lq > Lk leaves the first Lq - Lk queries keyless (zero dq);
    zero-length sequences and rows past cu[B] get nothing."""
    rng = np.random.default_rng(56)
    lq, lk = [6, 0, 3], [2, 0, 3]
    h, d = 2, 4
    q, dout = _rand(rng, sum(lq) + 2, h, d), _rand(rng, sum(lq) + 2, h, d)
    k, v = _rand(rng, sum(lk) + 3, h, d), _rand(rng, sum(lk) + 3, h, d)
    cq, ck = _cu(lq), _cu(lk)
    dq, dk, dv = oracle.varlen_attention_bwd(q, k, v, dout, cq, ck, 0.5, True)
    assert np.array_equal(dq[:4], np.zeros_like(dq[:4]))
    assert np.max(np.abs(dq[5])) > 1e-3
    assert np.array_equal(dq[9:], np.zeros_like(dq[9:]))
    assert np.array_equal(dk[5:], np.zeros_like(dk[5:])) and np.array_equal(dv[5:], np.zeros_like(dv[5:]))


def test_bwd_sequence_independence():
    rng = np.random.default_rng(57)
    lengths = [8, 5, 11]
    h, d = 2, 4
    t = sum(lengths)
    q, k, v, dout = (_rand(rng, t, h, d) for _ in range(4))
    cu = _cu(lengths)
    a = oracle.varlen_attention_bwd(q, k, v, dout, cu, cu, 0.5, True)
    k2, v2 = k.copy(), v.copy()
    k2[cu[1]:cu[2]] += 3.0
    v2[cu[1]:cu[2]] *= -2.0
    b = oracle.varlen_attention_bwd(q, k2, v2, dout, cu, cu, 0.5, True)
    for x, y in zip(a, b):
        for i in (0, 2):
            assert np.array_equal(x[cu[i]:cu[i + 1]], y[cu[i]:cu[i + 1]])


def test_bwd_sampled_rows_match_full():
    rng = np.random.default_rng(58)
    lengths = [17, 3, 40]
    h, d = 2, 8
    t = sum(lengths)
    q, k, v, dout = (_rand(rng, t, h, d) for _ in range(4))
    cu = _cu(lengths)
    for causal in (False, True):
        dq, dk, dv = oracle.varlen_attention_bwd(q, k, v, dout, cu, cu, 0.3, causal)
        qs = [(0, 0), (16, 1), (18, 0), (59, 1), (30, 1)]
        ks = [(5, 1), (17, 0), (19, 1), (20, 1), (59, 0)]
        a, b, c = oracle.varlen_attention_bwd_rows(q, k, v, dout, cu, cu, 0.3, causal, qs, ks)
        assert np.max(np.abs(a - np.asarray([dq[r, hh] for r, hh in qs]))) < 1e-13
        assert np.max(np.abs(b - np.asarray([dk[r, hh] for r, hh in ks]))) < 1e-13
        assert np.max(np.abs(c - np.asarray([dv[r, hh] for r, hh in ks]))) < 1e-13


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by a pin above
# --------------------------------------------------------------------------

def _plant(monkeypatch, body):
    """Replace _attend_one_bwd by a variant built from the same first steps."""
    def wrong(qi, ki, vi, doi, scale, causal, positions, lq):
        lk = ki.shape[0]
        vis = varlen_oracle._visibility(positions, lq, lk, causal)
        s = scale * (qi @ ki.T)
        live = vis.any(axis=1)
        m = np.where(live, np.where(vis, s, -np.inf).max(axis=1), 0.0)
        w = np.where(vis, np.exp(s - m[:, None]), 0.0)
        p = np.zeros_like(w)
        p[live] = w[live] / w[live].sum(axis=1, keepdims=True)
        return body(qi, ki, vi, doi, scale, p)
    monkeypatch.setattr(varlen_oracle, "_attend_one_bwd", wrong)


def test_planted_missing_row_term_is_caught(monkeypatch):
    def body(qi, ki, vi, doi, scale, p):
        ds = p * (doi @ vi.T)  # the rowsum(P * dP) term dropped
        return scale * ds @ ki, scale * ds.T @ qi, p.T @ doi
    _plant(monkeypatch, body)
    with pytest.raises(AssertionError):
        test_bwd_invariants(False)


def test_planted_unscaled_key_gradient_is_caught(monkeypatch):
    def body(qi, ki, vi, doi, scale, p):
        dp = doi @ vi.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        return scale * ds @ ki, ds.T @ qi, p.T @ doi
    _plant(monkeypatch, body)
    with pytest.raises(AssertionError):
        test_bwd_matches_finite_differences([1, 4, 6], [1, 4, 6], False)


def test_planted_values_for_keys_is_caught(monkeypatch):
    def body(qi, ki, vi, doi, scale, p):
        dp = doi @ vi.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        return scale * ds @ vi, scale * ds.T @ qi, p.T @ doi  # dq built from V
    _plant(monkeypatch, body)
    with pytest.raises(AssertionError):
        test_bwd_matches_autograd_of_padded_sdpa(0, True)
