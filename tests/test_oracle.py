"""Pins for the CPU oracle: worked examples, closed forms, invariants, brute force.

Nothing here compares the oracle with itself: each test checks it against a
value the pages print, a closed form, a library routine (torch SDPA on the CPU
in float64, the padded reference of "gigl.nn.packed_attention") or a pure
Python brute force.  The mutation tests at the end plant plausible mistakes in
the oracle and check that a pin catches each one.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import varlen_oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _cu(lengths):
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return np.asarray(out, dtype=np.int32)


# --------------------------------------------------------------------------
# pack_sequences
# --------------------------------------------------------------------------

def test_pack_worked_example():
    g = _golden("pack_sequences_example.json")
    flat, cu = oracle.pack_sequences(g["lengths"], g["max_seq_len"])
    assert flat.dtype == np.int64 and cu.dtype == np.int32
    assert flat.tolist() == g["flat_index"]
    assert cu.tolist() == [0, 3, 4, 6]


@pytest.mark.parametrize("seed", range(5))
def test_pack_gathers_real_tokens(seed):
    """grid.flatten()[flat_index] yields, in order, exactly the real tokens."""
    rng = np.random.default_rng(seed)
    b = int(rng.integers(1, 20))
    max_len = int(rng.integers(1, 40))
    lengths = rng.integers(1, max_len + 1, size=b)
    flat, cu = oracle.pack_sequences(lengths, max_len)
    grid = np.full((b, max_len, 2), -1, dtype=np.int64)
    for i in range(b):
        for j in range(lengths[i]):
            grid[i, j] = (i, j)
    packed = grid.reshape(b * max_len, 2)[flat]
    expect = [(i, j) for i in range(b) for j in range(lengths[i])]
    assert [tuple(r) for r in packed.tolist()] == expect
    assert cu[0] == 0 and cu[-1] == lengths.sum()
    assert np.all(np.diff(cu) == lengths)
    assert np.all(np.diff(flat) > 0)
    for i in range(b):
        assert flat[cu[i]] == i * max_len


def test_pack_rejects_bad_lengths():
    with pytest.raises(ValueError):
        oracle.pack_sequences([3, 0, 2], 3)
    with pytest.raises(ValueError):
        oracle.pack_sequences([3, 4], 3)
    with pytest.raises(ValueError):
        oracle.pack_sequences([], 3)


def test_pack_overflow():
    """cu_seqlens is int32, so the token count must fit in int32."""
    n = 2**30 + 1
    with pytest.raises(OverflowError):
        oracle.pack_sequences([n, n], n)
    # one token below the limit is still accepted by the length checks
    ok_total = oracle.INT32_MAX
    assert ok_total == 2**31 - 1


# --------------------------------------------------------------------------
# ragged grid
# --------------------------------------------------------------------------

def test_grid_worked_example():
    g = _golden("chunk_offsets_example.json")
    bo, gm, order = oracle.build_ragged_grid(g["cu_seqlens"], g["chunk"])
    assert bo.tolist() == g["chunk_offsets"]
    assert bo.tolist() != g["wrong_ceil_div_of_cu_seqlens"]
    assert gm.tolist() == [0, 0, 1]
    for d in g["decode"]:
        seq, local, start = oracle.decode_tile(bo, g["cu_seqlens"], d["flat_chunk"], g["chunk"])
        assert (seq, local, start) == (d["sequence"], d["local_chunk"], d["token_start"])
        assert gm[d["flat_chunk"]] == d["sequence"]
    # longest-first order: sequence 0 (65 tokens) first, its tiles last to first
    assert order.tolist() == [1, 0, 2]


def _random_lengths(rng, with_zeros):
    b = int(rng.integers(1, 30))
    lengths = rng.integers(0 if with_zeros else 1, 300, size=b)
    if with_zeros and b > 2:
        lengths[-2:] = 0  # capacity tail [.., L, L, L]
    return lengths


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("block_m", [1, 16, 64, 128])
def test_grid_invariants(seed, block_m):
    rng = np.random.default_rng(100 + seed)
    lengths = _random_lengths(rng, with_zeros=seed % 2 == 1)
    cu = _cu(lengths)
    bo, gm, order = oracle.build_ragged_grid(cu, block_m)
    g = int(bo[-1])
    # per-sequence ceiling, checked against math.ceil on each length
    assert [int(x) for x in np.diff(bo)] == [math.ceil(int(n) / block_m) for n in lengths]
    assert bo[0] == 0 and len(gm) == g and len(order) == g
    # ownership agrees with the page's decode; zero-length sequences own nothing
    for f in range(g):
        seq, local, start = oracle.decode_tile(bo, cu, f, block_m)
        assert gm[f] == seq and lengths[seq] > 0
        assert cu[seq] <= start < cu[seq + 1]
    # tile_order is a permutation, longest sequence first, tiles descending
    assert sorted(order.tolist()) == list(range(g))
    owners = gm[order]
    lens = lengths[owners]
    assert np.all(np.diff(lens) <= 0)
    for a, b in zip(order[:-1], order[1:]):
        if gm[a] == gm[b]:
            assert b == a - 1
    # capacity bound of "Scheduling without max_seqlen"
    t = int(cu[-1])
    assert g <= oracle.grid_capacity(t, len(lengths), block_m)


def test_grid_capacity_is_tight_and_bounds_all_splits():
    """Brute force over every split of <= T tokens over N slots (tiny sizes)."""
    for t_cap, n_cap, c in [(5, 3, 2), (7, 4, 3), (6, 6, 4), (4, 2, 1)]:
        best = 0
        for lengths in itertools.product(range(t_cap + 1), repeat=n_cap):
            if sum(lengths) > t_cap:
                continue
            bo, _, _ = oracle.build_ragged_grid(_cu(lengths), c)
            best = max(best, int(bo[-1]))
        assert best == oracle.grid_capacity(t_cap, n_cap, c)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def _rand(rng, t, h, d):
    return rng.standard_normal((t, h, d))


def _sdpa_padded(q, k, v, lengths, scale, causal):
    """torch SDPA on a padded [B, H, L, D] grid in float64, real rows kept.

    The padded reference of "gigl.nn.packed_attention" (CPU path): a boolean
    key mask (true = valid) for non-causal, a lower-triangular mask for causal.
    """
    b = len(lengths)
    lmax = int(max(lengths))
    h, d = q.shape[1], q.shape[2]
    cu = _cu(lengths)
    qp = torch.zeros(b, h, lmax, d, dtype=torch.float64)
    kp = torch.zeros_like(qp)
    vp = torch.zeros_like(qp)
    for i in range(b):
        n = int(lengths[i])
        qp[i, :, :n] = torch.from_numpy(q[cu[i]:cu[i + 1]]).transpose(0, 1)
        kp[i, :, :n] = torch.from_numpy(k[cu[i]:cu[i + 1]]).transpose(0, 1)
        vp[i, :, :n] = torch.from_numpy(v[cu[i]:cu[i + 1]]).transpose(0, 1)
    key_valid = torch.arange(lmax)[None, :] < torch.as_tensor(lengths)[:, None]  # [B, L]
    mask = key_valid[:, None, None, :].expand(b, 1, lmax, lmax)
    if causal:
        tri = torch.ones(lmax, lmax, dtype=torch.bool).tril()
        mask = mask & tri
    # rows that would see nothing (padding rows) get their own key to stay finite
    eye = torch.eye(lmax, dtype=torch.bool)
    mask = mask | (~key_valid[:, None, :, None] & eye)
    out = torch.nn.functional.scaled_dot_product_attention(qp, kp, vp, attn_mask=mask, scale=scale)
    res = np.zeros_like(q)
    for i in range(b):
        n = int(lengths[i])
        res[cu[i]:cu[i + 1]] = out[i, :, :n].transpose(0, 1).numpy()
    return res


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", range(3))
def test_attention_matches_padded_sdpa(seed, causal):
    rng = np.random.default_rng(seed)
    lengths = np.asarray([1, 7, 64, 3, 33, 1, 20], dtype=np.int64)
    rng.shuffle(lengths)
    h, d = 2, 16
    t = int(lengths.sum())
    q, k, v = _rand(rng, t, h, d), _rand(rng, t, h, d), _rand(rng, t, h, d)
    scale = float(np.float32(0.25))
    cu = _cu(lengths)
    out, lse = oracle.varlen_attention(q, k, v, cu, cu, scale, causal)
    ref = _sdpa_padded(q, k, v, lengths, scale, causal)
    assert np.max(np.abs(out - ref)) < 1e-12
    assert np.all(np.isfinite(lse))


def test_attention_pure_python_brute_force():
    rng = np.random.default_rng(7)
    lengths = [3, 1, 5]
    h, d = 2, 4
    t = sum(lengths)
    q, k, v = _rand(rng, t, h, d), _rand(rng, t, h, d), _rand(rng, t, h, d)
    scale = 0.7
    cu = _cu(lengths)
    for causal in (False, True):
        out, lse = oracle.varlen_attention(q, k, v, cu, cu, scale, causal)
        for i, n in enumerate(lengths):
            base = int(cu[i])
            for hh in range(h):
                for p in range(n):
                    keys = [j for j in range(n) if (not causal or j <= p)]
                    s = [scale * sum(q[base + p, hh, x] * k[base + j, hh, x] for x in range(d)) for j in keys]
                    z = sum(math.exp(x) for x in s)
                    for x in range(d):
                        o = sum(math.exp(s[a]) * v[base + j, hh, x] for a, j in enumerate(keys)) / z
                        assert abs(o - out[base + p, hh, x]) < 1e-12
                    assert abs(math.log(z) - lse[hh, base + p]) < 1e-12


def test_length_one_returns_own_value_row():
    rng = np.random.default_rng(3)
    lengths = [4, 1, 6]
    h, d = 3, 16
    t = sum(lengths)
    q, k, v = _rand(rng, t, h, d), _rand(rng, t, h, d), _rand(rng, t, h, d)
    cu = _cu(lengths)
    scale = 0.25
    for causal in (False, True):
        out, lse = oracle.varlen_attention(q, k, v, cu, cu, scale, causal)
        row = int(cu[1])
        assert np.allclose(out[row], v[row], rtol=0, atol=1e-15)
        for hh in range(h):
            assert abs(lse[hh, row] - scale * float(q[row, hh] @ k[row, hh])) < 1e-12


def test_zero_query_gives_mean_and_log_length():
    rng = np.random.default_rng(4)
    lengths = [5, 9]
    h, d = 2, 8
    t = sum(lengths)
    q = np.zeros((t, h, d))
    k, v = _rand(rng, t, h, d), _rand(rng, t, h, d)
    cu = _cu(lengths)
    out, lse = oracle.varlen_attention(q, k, v, cu, cu, 0.3, False)
    for i, n in enumerate(lengths):
        sl = slice(cu[i], cu[i + 1])
        assert np.allclose(out[sl], v[sl].mean(axis=0)[None], atol=1e-14)
        assert np.allclose(lse[:, sl], math.log(n), atol=1e-14)


def test_identical_keys_give_uniform_weights():
    rng = np.random.default_rng(5)
    lengths = [6]
    h, d = 1, 8
    q = _rand(rng, 6, h, d)
    k = np.repeat(_rand(rng, 1, h, d), 6, axis=0)
    v = _rand(rng, 6, h, d)
    out, lse = oracle.varlen_attention(q, k, v, _cu(lengths), _cu(lengths), 0.5, False)
    assert np.allclose(out, v.mean(axis=0)[None], atol=1e-14)
    expect = 0.5 * np.einsum("thd,hd->ht", q, k[0]) + math.log(6)
    assert np.allclose(lse, expect, atol=1e-13)


def test_constant_values_pass_through():
    rng = np.random.default_rng(6)
    lengths = [3, 8, 1]
    h, d = 2, 16
    t = sum(lengths)
    q, k = _rand(rng, t, h, d), _rand(rng, t, h, d)
    c = rng.standard_normal((h, d))
    v = np.broadcast_to(c, (t, h, d)).copy()
    for causal in (False, True):
        out, _ = oracle.varlen_attention(q, k, v, _cu(lengths), _cu(lengths), 0.25, causal)
        assert np.allclose(out, v, atol=1e-14)


def test_causal_first_and_last_rows():
    rng = np.random.default_rng(8)
    lengths = [10, 4]
    h, d = 2, 16
    t = sum(lengths)
    q, k, v = _rand(rng, t, h, d), _rand(rng, t, h, d), _rand(rng, t, h, d)
    cu = _cu(lengths)
    oc, lc = oracle.varlen_attention(q, k, v, cu, cu, 0.25, True)
    of, lf = oracle.varlen_attention(q, k, v, cu, cu, 0.25, False)
    for i in range(2):
        first, last = int(cu[i]), int(cu[i + 1]) - 1
        assert np.allclose(oc[first], v[first], atol=1e-15)
        for hh in range(h):
            assert abs(lc[hh, first] - 0.25 * float(q[first, hh] @ k[first, hh])) < 1e-12
        assert np.allclose(oc[last], of[last], atol=1e-14)
        assert np.allclose(lc[:, last], lf[:, last], atol=1e-13)
        # causal rows differ from full rows before the last one
        assert not np.allclose(oc[first:last], of[first:last])


def test_first_token_equals_full_rows():
    g = _golden("pack_sequences_example.json")
    rng = np.random.default_rng(9)
    h, d = g["heads"], g["head_dim"]
    flat, cu = oracle.pack_sequences(g["lengths"], g["max_seq_len"])
    t = len(flat)
    x = _rand(rng, t, h, d)
    full, lse_full = oracle.varlen_attention(x, x, x, cu, cu, 1 / math.sqrt(d), False)
    assert list(full.shape) == g["output_shape"]
    first, lse_first = oracle.varlen_attention(x[cu[:-1]], x, x, None, cu, 1 / math.sqrt(d), False,
                                               query_is_first_token=True)
    assert list(first.shape) == g["first_token_output_shape"]
    assert np.allclose(first, full[cu[:-1]], atol=1e-15)
    assert np.allclose(lse_first, lse_full[:, cu[:-1]], atol=1e-15)


def test_first_token_on_lognormal_batch():
    wl = workloads.make_workload(2, with_values=False)
    lengths = wl.lengths[:40]
    rng = np.random.default_rng(10)
    t = int(lengths.sum())
    q, k, v = _rand(rng, t, 2, 16), _rand(rng, t, 2, 16), _rand(rng, t, 2, 16)
    cu = _cu(lengths)
    full, lf = oracle.varlen_attention(q, k, v, cu, cu, 0.25, False)
    first, l1 = oracle.varlen_attention(q[cu[:-1]], k, v, None, cu, 0.25, False, query_is_first_token=True)
    assert np.allclose(first, full[cu[:-1]], atol=1e-15)
    assert np.allclose(l1, lf[:, cu[:-1]], atol=1e-15)


def test_sequence_independence():
    rng = np.random.default_rng(11)
    lengths = [5, 12, 7]
    h, d = 2, 16
    t = sum(lengths)
    q, k, v = _rand(rng, t, h, d), _rand(rng, t, h, d), _rand(rng, t, h, d)
    cu = _cu(lengths)
    base, _ = oracle.varlen_attention(q, k, v, cu, cu, 0.25, False)
    k2, v2 = k.copy(), v.copy()
    k2[cu[1]:cu[2]] += 3.0
    v2[cu[1]:cu[2]] -= 1.0
    pert, _ = oracle.varlen_attention(q, k2, v2, cu, cu, 0.25, False)
    for i in (0, 2):
        sl = slice(cu[i], cu[i + 1])
        assert np.array_equal(base[sl], pert[sl])
    assert not np.allclose(base[cu[1]:cu[2]], pert[cu[1]:cu[2]])


def test_key_value_permutation_invariance():
    rng = np.random.default_rng(12)
    lengths = [9, 4]
    h, d = 2, 8
    t = sum(lengths)
    q, k, v = _rand(rng, t, h, d), _rand(rng, t, h, d), _rand(rng, t, h, d)
    cu = _cu(lengths)
    base, lb = oracle.varlen_attention(q, k, v, cu, cu, 0.4, False)
    perm = np.concatenate([rng.permutation(9), 9 + rng.permutation(4)])
    out, lo = oracle.varlen_attention(q, k[perm], v[perm], cu, cu, 0.4, False)
    assert np.allclose(base, out, atol=1e-13) and np.allclose(lb, lo, atol=1e-13)


def test_sequence_permutation_moves_blocks():
    rng = np.random.default_rng(13)
    lengths = [3, 6, 2]
    h, d = 1, 8
    t = sum(lengths)
    q, k, v = _rand(rng, t, h, d), _rand(rng, t, h, d), _rand(rng, t, h, d)
    cu = _cu(lengths)
    base, _ = oracle.varlen_attention(q, k, v, cu, cu, 0.4, True)
    order = [2, 0, 1]
    idx = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in order])
    cu2 = _cu([lengths[i] for i in order])
    out, _ = oracle.varlen_attention(q[idx], k[idx], v[idx], cu2, cu2, 0.4, True)
    assert np.array_equal(out, base[idx])


def test_zero_length_sequences_and_unowned_rows():
    rng = np.random.default_rng(14)
    lengths = [4, 0, 3, 0, 0]
    h, d = 2, 8
    cap = 10  # physical capacity rows beyond the active 7
    q, k, v = _rand(rng, cap, h, d), _rand(rng, cap, h, d), _rand(rng, cap, h, d)
    cu = _cu(lengths)
    out, lse = oracle.varlen_attention(q, k, v, cu, cu, 0.3, False)
    ref, _ = oracle.varlen_attention(q[:7], k[:7], v[:7], _cu([4, 3]), _cu([4, 3]), 0.3, False)
    assert np.array_equal(out[:7], ref)
    assert np.all(out[7:] == 0) and np.all(np.isnan(lse[:, 7:]))


def test_causal_bottom_right_with_longer_keys():
    """Lq < Lk: the last query sees every key, the first sees Lk - Lq + 1."""
    rng = np.random.default_rng(15)
    h, d = 1, 8
    q = _rand(rng, 3, h, d)
    k, v = _rand(rng, 5, h, d), _rand(rng, 5, h, d)
    out, _ = oracle.varlen_attention(q, k, v, [0, 3], [0, 5], 0.5, True)
    full, _ = oracle.varlen_attention(q, k, v, [0, 3], [0, 5], 0.5, False)
    assert np.allclose(out[2], full[2], atol=1e-15)
    first, _ = oracle.varlen_attention(q[:1], k[:3], v[:3], [0, 1], [0, 3], 0.5, False)
    assert np.allclose(out[0], first[0], atol=1e-15)


def test_sampled_rows_match_full():
    wl = workloads.make_workload(1)
    cu = wl.cu_seqlens_host()
    out, lse = oracle.varlen_attention(wl.q, wl.k, wl.v, cu, cu, wl.scale, True)
    samples = [(0, 0), (int(cu[3]), 1), (wl.total_tokens - 1, 1), (int(cu[5]) - 1, 0)]
    so, sl = oracle.varlen_attention_rows(wl.q, wl.k, wl.v, cu, cu, wl.scale, True, samples)
    for n, (r, h) in enumerate(samples):
        # one-row and many-row BLAS calls may sum in a different order
        assert np.max(np.abs(so[n] - out[r, h])) < 1e-12
        assert abs(sl[n] - lse[h, r]) < 1e-12


# --------------------------------------------------------------------------
# workload generators
# --------------------------------------------------------------------------

def test_zipf_generator_invariants():
    lengths = workloads.draw_lengths(4)
    assert lengths.sum() == 65536 and lengths.min() >= 1 and len(lengths) == 64
    # a permutation of the rank-ordered split
    rng = np.random.default_rng(0)
    again = workloads.zipf_lengths(65536, 64, rng)
    assert sorted(again.tolist()) == sorted(lengths.tolist())
    # weight proportional to 1/rank: the longest is about total / H_64
    h64 = sum(1.0 / r for r in range(1, 65))
    assert abs(int(lengths.max()) - (65536 - 64) / h64 - 1) <= 1
    with pytest.raises(ValueError):
        workloads.zipf_lengths(10, 11, rng)


def test_zipf_lengths_match_exact_apportionment():
    """The Zipf batch's lengths equal the exact rational largest-remainder
    split of tests/golden/zipf_lengths_workload4.json (written by
    tests/golden/make_zipf_lengths.py with fractions, not floats)."""
    doc = json.load(open(os.path.join(GOLDEN, "zipf_lengths_workload4.json")))
    assert workloads.draw_lengths(4).tolist() == doc["lengths"]
    assert workloads.draw_lengths(6).tolist() == doc["lengths"]
    # sequence i's length follows its rank: longer for a smaller rank
    order = np.argsort(doc["ranks"])
    assert all(np.diff(np.asarray(doc["lengths"])[order]) <= 0)


def test_largest_remainder_apportionment():
    q = np.asarray([2.5, 1.25, 0.25])
    assert workloads._largest_remainder(q, 4).tolist() == [3, 1, 0]
    # equal remainders are served in index order
    assert workloads._largest_remainder(np.asarray([0.5, 0.5, 1.0]), 2).tolist() == [1, 0, 1]


def test_workload_shapes():
    for k in (1, 2, 3, 5):
        lengths = workloads.draw_lengths(k)
        assert lengths.min() >= 1
    assert 1 in workloads.draw_lengths(1).tolist()
    l5 = workloads.draw_lengths(5)
    assert l5[-1] == 32768 and len(l5) == 256 and l5[:-1].min() >= 64 and l5[:-1].max() <= 256
    l3 = workloads.draw_lengths(3)
    assert l3.min() >= 8 and l3.max() <= 384


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by a pin above
# --------------------------------------------------------------------------

def test_planted_causal_sign_error_is_caught(monkeypatch):
    def wrong(positions, lq, lk, causal):
        p = np.asarray(positions)[:, None]
        j = np.arange(lk)[None, :]
        return np.ones((p.shape[0], lk), bool) if not causal else j >= p - (lk - lq)
    monkeypatch.setattr(varlen_oracle, "_visibility", wrong)
    with pytest.raises(AssertionError):
        test_causal_first_and_last_rows()


def test_planted_value_key_swap_is_caught(monkeypatch):
    real = varlen_oracle._attend_one

    def swapped(qi, ki, vi, *a, **kw):
        return real(qi, ki, ki, *a, **kw)
    monkeypatch.setattr(varlen_oracle, "_attend_one", swapped)
    with pytest.raises(AssertionError):
        test_constant_values_pass_through()


def test_planted_dropped_scale_is_caught(monkeypatch):
    real = varlen_oracle._attend_one

    def unscaled(qi, ki, vi, scale, *a, **kw):
        return real(qi, ki, vi, 1.0, *a, **kw)
    monkeypatch.setattr(varlen_oracle, "_attend_one", unscaled)
    with pytest.raises(AssertionError):
        test_attention_matches_padded_sdpa(0, False)


def test_planted_ceil_of_prefix_is_caught(monkeypatch):
    real = varlen_oracle.build_ragged_grid

    def ceil_of_cu(cu_seqlens, block_m):
        bo, gm, order = real(cu_seqlens, block_m)
        cu = np.asarray(cu_seqlens)
        return np.asarray([-(-int(c) // block_m) for c in cu], np.int32), gm, order
    monkeypatch.setattr(oracle, "build_ragged_grid", ceil_of_cu)
    with pytest.raises(AssertionError):
        test_grid_worked_example()
