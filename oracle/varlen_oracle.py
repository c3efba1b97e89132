"""Plain fp64 / integer oracle for packed variable-length attention.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the library.

The oracle takes arrays in and gives arrays out; it draws no random numbers and
reads no files.  Integer metadata is built with pure-Python loops; attention is
numpy float64, one (sequence, head) at a time, with a two-pass softmax (first
the row maximum, then the exponentials), not the online softmax the GPU uses.

Readings taken where the pages leave a point open (each also listed in the
design notes of the repository):

* flat_index is int64 and indexes the row-major padded grid
  ``[num_seqs, max_seq_len]``: token j of sequence i is ``i*max_seq_len + j``.
* block_offsets has ``num_seqs + 1`` entries with a leading 0, the last one
  being the number of active tiles.
* A tile belongs to the unique sequence i with
  ``block_offsets[i] <= f < block_offsets[i+1]``; zero-length sequences own no
  tile.
* tile_order (longest sequence first): sequences sorted by length, longest
  first, ties to the lower index; each contributes its tiles from the last
  local tile down to local tile 0.
* causal masking is in local positions, aligned bottom-right when the query
  and key lengths differ: key j is visible to query p iff
  ``j <= p + (Lk - Lq)``.  A first-token query sits at position 0.
* lse is the natural log of the softmax denominator, ``[H, rows_q]``, and is
  -inf (with a zero output row) when a query sees no key.
"""

from __future__ import annotations

import numpy as np

INT32_MAX = 2**31 - 1


# ---------------------------------------------------------------------------
# Packing ("gigl.nn.packed_attention": "Data flow of a packed forward",
# "Example", "Constraints")
# ---------------------------------------------------------------------------

def pack_sequences(lengths, max_seq_len: int):
    """lengths -> (flat_index int64 [T], cu_seqlens int32 [B+1]).

    cu_seqlens[0] = 0 and cu_seqlens[i+1] = cu_seqlens[i] + lengths[i]; the
    packed buffer is ``padded_grid.flatten()[flat_index]``, so flat_index lists,
    sequence after sequence, the row-major positions of the real tokens in the
    padded ``[B, max_seq_len]`` grid.  Every length must be >= 1 (empty
    sequences are unsupported on that page) and <= max_seq_len, and the token
    count must fit in int32 because cu_seqlens is int32.
    """
    lengths = [int(x) for x in np.asarray(lengths).reshape(-1).tolist()]
    if len(lengths) < 1:
        raise ValueError("need at least one sequence")
    if max_seq_len < 1:
        raise ValueError("max_seq_len must be >= 1")
    cu = [0]
    for i, n in enumerate(lengths):
        if n < 1:
            raise ValueError(f"sequence {i} has length {n} < 1")
        if n > max_seq_len:
            raise ValueError(f"sequence {i} has length {n} > max_seq_len {max_seq_len}")
        cu.append(cu[-1] + n)
        if cu[-1] > INT32_MAX:
            raise OverflowError("token count does not fit in int32")
    flat = []
    for i, n in enumerate(lengths):
        for j in range(n):
            flat.append(i * max_seq_len + j)
    return np.asarray(flat, dtype=np.int64), np.asarray(cu, dtype=np.int32)


# ---------------------------------------------------------------------------
# Ragged grid ("PyCoRa": "CoRa Metadata"; "So you wanna CUDA Graph":
# "Scheduling without max_seqlen")
# ---------------------------------------------------------------------------

def grid_capacity(total_tokens: int, num_seqs: int, block_m: int) -> int:
    """G_cap(T, N, C) = M_max + floor((T - M_max) / C) with M_max = min(T, N).

    The page proves this bounds the number of active tiles for any split of at
    most T tokens over at most N sequences.
    """
    m_max = min(total_tokens, num_seqs)
    return m_max + (total_tokens - m_max) // block_m


def _tiles_of(length: int, block_m: int) -> int:
    """ceil(length / block_m), applied per sequence (chunking restarts at
    every sequence boundary), with integer arithmetic only."""
    tiles = 0
    covered = 0
    while covered < length:
        tiles += 1
        covered += block_m
    return tiles


def build_ragged_grid(cu_seqlens, block_m: int):
    """cu_seqlens -> (block_offsets [B+1], grid_mapping [G], tile_order [G]), int32.

    block_offsets[0] = 0, block_offsets[i+1] = block_offsets[i] + ceil(len_i/C)
    (the page's chunk_offsets); grid_mapping[f] is the sequence owning flat
    tile f; tile_order lists flat tiles longest sequence first (see module
    docstring).
    """
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1).tolist()]
    if len(cu) < 2 or cu[0] != 0:
        raise ValueError("cu_seqlens must start at 0 and have at least 2 entries")
    if block_m < 1:
        raise ValueError("block_m must be >= 1")
    num_seqs = len(cu) - 1
    lengths = []
    for i in range(num_seqs):
        n = cu[i + 1] - cu[i]
        if n < 0:
            raise ValueError("cu_seqlens must be non-decreasing")
        lengths.append(n)

    block_offsets = [0]
    for n in lengths:
        block_offsets.append(block_offsets[-1] + _tiles_of(n, block_m))

    grid_mapping = []
    for i in range(num_seqs):
        for _ in range(block_offsets[i], block_offsets[i + 1]):
            grid_mapping.append(i)

    seq_order = sorted(range(num_seqs), key=lambda i: (-lengths[i], i))
    tile_order = []
    for i in seq_order:
        for t in reversed(range(block_offsets[i + 1] - block_offsets[i])):
            tile_order.append(block_offsets[i] + t)

    return (np.asarray(block_offsets, dtype=np.int32),
            np.asarray(grid_mapping, dtype=np.int32),
            np.asarray(tile_order, dtype=np.int32))


def decode_tile(block_offsets, cu_seqlens, flat_tile: int, block_m: int):
    """Flat tile -> (sequence, local tile, first packed token).

    sequence = (first index whose block_offsets entry exceeds flat_tile) - 1,
    local = flat_tile - block_offsets[sequence],
    token_start = cu_seqlens[sequence] + local * C.
    """
    bo = [int(x) for x in np.asarray(block_offsets).tolist()]
    first_greater = None
    for idx, val in enumerate(bo):
        if val > flat_tile:
            first_greater = idx
            break
    if first_greater is None:
        raise IndexError("flat tile beyond the active tiles")
    seq = first_greater - 1
    local = flat_tile - bo[seq]
    start = int(np.asarray(cu_seqlens)[seq]) + local * block_m
    return seq, local, start


# ---------------------------------------------------------------------------
# Attention ("PyCoRa": "Ragged Flash Attention"; "gigl.nn.packed_attention":
# "packed_attention" and "Example")
# ---------------------------------------------------------------------------

def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor: widen exactly through float32
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def _visibility(positions, lq: int, lk: int, causal: bool) -> np.ndarray:
    """[Rq, Lk] boolean: key j visible to the query at local position p.

    Non-causal: every key of the sequence.  Causal: j <= p + (Lk - Lq).
    """
    p = np.asarray(positions, dtype=np.int64)[:, None]
    j = np.arange(lk, dtype=np.int64)[None, :]
    if not causal:
        return np.ones((p.shape[0], lk), dtype=bool)
    return j <= p + (lk - lq)


def _attend_one(qi, ki, vi, scale: float, causal: bool, positions, lq: int):
    """Exact softmax(scale * q k^T) v for one sequence and head.

    qi [Rq, D] are the query rows at local positions ``positions`` (Lq = lq),
    ki / vi [Lk, D].  Two passes: row max over visible keys, then exp and sum.
    Returns (out [Rq, D], lse [Rq]); rows that see no key give 0 and -inf.
    """
    lk = ki.shape[0]
    rq = qi.shape[0]
    out = np.zeros((rq, vi.shape[1]))
    lse = np.full(rq, -np.inf)
    if lk == 0 or rq == 0:
        return out, lse
    vis = _visibility(positions, lq, lk, causal)            # [Rq, Lk]
    scores = scale * (qi @ ki.T)                              # [Rq, Lk]
    live = vis.any(axis=1)                                    # rows seeing a key
    m = np.where(vis, scores, -np.inf).max(axis=1)            # pass 1: row max
    m_safe = np.where(live, m, 0.0)
    w = np.where(vis, np.exp(scores - m_safe[:, None]), 0.0)  # pass 2: weights
    den = w.sum(axis=1)
    out[live] = (w[live] @ vi) / den[live, None]
    lse[live] = m[live] + np.log(den[live])
    return out, lse


def varlen_attention(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float,
                     causal: bool = False, query_is_first_token: bool = False):
    """Packed attention: every sequence attends only to itself.

    q [rows_q, H, D], k/v [T_k, H, D] (float arrays or CPU tensors, widened to
    float64).  Sequence i owns keys ``k[cu_k[i]:cu_k[i+1]]``; its queries are
    ``q[cu_q[i]:cu_q[i+1]]``, or the single row ``q[i]`` (local position 0)
    when ``query_is_first_token``.  ``scale`` is used as given (callers pass a
    float32 value).  Returns (out [rows_q, H, D] float64, lse [H, rows_q]
    float64).  Rows of q not owned by any sequence stay zero in ``out`` and
    NaN in ``lse`` (the GPU never writes them).
    """
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    cu_q = [int(x) for x in np.asarray(cu_seqlens_q).tolist()] if cu_seqlens_q is not None else None
    cu_k = [int(x) for x in np.asarray(cu_seqlens_k).tolist()]
    num_seqs = len(cu_k) - 1
    rows_q, heads, dim = q64.shape
    out = np.zeros((rows_q, heads, v64.shape[2]))
    lse = np.full((heads, rows_q), np.nan)
    for i in range(num_seqs):
        k0, k1 = cu_k[i], cu_k[i + 1]
        lk = k1 - k0
        if query_is_first_token:
            rows = [i]
            positions = [0]
            lq = lk
        else:
            q0, q1 = cu_q[i], cu_q[i + 1]
            rows = list(range(q0, q1))
            positions = list(range(q1 - q0))
            lq = q1 - q0
        if not rows:
            continue
        for h in range(heads):
            o, l = _attend_one(q64[rows, h, :], k64[k0:k1, h, :], v64[k0:k1, h, :],
                               float(scale), causal, positions, lq)
            out[rows, h, :] = o
            lse[h, rows] = l
    return out, lse


def varlen_attention_rows(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float,
                          causal: bool, samples):
    """The same definition evaluated only at sampled (row, head) pairs.

    For checks at full workload sizes, where the whole oracle would take too
    long.  ``samples`` is a list of (packed query row, head); the row's
    sequence is found by a linear scan of cu_seqlens_q.  Only the slices a
    sample needs are widened to float64.  Returns (out [n, D] float64,
    lse [n] float64).
    """
    cu_q = [int(x) for x in np.asarray(cu_seqlens_q).tolist()]
    cu_k = [int(x) for x in np.asarray(cu_seqlens_k).tolist()]
    # Samples of one (sequence, head) share that sequence's keys: they are
    # evaluated together, each row exactly as in varlen_attention.
    groups = {}
    for n, (row, h) in enumerate(samples):
        seq = None
        for i in range(len(cu_q) - 1):
            if cu_q[i] <= row < cu_q[i + 1]:
                seq = i
                break
        if seq is None:
            raise ValueError(f"row {row} belongs to no sequence")
        groups.setdefault((seq, h), []).append((n, row))
    dim = v.shape[2]
    outs = np.zeros((len(samples), dim))
    lses = np.zeros(len(samples))
    for (seq, h), members in groups.items():
        lq = cu_q[seq + 1] - cu_q[seq]
        k0, k1 = cu_k[seq], cu_k[seq + 1]
        rows = [row for _, row in members]
        qi = _as_f64(q[rows, h, :])
        ki = _as_f64(k[k0:k1, h, :])
        vi = _as_f64(v[k0:k1, h, :])
        o, l = _attend_one(qi, ki, vi, float(scale), causal, [row - cu_q[seq] for row in rows], lq)
        for j, (n, _) in enumerate(members):
            outs[n] = o[j]
            lses[n] = l[j]
    return outs, lses


# ---------------------------------------------------------------------------
# Gradients ("gigl.nn.packed_attention", "Why this exists": training takes the
# gradients of the same packed attention; "So you wanna CUDA Graph",
# "Correctness tangent": gradients of inactive rows may stay undefined;
# "DanLing NestedTensor" 3.4 and 4: gradients flow through the packed payload
# and are checked at the same precision)
#
# The pages define no backward algorithm of their own, so the oracle is the
# gradient of the forward definition written out.  For one sequence and head,
# with P the softmax weights (zero for invisible keys) and dO the incoming
# gradient of the output:
#   dV = P^T dO
#   dP = dO V^T
#   dS = P * (dP - rowsum(P * dP))     (the softmax Jacobian applied row-wise)
#   dQ = scale * dS K,   dK = scale * dS^T Q
# A query that sees no key has P = 0, hence zero dQ and no contribution to
# dK or dV.
# ---------------------------------------------------------------------------

def _attend_one_bwd(qi, ki, vi, doi, scale: float, causal: bool, positions, lq: int):
    """Gradients of sum(dO * softmax(scale q k^T) v) for one sequence and head.

    qi / doi [Rq, D] are the query rows at local positions ``positions``
    (Lq = lq) and their output gradients; ki / vi [Lk, D].  Returns
    (dq [Rq, D], dk [Lk, D], dv [Lk, D]); dk and dv only hold the
    contributions of the given query rows.
    """
    lk = ki.shape[0]
    rq = qi.shape[0]
    dq = np.zeros((rq, qi.shape[1]))
    dk = np.zeros((lk, ki.shape[1]))
    dv = np.zeros((lk, vi.shape[1]))
    if lk == 0 or rq == 0:
        return dq, dk, dv
    vis = _visibility(positions, lq, lk, causal)
    scores = scale * (qi @ ki.T)
    live = vis.any(axis=1)
    m = np.where(vis, scores, -np.inf).max(axis=1)
    m_safe = np.where(live, m, 0.0)
    w = np.where(vis, np.exp(scores - m_safe[:, None]), 0.0)
    den = w.sum(axis=1)
    p = np.zeros_like(w)
    p[live] = w[live] / den[live, None]                   # softmax weights
    dv = p.T @ doi
    dp = doi @ vi.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (ds @ ki)
    dk = scale * (ds.T @ qi)
    return dq, dk, dv


def varlen_attention_bwd(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, scale: float,
                         causal: bool = False):
    """Gradients of packed attention with respect to q, k and v.

    Same conventions as ``varlen_attention`` (no first-token mode): q / dout
    [rows_q, H, D], k / v [T_k, H, D].  Returns (dq [rows_q, H, D],
    dk [T_k, H, D], dv [T_k, H, D]) in float64; rows owned by no sequence stay
    zero (the GPU never writes them).
    """
    q64, k64, v64, do64 = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    cu_q = [int(x) for x in np.asarray(cu_seqlens_q).tolist()]
    cu_k = [int(x) for x in np.asarray(cu_seqlens_k).tolist()]
    heads = q64.shape[1]
    dq = np.zeros(q64.shape)
    dk = np.zeros(k64.shape)
    dv = np.zeros(v64.shape)
    for i in range(len(cu_k) - 1):
        q0, q1 = cu_q[i], cu_q[i + 1]
        k0, k1 = cu_k[i], cu_k[i + 1]
        positions = list(range(q1 - q0))
        for h in range(heads):
            a, b, c = _attend_one_bwd(q64[q0:q1, h], k64[k0:k1, h], v64[k0:k1, h], do64[q0:q1, h],
                                      float(scale), causal, positions, q1 - q0)
            dq[q0:q1, h] = a
            dk[k0:k1, h] = b
            dv[k0:k1, h] = c
    return dq, dk, dv


def varlen_attention_bwd_rows(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, scale: float,
                              causal: bool, q_samples, k_samples):
    """The same gradients at sampled rows, for checks at full workload sizes.

    ``q_samples``: (packed query row, head) pairs -> dq rows (one query row at
    a time: dq of a row depends on that row only).  ``k_samples``: (packed key
    row, head) pairs -> dk and dv rows; every query of the key's sequence
    contributes, so the whole (sequence, head) is evaluated once per distinct
    pair.  Returns (dq [n_q, D], dk [n_k, D], dv [n_k, D]) in float64.
    """
    cu_q = [int(x) for x in np.asarray(cu_seqlens_q).tolist()]
    cu_k = [int(x) for x in np.asarray(cu_seqlens_k).tolist()]

    def owner(cu, row):
        for i in range(len(cu) - 1):
            if cu[i] <= row < cu[i + 1]:
                return i
        raise ValueError(f"row {row} belongs to no sequence")

    dqs = []
    for row, h in q_samples:
        i = owner(cu_q, row)
        k0, k1 = cu_k[i], cu_k[i + 1]
        a, _, _ = _attend_one_bwd(_as_f64(q[row:row + 1, h]), _as_f64(k[k0:k1, h]), _as_f64(v[k0:k1, h]),
                                  _as_f64(dout[row:row + 1, h]), float(scale), causal,
                                  [row - cu_q[i]], cu_q[i + 1] - cu_q[i])
        dqs.append(a[0])
    dks, dvs = [], []
    cache = {}
    for row, h in k_samples:
        i = owner(cu_k, row)
        if (i, h) not in cache:
            q0, q1 = cu_q[i], cu_q[i + 1]
            k0, k1 = cu_k[i], cu_k[i + 1]
            _, b, c = _attend_one_bwd(_as_f64(q[q0:q1, h]), _as_f64(k[k0:k1, h]), _as_f64(v[k0:k1, h]),
                                      _as_f64(dout[q0:q1, h]), float(scale), causal,
                                      list(range(q1 - q0)), q1 - q0)
            cache[(i, h)] = (b, c)
        b, c = cache[(i, h)]
        dks.append(b[row - cu_k[i]])
        dvs.append(c[row - cu_k[i]])
    d = q.shape[2]
    return (np.asarray(dqs).reshape(-1, d), np.asarray(dks).reshape(-1, d),
            np.asarray(dvs).reshape(-1, d))


# ---------------------------------------------------------------------------
# Ragged matrix multiplication ("PyCoRa", "Ragged Matrix Multiplication":
# each sequence of the packed batch is multiplied by its own weight matrix;
# with one weight shared by all sequences this is the packed projection of
# "gigl.nn.packed_attention", "Why this exists": linear layers on the
# [num_tokens, dim] buffer)
# ---------------------------------------------------------------------------

def ragged_matmul(x, weight, cu_seqlens, bias=None, shared_weight=False, shared_bias=False):
    """y[rows of sequence i] = x[rows of sequence i] @ weight_i^T + bias_i.

    x [rows, K]; weight [B, N, K] (one [N, K] matrix per sequence, the
    layout of a linear layer's weight), or [N, K] when ``shared_weight``;
    bias None, [B, N], or [N] when ``shared_bias``.  Returns y [rows, N] in
    float64; rows owned by no sequence stay zero (the GPU never writes them).
    """
    x64 = _as_f64(x)
    w64 = _as_f64(weight)
    b64 = None if bias is None else _as_f64(bias)
    cu = [int(c) for c in np.asarray(cu_seqlens).tolist()]
    n_out = w64.shape[-2]
    y = np.zeros((x64.shape[0], n_out))
    for i in range(len(cu) - 1):
        r0, r1 = cu[i], cu[i + 1]
        if r1 == r0:
            continue
        w = w64 if shared_weight else w64[i]
        y[r0:r1] = x64[r0:r1] @ w.T
        if b64 is not None:
            y[r0:r1] += b64 if shared_bias else b64[i]
    return y


# ---------------------------------------------------------------------------
# Document ids -> cu_seqlens ("DanLing NestedTensor" 3.3: varlen kernels
# consume the partitions' segment boundaries; "So you wanna CUDA Graph",
# "Terminology time": a fixed-capacity cu_seqlens ends in repeated totals
# for the unused slots)
# ---------------------------------------------------------------------------

def cu_seqlens_from_ids(ids, max_seqs: int):
    """Boundaries of the runs of equal ids in one packed sequence.

    ``ids`` [T] integers: tokens of one document are contiguous, and a change
    of id between neighbouring tokens starts a new sequence.  Returns
    (cu [max_seqs + 1] int32 with cu[0] = 0, the run starts, then T repeated
    for the unused slots; num_seqs).  Raises if there are more runs than
    max_seqs.
    """
    ids = [int(x) for x in np.asarray(ids).reshape(-1).tolist()]
    starts = [t for t in range(len(ids)) if t == 0 or ids[t] != ids[t - 1]]
    if len(starts) > max_seqs:
        raise ValueError("more runs than max_seqs")
    cu = starts + [len(ids)] * (max_seqs + 1 - len(starts))
    return np.asarray(cu, dtype=np.int32), len(starts)


def document_masked_attention(q, k, v, ids, scale: float, causal: bool = False):
    """Attention over one packed sequence of T tokens in which query p may
    see key j only if ids[p] == ids[j] (and j <= p when causal): the
    sample-id mask, written as a [T, T] mask over the whole sequence rather
    than per sequence.  Returns (out [T, H, D], lse [H, T]) in float64."""
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    ids = np.asarray(ids).reshape(-1)
    t, heads, _ = q64.shape
    same = ids[:, None] == ids[None, :]
    if causal:
        same = same & np.tril(np.ones((t, t), dtype=bool))
    out = np.zeros((t, heads, v64.shape[2]))
    lse = np.full((heads, t), -np.inf)
    for h in range(heads):
        s = scale * (q64[:, h] @ k64[:, h].T)
        m = np.where(same, s, -np.inf).max(axis=1)
        w = np.where(same, np.exp(s - m[:, None]), 0.0)
        den = w.sum(axis=1)
        out[:, h] = (w @ v64[:, h]) / den[:, None]
        lse[h] = m + np.log(den)
    return out, lse
