"""GPU tier: attention gradients through the C ABI against the CPU oracle.

The HIP forward supplies out and lse, the HIP backward the gradients; the
oracle (``oracle.varlen_attention_bwd``) computes the exact fp64 gradients of
the same rounded q, k, v and dout.

Tolerance (derived; the pages give none for gradients), per gradient row
(one token and head, D elements): max |gpu - oracle| <= 2e-2 + 2^-7 * max
|oracle| over the row, for bf16/fp16.  Where the error comes from:
  * the final rounding to the element type: at most half an ulp, 2^-8 of the
    element for bf16;
  * P and dS are rounded to the element type before their products (matrix
    cores take bf16/fp16 operands), a relative 2^-9 (bf16) per term.  A dK
    row is scale * sum_p dS[p, j] q[p], a sum of terms that largely cancel,
    so this error tracks the size of the terms -- about the size of the
    row's largest elements -- and not the element itself.  Many queries on
    few keys make it largest (the cross-length case below: 66 queries on 2
    keys give errors up to 0.5 % of the row's largest element);
  * delta = rowsum(dO * O) is formed from the element-type forward output,
    which moves it by about 2^-9 * sqrt(D) * |dO| |O| (measured: smaller
    than the dS term).
Together these stay below 2^-7 of the row's largest element; 2e-2 absolute
covers rows of small gradients, as for the forward's output.  fp32 inputs
keep every operand in fp32 (fp32 matrix cores): 1e-4 absolute, as for the
forward's output, plus 2^-14 of the row's largest element for the
accumulation over long rows.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import variable_length_packed_pack_amd as vlp
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"
ATOL = {"fp32": 1e-4, "fp16": 2e-2, "bf16": 2e-2}
RTOL = {"fp32": 2.0 ** -14, "fp16": 2.0 ** -7, "bf16": 2.0 ** -7}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vlp.load_library()
    vlp.check_library_current()
    yield
    torch.cuda.synchronize()


def _cu(lengths):
    return torch.from_numpy(np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32))


def _excess(got, ref, dtype):
    """max over gradient rows of max|got - ref| - (atol + rtol * max|ref|),
    rows along the last axis; <= 0 passes."""
    got = np.asarray(got, dtype=np.float64)
    if not got.size:
        return -1.0
    err = np.max(np.abs(got - ref), axis=-1)
    return float(np.max(err - (ATOL[dtype] + RTOL[dtype] * np.max(np.abs(ref), axis=-1))))


def _run(q, k, v, dout, cu_q, cu_k, scale, causal, max_seqlen=0):
    """HIP forward then HIP backward on device copies; returns host tensors."""
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
    cqd, ckd = cu_q.to(DEV), cu_k.to(DEV)
    out, lse = vlp.varlen_attn_fwd(qd, kd, vd, cqd, ckd, max_seqlen, scale, causal)
    dq, dk, dv = vlp.varlen_attn_bwd(qd, kd, vd, out, dod, lse, cqd, ckd, max_seqlen, scale, causal)
    torch.cuda.synchronize()
    return dq.float().cpu().numpy(), dk.float().cpu().numpy(), dv.float().cpu().numpy()


def _check_all(q, k, v, dout, cu_q, cu_k, scale, causal, dtype, label):
    _say(f"[bwd] {label} dtype={dtype} B={len(cu_q) - 1} Tq={int(cu_q[-1])} Tk={int(cu_k[-1])} "
         f"H={q.shape[1]} D={q.shape[2]} causal={causal}")
    dq, dk, dv = _run(q, k, v, dout, cu_q, cu_k, scale, causal)
    rq, rk, rv = oracle.varlen_attention_bwd(q, k, v, dout, cu_q.numpy(), cu_k.numpy(), scale, causal)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    e = (_excess(dq[:tq], rq[:tq], dtype), _excess(dk[:tk], rk[:tk], dtype), _excess(dv[:tk], rv[:tk], dtype))
    _say(f"[bwd]   excess over tolerance dq {e[0]:.3e} dk {e[1]:.3e} dv {e[2]:.3e}; "
         f"max|ref| {np.max(np.abs(rq)):.2f} {np.max(np.abs(rk)):.2f} {np.max(np.abs(rv)):.2f}")
    assert max(e) <= 0.0, e
    return dq, dk, dv


def _workload_with_grad(k, dtype):
    wl = workloads.make_workload(k, dtype_override=dtype)
    dout = workloads.random_dout(wl.total_tokens, wl.heads, wl.head_dim, wl.dtype, workloads.GRAD_SEED_BASE + k)
    return wl, dout


# --------------------------------------------------------------------------
# whole workloads, every row
# --------------------------------------------------------------------------

@pytest.mark.parametrize("k,dtype", [(1, "fp32"), (1, "bf16"), (2, "fp32"), (2, "bf16"), (2, "fp16"), (3, "bf16"),
                                     (3, "fp16"), (3, "fp32")])
def test_bwd_workload_every_row(k, dtype):
    wl, dout = _workload_with_grad(k, dtype)
    cu = torch.from_numpy(wl.cu_seqlens_host())
    _check_all(wl.q, wl.k, wl.v, dout, cu, cu, wl.scale, wl.causal, dtype, wl.name)
    _check_all(wl.q, wl.k, wl.v, dout, cu, cu, wl.scale, not wl.causal, dtype, wl.name + " (mask flipped)")


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("head_dim", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_every_head_dim(dtype, head_dim, causal):
    bm = vlp.bwd_block_m(workloads.DTYPES[dtype], head_dim, causal)
    lengths = [1, bm - 1, bm, bm + 1, 3, 2 * bm + 5, 37, 64, 65]
    wl = workloads.custom_workload(lengths, 3, head_dim, dtype, causal, seed=100 + head_dim + causal)
    dout = workloads.random_dout(wl.total_tokens, 3, head_dim, dtype, seed=200 + head_dim)
    cu = _cu(lengths)
    _check_all(wl.q, wl.k, wl.v, dout, cu, cu, wl.scale, causal, dtype, f"lengths {lengths}")


def test_bwd_single_long_sequence():
    wl = workloads.custom_workload([1500], 2, 128, "bf16", True, seed=16)
    dout = workloads.random_dout(1500, 2, 128, "bf16", seed=17)
    cu = _cu([1500])
    for causal in (True, False):
        _check_all(wl.q, wl.k, wl.v, dout, cu, cu, wl.scale, causal, "bf16", "one long sequence")


def test_bwd_cross_lengths_keyless_queries_and_unowned_rows():
    """Lq != Lk (bottom-right causal), zero-length sequences on either side,
    queries that see no key, and NaN-poisoned capacity rows that must neither
    leak in nor be written."""
    rng = np.random.default_rng(18)
    lq = [5, 40, 0, 130, 7, 66]
    lk = [9, 40, 3, 200, 0, 2]
    h, d = 2, 128
    cap_q, cap_k = sum(lq) + 11, sum(lk) + 13
    cq, ck = _cu(lq), _cu(lk)
    for dtype in ("bf16", "fp16", "fp32"):
        tdt = workloads.DTYPES[dtype]

        def draw(rows, total):
            x = torch.full((total, h, d), float("nan"), dtype=tdt)
            x[:rows] = torch.from_numpy(rng.standard_normal((rows, h, d), dtype=np.float32)).to(tdt)
            return x
        q, dout = draw(sum(lq), cap_q), draw(sum(lq), cap_q)
        k, v = draw(sum(lk), cap_k), draw(sum(lk), cap_k)
        for causal in (False, True):
            qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, dout))
            out, lse = vlp.varlen_attn_fwd(qd, kd, vd, cq.to(DEV), ck.to(DEV), 0, 0.09, causal)
            dq = torch.full_like(qd, float("nan"))
            dk = torch.full_like(kd, float("nan"))
            dv = torch.full_like(vd, float("nan"))
            vlp.varlen_attn_bwd(qd, kd, vd, out, dod, lse, cq.to(DEV), ck.to(DEV), 0, 0.09, causal, dq, dk, dv)
            torch.cuda.synchronize()
            tq, tk = sum(lq), sum(lk)
            rq, rk, rv = oracle.varlen_attention_bwd(q[:tq], k[:tk], v[:tk], dout[:tq], cq.numpy(), ck.numpy(),
                                                     0.09, causal)
            g = [x.float().cpu().numpy() for x in (dq, dk, dv)]
            e = (_excess(g[0][:tq], rq, dtype), _excess(g[1][:tk], rk, dtype), _excess(g[2][:tk], rv, dtype))
            _say(f"[bwd] cross lengths {dtype} causal={causal}: excess {e}")
            assert max(e) <= 0.0, e
            assert np.isnan(g[0][tq:]).all() and np.isnan(g[1][tk:]).all() and np.isnan(g[2][tk:]).all()
            if causal:  # sequence 0: Lq 5 < Lk 9, so every query sees a key; sequence 5: 64 keyless queries
                s5 = slice(int(cq[5]), int(cq[5]) + 64)
                assert (g[0][s5] == 0).all()


@pytest.mark.parametrize("dtype,head_dim", [("fp32", 64), ("bf16", 128), ("fp16", 64), ("bf16", 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_negative_scale(dtype, head_dim, causal):
    """Gradients under a negative softmax scale against the oracle, and their
    relation to the positive scale on negated queries: dq(q, -s) = -dq(-q, s)
    and dv equal bit for bit (the kernels run |s| with the resident operand of
    the score products negated, so both runs feed the matrix cores the same
    values); dk(q, -s) sums dS q where the other run sums dS (-q), and the
    matrix cores' fp32 accumulation is not symmetric under negation to the
    last bit, so dk agrees to a few ulp."""
    lengths = [1, 70, 300, 129, 65]
    scale = -1.5 / math.sqrt(head_dim)
    wl = workloads.custom_workload(lengths, 2, head_dim, dtype, causal, seed=31 + head_dim)
    dout = workloads.random_dout(wl.total_tokens, 2, head_dim, dtype, seed=32 + head_dim)
    cu = _cu(lengths)
    dq, dk, dv = _check_all(wl.q, wl.k, wl.v, dout, cu, cu, scale, causal, dtype, "negative scale")
    dq2, dk2, dv2 = _run(-wl.q, wl.k, wl.v, dout, cu, cu, -scale, causal)
    for name, a, b in (("dq", dq, -dq2), ("dk", dk, dk2), ("dv", dv, dv2)):
        n = int(np.sum(a != b))
        _say(f"[bwd]   {name}: {n} elements differ from the negated-query run, max {np.max(np.abs(a - b)):.3e}")
        if name == "dk":
            assert np.all(np.abs(a - b) <= 2.0 ** -6 * np.abs(b) + 1e-6)
        else:
            assert n == 0


def test_bwd_zero_scale():
    """scale = 0: uniform weights; dq and dk are exactly zero."""
    lengths = [1, 70, 129, 5]
    wl = workloads.custom_workload(lengths, 2, 64, "bf16", True, seed=19)
    dout = workloads.random_dout(wl.total_tokens, 2, 64, "bf16", seed=20)
    cu = _cu(lengths)
    for causal in (False, True):
        dq, dk, dv = _check_all(wl.q, wl.k, wl.v, dout, cu, cu, 0.0, causal, "bf16", "scale 0")
        assert (dq == 0).all() and (dk == 0).all()


# --------------------------------------------------------------------------
# determinism and independence (bitwise, GPU against itself)
# --------------------------------------------------------------------------

def test_bwd_bitwise_deterministic_and_sequence_independent():
    lengths = [300, 17, 129, 1, 64]
    h, d = 4, 128
    wl = workloads.custom_workload(lengths, h, d, "bf16", True, seed=21)
    dout = workloads.random_dout(wl.total_tokens, h, d, "bf16", seed=22)
    cu = _cu(lengths)
    a = _run(wl.q, wl.k, wl.v, dout, cu, cu, wl.scale, True)
    b = _run(wl.q, wl.k, wl.v, dout, cu, cu, wl.scale, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # perturb sequence 1 only: every other sequence's gradients are unchanged
    s = slice(int(cu[1]), int(cu[2]))
    q2, k2, v2, d2 = wl.q.clone(), wl.k.clone(), wl.v.clone(), dout.clone()
    q2[s] *= 2
    k2[s] += 1
    v2[s] = -v2[s]
    d2[s] *= 3
    c = _run(q2, k2, v2, d2, cu, cu, wl.scale, True)
    keep = np.ones(wl.total_tokens, bool)
    keep[s] = False
    for x, y in zip(a, c):
        assert np.array_equal(x[keep], y[keep])


def test_bwd_cached_grids_phases_and_tile_order_bitwise():
    """The cached-grid entry point equals the workspace one bit for bit, run
    as one call or as the dq phase then the dk/dv phase, with the longest-
    first or the natural tile order."""
    lengths = [300, 17, 0, 129, 1, 64, 200]
    h, d = 4, 128
    wl = workloads.custom_workload(lengths, h, d, "bf16", True, seed=24)
    dout = workloads.random_dout(wl.total_tokens, h, d, "bf16", seed=25)
    cu = _cu(lengths)
    q, k, v, do = (t.to(DEV) for t in (wl.q, wl.k, wl.v, dout))
    cud = cu.to(DEV)
    out, lse = vlp.varlen_attn_fwd(q, k, v, cud, cud, 0, wl.scale, True)
    ref = vlp.varlen_attn_bwd(q, k, v, out, do, lse, cud, cud, 0, wl.scale, True)
    def dev_grid(block):
        gh = vlp.build_ragged_grid(cu, block)
        return vlp.RaggedGrid(gh.grid_mapping.to(DEV), gh.block_offsets.to(DEV), gh.tile_order.to(DEV),
                              gh.num_blocks, block)
    gq = dev_grid(vlp.bwd_block_m(q.dtype, d, True))
    gk = dev_grid(vlp.VLP_BWD_BLOCK_K)
    nq, nk = gq._replace(tile_order=None), gk._replace(tile_order=None)
    for grids, phases in (((gq, gk), (3,)), ((gq, gk), (1, 2)), ((nq, nk), (3,))):
        dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
        stats = torch.empty(2, h, q.shape[0], dtype=torch.float32, device=DEV)
        for ph in phases:
            vlp.varlen_attn_bwd(q, k, v, out, do, lse, cud, cud, 0, wl.scale, True, dq, dk, dv, grids=grids,
                                row_stats=stats, phases=ph)
        torch.cuda.synchronize()
        for x, y in zip((dq, dk, dv), ref):
            assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_bwd_strided_views_of_fused_buffers(dtype, head_dim):
    """q, k, v from one [T, 3, H, D] projection, dout a view into a wider
    buffer, dq/dk/dv written into views of one [T, 3, H, D] gradient buffer:
    bit-identical to contiguous tensors, and nothing outside the views is
    written."""
    lengths = [1, 200, 64, 129, 3, 77]
    t, h = sum(lengths), 2
    tdt = workloads.DTYPES[dtype]
    g = torch.Generator().manual_seed(40 + head_dim)
    qkv = torch.randn(t, 3, h, head_dim, generator=g).to(tdt).to(DEV)
    dwide = torch.randn(t, 2, h, head_dim, generator=g).to(tdt).to(DEV)
    q, k, v = qkv.unbind(1)
    do = dwide[:, 1]
    cu = _cu(lengths).to(DEV)
    scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    for causal in (False, True):
        qc, kc, vc, doc = q.contiguous(), k.contiguous(), v.contiguous(), do.contiguous()
        out, lse = vlp.varlen_attn_fwd(qc, kc, vc, cu, cu, 0, scale, causal)
        ref = vlp.varlen_attn_bwd(qc, kc, vc, out, doc, lse, cu, cu, 0, scale, causal)
        dqkv = torch.full((t, 3, h, head_dim), float("nan"), dtype=tdt, device=DEV)
        dq, dk, dv = dqkv.unbind(1)
        vlp.varlen_attn_bwd(q, k, v, out, do, lse, cu, cu, 0, scale, causal, dq, dk, dv)
        torch.cuda.synchronize()
        for x, y in zip((dq, dk, dv), ref):
            assert torch.equal(x, y)
        assert not torch.isnan(dqkv.float()).any().item()


# --------------------------------------------------------------------------
# the Zipf batch at full size, in the configuration the benchmark times
# --------------------------------------------------------------------------

def test_bwd_zipf_full_size_sampled():
    wl, dout = _workload_with_grad(4, "bf16")
    cu = wl.cu_seqlens_host()
    _say(f"[bwd] zipf full size B={wl.num_seqs} T={wl.total_tokens} H={wl.heads} D={wl.head_dim} causal")
    dq, dk, dv = _run(wl.q, wl.k, wl.v, dout, torch.from_numpy(cu), torch.from_numpy(cu), wl.scale, True,
                      wl.max_len)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    rng = np.random.default_rng(23)
    lengths = np.diff(cu)
    longest = int(np.argmax(lengths))
    q_samples = [(int(rng.integers(0, wl.total_tokens)), int(rng.integers(0, wl.heads))) for _ in range(48)]
    q_samples += [(int(cu[longest + 1]) - 1, 5), (int(cu[longest]), 2)]
    seqs = [longest] + [int(x) for x in rng.choice(np.flatnonzero(lengths < 2000), 3, replace=False)]
    k_samples = []
    for j, i in enumerate(seqs):
        h = int(rng.integers(0, wl.heads))
        rows = [int(cu[i]), int(cu[i + 1]) - 1] + [int(x) for x in rng.integers(cu[i], cu[i + 1], 6)]
        k_samples += [(r, h) for r in rows]
    rq, rk, rv = oracle.varlen_attention_bwd_rows(wl.q, wl.k, wl.v, dout, cu, cu, wl.scale, True,
                                                  q_samples, k_samples)
    gq = np.asarray([dq[r, h] for r, h in q_samples])
    gk = np.asarray([dk[r, h] for r, h in k_samples])
    gv = np.asarray([dv[r, h] for r, h in k_samples])
    e = (_excess(gq, rq, "bf16"), _excess(gk, rk, "bf16"), _excess(gv, rv, "bf16"))
    _say(f"[bwd]   {len(q_samples)} dq rows, {len(k_samples)} dk/dv rows: excess {e}")
    assert max(e) <= 0.0, e
