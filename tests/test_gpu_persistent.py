"""GPU tier: the persistent schedule through the C ABI.

"So you wanna CUDA Graph", "Graph overcapture: bound capacity-sized
launches": a launch recorded for a token and sequence capacity keeps its
size on every replay; the persistent schedule launches at most a fixed
worker count and each worker strides over the tasks that are active in this
replay (read on the device).  Each task computes exactly what the static
grid's workgroup for that task computes, so the checks are bitwise equality
with the static entry points (whose parity with the oracle the other GPU
tests establish) for worker counts from 1 (one workgroup runs every task) up
to the device's resident count, plus a direct oracle comparison and the
cases the schedule exists for: capacities far above the active work with
NaN-poisoned capacity rows that must be neither read nor written, and a
captured HIP graph replayed for different lengths.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import variable_length_packed_pack_amd as vlp
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"
LENGTHS = [1, 63, 64, 65, 129, 0, 300, 17]
WORKERS = [1, 5, 0]  # one worker for everything, an odd count, the resident count


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


_BITS = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.float16: torch.int16}


def _same(a, b):
    """Bitwise equality (NaN payloads included)."""
    return a.dtype == b.dtype and torch.equal(a.view(_BITS[a.dtype]), b.view(_BITS[b.dtype]))


def _fwd_both(q, k, v, cu_q, cu_k, causal, first_token, workers):
    """Static and persistent forward into NaN-filled buffers; returns both."""
    res = []
    for nw in (None, workers):
        out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=DEV)
        lse = torch.full((q.shape[1], q.shape[0]), float("nan"), device=DEV)
        vlp.varlen_attn_fwd(q, k, v, cu_q, cu_k, 0, None, causal, first_token, out=out, lse=lse, num_workers=nw)
        res.append((out, lse))
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("workers", WORKERS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("head_dim", [16, 64, 128])
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_forward_bitwise_equal_to_static_grid(dtype, head_dim, causal, workers):
    wl = workloads.custom_workload(LENGTHS, 3, head_dim, dtype, causal, seed=31)
    cu = _cu(LENGTHS).to(DEV)
    _say(f"[persistent] fwd {dtype} D={head_dim} causal={causal} workers={workers}")
    (o1, l1), (o2, l2) = _fwd_both(wl.q.to(DEV), wl.k.to(DEV), wl.v.to(DEV), cu, cu, causal, False, workers)
    assert _same(o1, o2) and _same(l1, l2)
    assert not torch.isnan(o2.float()).any().item()


@pytest.mark.parametrize("workers", WORKERS)
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_first_token_bitwise_equal_to_static_grid(dtype, workers):
    lengths = [5, 300, 1, 77, 1024, 2, 9]
    wl = workloads.custom_workload(lengths, 6, 64, dtype, False, seed=32)
    cu = _cu(lengths)
    q = wl.q[cu[:-1].long()].contiguous().to(DEV)
    for causal in (False, True):
        (o1, l1), (o2, l2) = _fwd_both(q, wl.k.to(DEV), wl.v.to(DEV), None, cu.to(DEV), causal, True, workers)
        assert _same(o1, o2) and _same(l1, l2)


def test_forward_matches_oracle_with_three_workers():
    lengths = [200, 1, 0, 129, 64]
    wl = workloads.custom_workload(lengths, 4, 128, "bf16", True, seed=33)
    cu = _cu(lengths)
    out, lse = vlp.varlen_attn_fwd(wl.q.to(DEV), wl.k.to(DEV), wl.v.to(DEV), cu.to(DEV), cu.to(DEV), 0, wl.scale,
                                   True, False, num_workers=3)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.varlen_attention(wl.q, wl.k, wl.v, cu.numpy(), cu.numpy(), wl.scale, True)
    err = np.max(np.abs(out.float().cpu().numpy() - ref))
    lerr = np.max(np.abs(lse.cpu().numpy() - ref_lse))
    _say(f"[persistent] oracle, 3 workers: out {err:.3e} lse {lerr:.3e}")
    assert err <= 2e-2 and lerr <= 1e-3


def _capacity_inputs(lengths, cap_rows, cap_seqs, heads, head_dim, dtype, seed):
    """Active lengths padded to cap_seqs sequences with a zero-length tail, in
    buffers of cap_rows rows whose unused rows hold NaN."""
    wl = workloads.custom_workload(lengths, heads, head_dim, dtype, False, seed=seed)
    t = wl.total_tokens
    tdt = workloads.DTYPES[dtype]
    bufs = []
    for src in (wl.q, wl.k, wl.v):
        b = torch.full((cap_rows, heads, head_dim), float("nan"), dtype=tdt)
        b[:t] = src
        bufs.append(b.to(DEV))
    cu = _cu(list(lengths) + [0] * (cap_seqs - len(lengths)))
    return wl, bufs, cu.to(DEV), t


@pytest.mark.parametrize("workers", [0, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_overcaptured_forward(causal, workers):
    """Capacity 16x the active tokens and 64 sequence slots for 5 sequences."""
    lengths = [100, 37, 1, 250, 64]
    wl, (q, k, v), cu, t = _capacity_inputs(lengths, 16 * 452, 64, 8, 128, "bf16", 34)
    (o1, l1), (o2, l2) = _fwd_both(q, k, v, cu, cu, causal, False, workers)
    assert _same(o1, o2) and _same(l1, l2)
    assert torch.isnan(o2[t:].float()).all().item() and torch.isnan(l2[:, t:]).all().item()
    assert not torch.isnan(o2[:t].float()).any().item()


def _bwd_case(lengths, heads, head_dim, dtype, causal, seed, cap_rows=None):
    wl = workloads.custom_workload(lengths, heads, head_dim, dtype, causal, seed=seed)
    t = wl.total_tokens
    rows = t if cap_rows is None else cap_rows
    tdt = workloads.DTYPES[dtype]

    def place(src):
        b = torch.full((rows, heads, head_dim), float("nan"), dtype=tdt)
        b[:t] = src
        return b.to(DEV)
    q, k, v = place(wl.q), place(wl.k), place(wl.v)
    dout = place(workloads.random_dout(t, heads, head_dim, dtype, seed + 100))
    cu = _cu(lengths).to(DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((heads, rows), float("nan"), device=DEV)
    vlp.varlen_attn_fwd(q, k, v, cu, cu, 0, None, causal, False, out=out, lse=lse)
    return q, k, v, out, lse, dout, cu, t


def _bwd_run(case, causal, workers):
    q, k, v, out, lse, dout, cu, _ = case
    grads = [torch.full_like(q, float("nan")) for _ in range(3)]
    vlp.varlen_attn_bwd(q, k, v, out, dout, lse, cu, cu, 0, None, causal, *grads, num_workers=workers)
    torch.cuda.synchronize()
    return grads


@pytest.mark.parametrize("workers", WORKERS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("head_dim", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_backward_bitwise_equal_to_static_grid(dtype, head_dim, causal, workers):
    _say(f"[persistent] bwd {dtype} D={head_dim} causal={causal} workers={workers}")
    case = _bwd_case(LENGTHS, 3, head_dim, dtype, causal, 35)
    g1 = _bwd_run(case, causal, None)
    g2 = _bwd_run(case, causal, workers)
    for a, b in zip(g1, g2):
        assert _same(a, b)
        assert not torch.isnan(b.float()).any().item()


@pytest.mark.parametrize("workers", [0, 6])
def test_overcaptured_backward_leaves_capacity_rows_alone(workers):
    lengths = [100, 1, 250, 64]
    case = _bwd_case(lengths, 8, 128, "bf16", True, 36, cap_rows=8 * 415)
    t = case[-1]
    g1 = _bwd_run(case, True, None)
    g2 = _bwd_run(case, True, workers)
    for a, b in zip(g1, g2):
        assert _same(a, b)
        assert torch.isnan(b[t:].float()).all().item() and not torch.isnan(b[:t].float()).any().item()


@pytest.mark.parametrize("workers", [1, 3, 8, 0])
@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_ragged_matmul_bitwise_equal_to_static_grid(dtype, shared, workers):
    lengths = [1, 127, 128, 129, 0, 300, 5]
    cu = _cu(lengths).to(DEV)
    rows = int(sum(lengths)) + 40
    g = torch.Generator().manual_seed(37)
    tdt = workloads.DTYPES[dtype]
    x = torch.randn(rows, 256, generator=g).to(tdt).to(DEV)
    wshape = (260, 256) if shared else (len(lengths), 260, 256)
    w = (torch.randn(*wshape, generator=g) / 16).to(tdt).to(DEV)
    bias = torch.randn(*wshape[:-1], generator=g).to(tdt).to(DEV)
    y1 = torch.full((rows, 260), float("nan"), dtype=tdt, device=DEV)
    y2 = y1.clone()
    vlp.ragged_matmul(x, w, cu, bias, out=y1)
    vlp.ragged_matmul(x, w, cu, bias, out=y2, num_workers=workers)
    torch.cuda.synchronize()
    assert _same(y1, y2)
    assert torch.isnan(y2[int(sum(lengths)):].float()).all().item()


def test_graph_replays_follow_the_active_lengths():
    """Forward and backward with the persistent schedule captured once in a
    HIP graph for 4096 token rows and 32 sequence slots, replayed for three
    length sets within that capacity (new cu_seqlens and values copied into
    the captured buffers), with eager work and synchronisation between the
    replays; every replay equals an eager static-grid run bit for bit."""
    cap_rows, cap_seqs, heads, head_dim, dtype = 4096, 32, 4, 128, "bf16"
    tdt = workloads.DTYPES[dtype]
    q, k, v, dout = (torch.zeros(cap_rows, heads, head_dim, dtype=tdt, device=DEV) for _ in range(4))
    cu = torch.zeros(cap_seqs + 1, dtype=torch.int32, device=DEV)
    out = torch.zeros_like(q)
    lse = torch.zeros(heads, cap_rows, device=DEV)
    dq, dk, dv = (torch.zeros_like(q) for _ in range(3))
    ws_f = torch.empty(vlp.workspace_size(cap_seqs, cap_rows, 128), dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(vlp.bwd_workspace_size(cap_seqs, cap_rows, cap_rows, heads, 128), dtype=torch.uint8,
                       device=DEV)

    def step():
        vlp.varlen_attn_fwd(q, k, v, cu, cu, 0, None, True, False, out=out, lse=lse, workspace=ws_f,
                            num_workers=0)
        vlp.varlen_attn_bwd(q, k, v, out, dout, lse, cu, cu, 0, None, True, dq, dk, dv, workspace=ws_b,
                            num_workers=0)

    def load(lengths, seed):
        wl = workloads.custom_workload(lengths, heads, head_dim, dtype, True, seed=seed)
        t = wl.total_tokens
        for buf, src in ((q, wl.q), (k, wl.k), (v, wl.v),
                         (dout, workloads.random_dout(t, heads, head_dim, dtype, seed + 1))):
            buf.zero_()
            buf[:t].copy_(src.to(DEV))
        cu.copy_(_cu(list(lengths) + [0] * (cap_seqs - len(lengths))).to(DEV))
        return t

    load([64], 40)
    step()  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for lengths, seed in (([1000, 3, 700, 1], 41), ([4096], 42), ([5] * 32, 43)):
        t = load(lengths, seed)
        for buf in (out, lse, dq, dk, dv):
            buf.fill_(7.0)
        graph.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in (out, lse, dq, dk, dv)]
        ref_out, ref_lse = vlp.varlen_attn_fwd(q, k, v, cu, cu, 0, None, True, False)
        ref_g = vlp.varlen_attn_bwd(q, k, v, ref_out, dout, ref_lse, cu, cu, 0, None, True)
        torch.cuda.synchronize()
        _say(f"[persistent] graph replay, lengths {lengths[:4]}{'...' if len(lengths) > 4 else ''}")
        assert _same(got[0][:t], ref_out[:t]) and _same(got[1][:, :t], ref_lse[:, :t])
        for a, b in zip(got[2:], ref_g):
            assert _same(a[:t], b[:t])


@pytest.mark.parametrize("workers", [1, 5, 8, 13, 0])
def test_every_task_runs_exactly_once(workers):
    """Every task of a persistent launch makes one claim on its queue, so the
    queue counters (in the workspace, after the three grid arrays, one
    256-byte line each) end at the number of tasks of each queue; together
    with the bitwise checks above, every active task ran exactly once and no
    capacity task ran at all."""
    lengths = [100, 37, 1, 250, 64, 0, 0]
    heads, head_dim, dtype = 8, 128, "bf16"
    tdt = workloads.DTYPES[dtype]
    bm = vlp.kernel_block_m(tdt, head_dim, True, False, len(lengths), 0, 0)
    b, t = len(lengths), int(sum(lengths))
    cap_rows = 4 * t
    wl, (q, k, v), cu, _ = _capacity_inputs(lengths[:5], cap_rows, b, heads, head_dim, dtype, 38)
    ws = torch.zeros(vlp.workspace_size(b, cap_rows, bm), dtype=torch.uint8, device=DEV)
    vlp.varlen_attn_fwd(q, k, v, cu, cu, 0, None, True, False, workspace=ws, num_workers=workers)
    torch.cuda.synchronize()

    def up(x):
        return (x + 255) // 256 * 256
    cap = vlp.grid_capacity(cap_rows, b, bm)
    off = up(4 * (b + 1)) + 2 * up(4 * cap)
    counters = ws[off:off + 8 * 256].cpu().view(torch.int32)[::64].tolist()
    tasks = sum((n + bm - 1) // bm for n in lengths) * heads
    width = cap * heads if workers == 0 else min(cap * heads, workers)  # the resident count is >= 8
    nq = min(8, width)
    expect = [len(range(x, tasks, nq)) if x < nq else 0 for x in range(8)]
    _say(f"[persistent] workers={workers}: queue counters {counters}, expected {expect}")
    assert counters == expect
