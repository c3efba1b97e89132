"""GPU tier: the HIP path through the C ABI against the CPU oracle.

Tolerances: out max-abs 1e-4 for fp32 and 2e-2 for bf16/fp16, lse 1e-3, the
oracle running in float64 on the same rounded inputs; metadata bit-exact.
Workloads 1-4 are checked on every row and head (4 at full size, in the
launch configuration the benchmark times); workload 5 on every row of its
255 short sequences and on the first, middle and last row of every query
tile of its 32,768-token sequence, in every head, plus properties of every
row.
"""

import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import variable_length_packed_pack_amd as vlp
import workloads

pytestmark = pytest.mark.gpu

TOL_OUT = {"fp32": 1e-4, "fp16": 2e-2, "bf16": 2e-2}
TOL_LSE = 1e-3
DEV = "cuda"


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


def _to_dev(wl):
    cu = torch.from_numpy(wl.cu_seqlens_host())
    return wl.q.to(DEV), wl.k.to(DEV), wl.v.to(DEV), cu.to(DEV), cu


def _gpu_forward(wl, causal=None, first_token=False, grid=None):
    q, k, v, cu_d, cu_h = _to_dev(wl)
    causal = wl.causal if causal is None else causal
    if first_token:
        q = q[cu_h[:-1].long()].contiguous()
    out, lse = vlp.varlen_attn_fwd(q, k, v, None if first_token else cu_d, cu_d, wl.max_len, wl.scale, causal,
                                   first_token, grid=grid)
    torch.cuda.synchronize()
    return out, lse


def _check_full(wl, causal=None, first_token=False):
    causal = wl.causal if causal is None else causal
    _say(f"[parity] {wl.name} dtype={wl.dtype} B={wl.num_seqs} T={wl.total_tokens} H={wl.heads} "
         f"D={wl.head_dim} causal={causal} first_token={first_token}")
    out, lse = _gpu_forward(wl, causal, first_token)
    cu = wl.cu_seqlens_host()
    q = wl.q[torch.from_numpy(cu[:-1]).long()] if first_token else wl.q
    ref, ref_lse = oracle.varlen_attention(q, wl.k, wl.v, None if first_token else cu, cu, wl.scale, causal,
                                           query_is_first_token=first_token)
    err = np.max(np.abs(out.float().cpu().numpy().astype(np.float64) - ref))
    lerr = np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse))
    _say(f"[parity]   out max-abs {err:.3e}  lse max-abs {lerr:.3e}")
    assert err <= TOL_OUT[wl.dtype], err
    assert lerr <= TOL_LSE, lerr
    return out, lse


# --------------------------------------------------------------------------
# metadata on the device
# --------------------------------------------------------------------------

@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("block_m", [32, 64, 128, 256, vlp.VLP_FIRST_TOKEN_BLOCK_M])
def test_device_grid_bit_exact(k, block_m):
    lengths = workloads.draw_lengths(k)
    cu = _cu(lengths)
    cap = vlp.grid_capacity(int(cu[-1]), len(lengths), block_m)
    g = vlp.build_ragged_grid(cu.to(DEV), block_m, grid_cap=cap)
    bo, gm, to = oracle.build_ragged_grid(cu.numpy(), block_m)
    n = len(gm)
    assert np.array_equal(g.block_offsets.cpu().numpy(), bo)
    assert np.array_equal(g.grid_mapping.cpu().numpy()[:n], gm)
    assert np.array_equal(g.tile_order.cpu().numpy()[:n], to)
    assert np.all(g.grid_mapping.cpu().numpy()[n:] == -1) and np.all(g.tile_order.cpu().numpy()[n:] == -1)


@pytest.mark.parametrize("seed", range(6))
def test_device_grid_fuzz_with_ties_and_empty_tails(seed):
    rng = np.random.default_rng(seed)
    b = int(rng.integers(1, 3000))
    lengths = rng.integers(0, 400, size=b)
    lengths[rng.integers(0, b, size=b // 2)] = 128
    if b > 3:
        lengths[-3:] = 0
    cu = _cu(lengths)
    for bm in (64, 128):
        cap = vlp.grid_capacity(int(cu[-1]) + 17, b, bm)
        g = vlp.build_ragged_grid(cu.to(DEV), bm, grid_cap=cap)
        bo, gm, to = oracle.build_ragged_grid(cu.numpy(), bm)
        assert np.array_equal(g.block_offsets.cpu().numpy(), bo)
        assert np.array_equal(g.grid_mapping.cpu().numpy()[:len(gm)], gm)
        assert np.array_equal(g.tile_order.cpu().numpy()[:len(to)], to)


@pytest.mark.parametrize("b", [1, 2, 63, 64, 65, 127, 1023, 1024, 1025, 2048, 3071, vlp.VLP_DEVICE_SORT_MAX_SEQS])
def test_device_grid_order_at_sort_sizes(b):
    """Longest-first order at sequence counts on both sides of the sort's
    power-of-two and per-thread boundaries, every sequence non-empty, with
    heavy ties."""
    rng = np.random.default_rng(1000 + b)
    lengths = rng.integers(1, 9, size=b) * 32
    cu = _cu(lengths)
    cap = vlp.grid_capacity(int(cu[-1]), b, 64)
    g = vlp.build_ragged_grid(cu.to(DEV), 64, grid_cap=cap)
    bo, gm, to = oracle.build_ragged_grid(cu.numpy(), 64)
    assert np.array_equal(g.block_offsets.cpu().numpy(), bo)
    assert np.array_equal(g.grid_mapping.cpu().numpy()[:len(gm)], gm)
    assert np.array_equal(g.tile_order.cpu().numpy()[:len(to)], to)


def test_device_grid_natural_order_beyond_sort_limit():
    rng = np.random.default_rng(9)
    b = vlp.VLP_DEVICE_SORT_MAX_SEQS + 5
    lengths = rng.integers(0, 50, size=b)
    cu = _cu(lengths)
    cap = vlp.grid_capacity(int(cu[-1]), b, 64)
    g = vlp.build_ragged_grid(cu.to(DEV), 64, grid_cap=cap)
    bo, gm, _ = oracle.build_ragged_grid(cu.numpy(), 64)
    assert np.array_equal(g.block_offsets.cpu().numpy(), bo)
    assert np.array_equal(g.grid_mapping.cpu().numpy()[:len(gm)], gm)
    assert np.array_equal(g.tile_order.cpu().numpy()[:len(gm)], np.arange(len(gm)))


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def test_workload_tiny_fp32():
    wl = workloads.make_workload(1)
    _check_full(wl)
    _check_full(wl, causal=True)
    _check_full(wl, first_token=True)


def test_pack_example_shapes_on_gpu():
    flat, cu = vlp.pack_sequences([3, 1, 2], 3)
    wl = workloads.custom_workload([3, 1, 2], 2, 8 * 2, "fp32", False, seed=5)
    out, _ = _gpu_forward(wl)
    assert list(out.shape) == [6, 2, 16]
    first, _ = _gpu_forward(wl, first_token=True)
    assert list(first.shape) == [3, 2, 16]
    assert flat.tolist() == [0, 1, 2, 3, 6, 7] and cu.tolist() == [0, 3, 4, 6]


def test_workload_graph_fp32():
    wl = workloads.make_workload(2)
    out, lse = _check_full(wl)
    first, lse_first = _check_full(wl, first_token=True)
    cu = wl.cu_seqlens_host()
    rows = torch.from_numpy(cu[:-1]).long().to(DEV)
    # first-token rows equal the full forward's rows cu[:-1] ("Data flow": anchor readout)
    assert (first - out[rows]).abs().max().item() <= 2 * TOL_OUT["fp32"]
    assert (lse_first - lse[:, rows]).abs().max().item() <= 2 * TOL_LSE


def test_workload_encoder_bf16():
    wl = workloads.make_workload(3)
    _check_full(wl)


def test_workload_encoder_fp16():
    wl = workloads.make_workload(3, dtype_override="fp16")
    _check_full(wl)


def _sample_rows(wl, rng, count):
    cu = wl.cu_seqlens_host()
    lengths = wl.lengths
    longest = int(np.argmax(lengths))
    picks = set()
    a, b = int(cu[longest]), int(cu[longest + 1])
    bm = vlp.kernel_block_m(workloads.DTYPES[wl.dtype], wl.head_dim, wl.causal)
    for r in (a, a + 1, a + bm - 1, a + bm, (a + b) // 2, b - bm, b - 1):
        if a <= r < b:
            picks.add(r)
    for i in rng.choice(len(lengths), size=min(16, len(lengths)), replace=False):
        s, e = int(cu[i]), int(cu[i + 1])
        picks.update({s, e - 1, int(rng.integers(s, e))})
    while len(picks) < count:
        picks.add(int(rng.integers(0, wl.total_tokens)))
    rows = sorted(picks)
    return [(r, int(rng.integers(0, wl.heads))) for r in rows]


def _row0_property(wl, out):
    """Causal row 0 of every sequence returns its own value row."""
    cu = wl.cu_seqlens_host()
    first_rows = torch.from_numpy(cu[:-1]).long().to(DEV)
    v0 = wl.v.to(DEV)[first_rows]
    assert (out[first_rows].float() - v0.float()).abs().max().item() <= TOL_OUT[wl.dtype]


def _oracle_per_head(q, k, v, cu_q, cu_k, scale, causal, workers=6):
    """oracle.varlen_attention evaluated one head at a time on a thread pool
    (numpy releases the GIL in its array work); heads are independent, so the
    result is the oracle's own, assembled."""
    from concurrent.futures import ThreadPoolExecutor

    heads = q.shape[1]

    def one(h):
        return oracle.varlen_attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], cu_q, cu_k, scale, causal)

    with ThreadPoolExecutor(max_workers=min(workers, heads)) as ex:
        parts = list(ex.map(one, range(heads)))
    return np.concatenate([o for o, _ in parts], axis=1), np.concatenate([l for _, l in parts], axis=0)


def test_workload_zipf_every_element():
    """The Zipf batch (64 sequences, 65,536 tokens, 16 heads x 128, causal,
    bf16) at full size, in the launch configuration the benchmark times
    (device grid build, static grid): every row and head against the
    oracle."""
    wl = workloads.make_workload(4)
    _say(f"[parity] {wl.name} B={wl.num_seqs} T={wl.total_tokens} H={wl.heads} D={wl.head_dim} "
         f"causal={wl.causal}: every element")
    out, lse = _gpu_forward(wl)
    cu = wl.cu_seqlens_host()
    ref, ref_lse = _oracle_per_head(wl.q, wl.k, wl.v, cu, cu, wl.scale, wl.causal)
    diff = np.abs(out.float().cpu().numpy().astype(np.float64) - ref)
    err = float(diff.max())
    lerr = float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse)))
    worst = np.unravel_index(int(np.argmax(diff)), diff.shape)
    _say(f"[parity]   {out.numel()} outputs: out max-abs {err:.3e} (row {worst[0]}, head {worst[1]}), "
         f"mean-abs {float(diff.mean()):.3e}; {lse.numel()} lse: max-abs {lerr:.3e}")
    assert err <= TOL_OUT[wl.dtype], err
    assert lerr <= TOL_LSE, lerr
    _row0_property(wl, out)


def test_workload_skewed_dense_rows():
    """The skewed batch (255 short sequences + one of 32,768 tokens, 32 heads
    x 128, causal, bf16) at full size: every row and head of the 255 short
    sequences, and the first, middle and last row of every 256-row query tile
    of the long sequence in every head, against the oracle."""
    wl = workloads.make_workload(5)
    _say(f"[parity] {wl.name} B={wl.num_seqs} T={wl.total_tokens} H={wl.heads} D={wl.head_dim} "
         f"causal={wl.causal}: short sequences whole, long sequence by tile rows")
    out, lse = _gpu_forward(wl)
    assert torch.isfinite(out.float()).all().item() and torch.isfinite(lse).all().item()
    cu = wl.cu_seqlens_host()
    long_seq = int(np.argmax(wl.lengths))
    assert long_seq == wl.num_seqs - 1  # the recipe places it last
    short_end = int(cu[long_seq])
    ref, ref_lse = _oracle_per_head(wl.q[:short_end], wl.k, wl.v, cu[:long_seq + 1], cu[:long_seq + 1],
                                    wl.scale, wl.causal)
    got = out[:short_end].float().cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(got - ref)))
    lerr = float(np.max(np.abs(lse[:, :short_end].cpu().numpy().astype(np.float64) - ref_lse)))
    _say(f"[parity]   short sequences, {got.size} outputs: out max-abs {err:.3e} lse max-abs {lerr:.3e}")
    assert err <= TOL_OUT[wl.dtype] and lerr <= TOL_LSE
    a, b = int(cu[long_seq]), int(cu[long_seq + 1])
    tile = 256
    rows = sorted({r for t0 in range(a, b, tile) for r in (t0, t0 + min(tile, b - t0) // 2, min(t0 + tile, b) - 1)})
    samples = [(r, h) for r in rows for h in range(wl.heads)]
    ref_r, ref_rl = oracle.varlen_attention_rows(wl.q, wl.k, wl.v, cu, cu, wl.scale, wl.causal, samples)
    ri = torch.tensor([r for r, _ in samples], device=DEV)
    hi = torch.tensor([h for _, h in samples], device=DEV)
    err = float(np.max(np.abs(out[ri, hi].float().cpu().numpy() - ref_r)))
    lerr = float(np.max(np.abs(lse[hi, ri].cpu().numpy() - ref_rl)))
    _say(f"[parity]   long sequence, {len(samples)} (row, head) pairs over {len(rows)} rows: "
         f"out max-abs {err:.3e} lse max-abs {lerr:.3e}")
    assert err <= TOL_OUT[wl.dtype] and lerr <= TOL_LSE
    _row0_property(wl, out)


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

EDGE_DTYPES = ["fp32", "bf16", "fp16"]


@pytest.mark.parametrize("dtype", EDGE_DTYPES)
@pytest.mark.parametrize("head_dim", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_every_head_dim(dtype, head_dim, causal):
    bm = vlp.kernel_block_m(workloads.DTYPES[dtype], head_dim, causal)
    lengths = [1, bm - 1, bm, bm + 1, 3, 2 * bm + 5, 37]
    wl = workloads.custom_workload(lengths, 3, head_dim, dtype, causal, seed=head_dim + 7 * causal)
    _check_full(wl)


@pytest.mark.parametrize("dtype", EDGE_DTYPES)
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("profile", ["ramp", "step"])
def test_scores_that_outgrow_the_running_max(dtype, head_dim, causal, profile):
    """Keys whose size grows along each sequence, so that later key blocks
    score far above every earlier one and the online softmax must move its
    reference max: "ramp" (key gain 1 + 0.1 j at local position j) moves it
    by about 14 exp2 units, above the rescale threshold, in every 64-key
    block; "step" (gain 1 for the first 64 keys, 64 after) jumps by more
    than 128 exp2 units, beyond the fp32 range of exp2, so no probability
    formed against the old reference can be kept.  q and k are random signs
    (times 0.5 and the gain), so every score is exact in fp32 and the
    comparison measures the softmax, not the rounding of large dot
    products."""
    lengths = [700, 65, 1, 300, 129]
    wl = workloads.custom_workload(lengths, 2, head_dim, dtype, causal, seed=head_dim + (profile == "step"))
    cu = wl.cu_seqlens_host()
    gain = torch.ones(wl.total_tokens, 1, 1)
    for i in range(wl.num_seqs):
        a, b = int(cu[i]), int(cu[i + 1])
        pos = torch.arange(b - a, dtype=torch.float32)
        gain[a:b, 0, 0] = 1.0 + 0.1 * pos if profile == "ramp" else torch.where(pos < 64, 1.0, 64.0)
    wl.k = (torch.sign(wl.k.float()) * gain).to(wl.q.dtype)
    wl.q = (0.5 * torch.sign(wl.q.float())).to(wl.q.dtype)
    _check_full(wl)


@pytest.mark.parametrize("heads,head_dim,dtype", [(32, 16, "bf16"), (64, 64, "fp16"), (32, 128, "bf16"),
                                                   (32, 64, "fp32"), (40, 32, "bf16")])
def test_many_heads_task_order(heads, head_dim, dtype):
    """Head counts that are multiples of 32 run each XCD's heads one after
    another (the other counts interleave them): every (tile, head) still runs
    exactly once -- static grid, persistent schedule with several worker
    counts and cached grid give the same bits, and match the oracle."""
    lengths = [300, 1, 129, 70, 513, 2]
    wl = workloads.custom_workload(lengths, heads, head_dim, dtype, True, seed=heads + head_dim)
    q, k, v, cu_d, cu_h = _to_dev(wl)
    out, lse = vlp.varlen_attn_fwd(q, k, v, cu_d, cu_d, 0, wl.scale, True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.varlen_attention(wl.q, wl.k, wl.v, cu_h.numpy(), cu_h.numpy(), wl.scale, True)
    err = np.max(np.abs(out.float().cpu().numpy() - ref))
    lerr = np.max(np.abs(lse.cpu().numpy() - ref_lse))
    _say(f"[parity] {heads} heads {dtype} D={head_dim}: out {err:.3e} lse {lerr:.3e}")
    assert err <= TOL_OUT[dtype] and lerr <= TOL_LSE
    for nw in (0, 3, 8, 37):
        o2, l2 = vlp.varlen_attn_fwd(q, k, v, cu_d, cu_d, 0, wl.scale, True, num_workers=nw)
        torch.cuda.synchronize()
        assert torch.equal(o2, out) and torch.equal(l2, lse), nw
    bm = vlp.kernel_block_m(q.dtype, head_dim, True)
    host = vlp.build_ragged_grid(cu_h, bm)
    g = vlp.RaggedGrid(host.grid_mapping.to(DEV), host.block_offsets.to(DEV), host.tile_order.to(DEV),
                       host.num_blocks, bm)
    o3, l3 = vlp.varlen_attn_fwd(q, k, v, cu_d, cu_d, 0, wl.scale, True, grid=g)
    torch.cuda.synchronize()
    assert torch.equal(o3, out) and torch.equal(l3, lse)


@pytest.mark.parametrize("dtype", EDGE_DTYPES)
def test_single_long_sequence(dtype):
    wl = workloads.custom_workload([1000], 2, 64, dtype, False, seed=11)
    _check_full(wl)
    _check_full(wl, causal=True)
    _check_full(wl, first_token=True)


def test_batch_of_length_one():
    wl = workloads.custom_workload([1] * 50, 4, 64, "bf16", False, seed=12)
    out, lse = _check_full(wl)
    assert torch.equal(out, wl.v.to(DEV))


def test_zero_length_tail_and_nan_poisoned_capacity():
    """cu_seqlens [0, .., L, L, L] over a larger physical buffer: rows >= L are
    never written, and NaN in the unused capacity rows never leaks in."""
    lengths = [70, 0, 33, 129, 0, 0]
    cap_rows = 300
    h, d = 4, 128
    for dtype in ("bf16", "fp32"):
        wl = workloads.custom_workload(lengths, h, d, dtype, True, seed=13)
        t = wl.total_tokens
        tdt = workloads.DTYPES[dtype]
        q = torch.full((cap_rows, h, d), float("nan"), dtype=tdt)
        k, v = q.clone(), q.clone()
        q[:t], k[:t], v[:t] = wl.q, wl.k, wl.v
        cu = _cu(lengths)
        out = torch.full((cap_rows, h, d), float("nan"), dtype=tdt, device=DEV)
        lse = torch.full((h, cap_rows), float("nan"), device=DEV)
        vlp.varlen_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), cu.to(DEV), 0, wl.scale, True, False,
                            out=out, lse=lse)
        torch.cuda.synchronize()
        ref, ref_lse = oracle.varlen_attention(wl.q, wl.k, wl.v, cu.numpy(), cu.numpy(), wl.scale, True)
        assert np.max(np.abs(out[:t].float().cpu().numpy() - ref)) <= TOL_OUT[dtype]
        assert np.max(np.abs(lse[:, :t].cpu().numpy() - ref_lse)) <= TOL_LSE
        assert torch.isnan(out[t:].float()).all().item() and torch.isnan(lse[:, t:]).all().item()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_zero_scale_gives_uniform_weights(dtype):
    """scale = 0: every visible key weighs the same, also where masking (a
    ragged edge, the causal triangle) cuts a block."""
    wl = workloads.custom_workload([1, 70, 129, 5], 2, 64, dtype, True, seed=15)
    q, k, v, cu_d, cu_h = _to_dev(wl)
    for causal in (False, True):
        out, lse = vlp.varlen_attn_fwd(q, k, v, cu_d, cu_d, 0, 0.0, causal)
        torch.cuda.synchronize()
        ref, ref_lse = oracle.varlen_attention(wl.q, wl.k, wl.v, cu_h.numpy(), cu_h.numpy(), 0.0, causal)
        assert torch.isfinite(out.float()).all().item()
        assert np.max(np.abs(out.float().cpu().numpy() - ref)) <= TOL_OUT[dtype]
        assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= TOL_LSE


@pytest.mark.parametrize("dtype", EDGE_DTYPES)
@pytest.mark.parametrize("head_dim", [16, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_negative_scale(dtype, head_dim, causal):
    """A negative softmax scale (the definition holds for any real scale)
    against the oracle, and bit-identical to the positive scale on negated
    queries: the kernels run |scale| on -q, an exact rewrite."""
    lengths = [1, 70, 300, 129, 5, 257]
    scale = -1.5 / math.sqrt(head_dim)
    wl = workloads.custom_workload(lengths, 2, head_dim, dtype, causal, seed=17 + head_dim)
    q, k, v, cu_d, cu_h = _to_dev(wl)
    out, lse = vlp.varlen_attn_fwd(q, k, v, cu_d, cu_d, 0, scale, causal)
    out2, lse2 = vlp.varlen_attn_fwd(-q, k, v, cu_d, cu_d, 0, -scale, causal)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.varlen_attention(wl.q, wl.k, wl.v, cu_h.numpy(), cu_h.numpy(), scale, causal)
    err = np.max(np.abs(out.float().cpu().numpy() - ref))
    lerr = np.max(np.abs(lse.cpu().numpy() - ref_lse))
    _say(f"[parity] negative scale {dtype} D={head_dim} causal={causal}: out {err:.3e} lse {lerr:.3e}")
    assert err <= TOL_OUT[dtype] and lerr <= TOL_LSE
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    # first-token mode, each form: head-parallel, key split, chunked
    for ft_lengths, hint in (([1, 70, 300, 5], 300), ([1500, 3, 1100], 1500), ([9000, 20, 4097], 9000)):
        wf = workloads.custom_workload(ft_lengths, 2, head_dim, dtype, False, seed=19 + head_dim)
        cu = wf.cu_seqlens_host()
        qf = wf.q[torch.from_numpy(cu[:-1]).long()].contiguous()
        cud = torch.from_numpy(cu).to(DEV)
        for c in (False, True):
            o, l = vlp.varlen_attn_fwd(qf.to(DEV), wf.k.to(DEV), wf.v.to(DEV), None, cud, hint, scale, c, True)
            torch.cuda.synchronize()
            r, rl = oracle.varlen_attention(qf, wf.k, wf.v, None, cu, scale, c, query_is_first_token=True)
            assert np.max(np.abs(o.float().cpu().numpy() - r)) <= TOL_OUT[dtype]
            assert np.max(np.abs(l.cpu().numpy() - rl)) <= TOL_LSE


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_strided_views_of_a_fused_projection(dtype, head_dim):
    """q, k, v as views of one [T, 3, H, D] projection output and out as a
    view into a wider buffer give bit-identical results to contiguous
    copies (the kernels only address rows differently)."""
    lengths = [1, 200, 64, 129, 3, 77]
    t, h = sum(lengths), 3
    tdt = workloads.DTYPES[dtype]
    g = torch.Generator().manual_seed(30 + head_dim)
    qkv = torch.randn(t, 3, h, head_dim, generator=g).to(tdt).to(DEV)
    q, k, v = qkv.unbind(1)
    assert not q.is_contiguous() and q.stride(0) == 3 * h * head_dim
    cu = _cu(lengths).to(DEV)
    scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    for causal in (False, True):
        ref_out, ref_lse = vlp.varlen_attn_fwd(q.contiguous(), k.contiguous(), v.contiguous(), cu, cu, 0, scale,
                                               causal)
        wide = torch.full((t, 2, h, head_dim), float("nan"), dtype=tdt, device=DEV)
        out, lse = vlp.varlen_attn_fwd(q, k, v, cu, cu, 0, scale, causal, out=wide[:, 1])
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        assert torch.isnan(wide[:, 0].float()).all().item()  # the other half of the buffer is untouched
    # first-token mode: one query per sequence, k and v still strided views
    qf = q[cu[:-1].long()].contiguous()
    ref_out, ref_lse = vlp.varlen_attn_fwd(qf, k.contiguous(), v.contiguous(), None, cu, 0, scale, False, True)
    out, lse = vlp.varlen_attn_fwd(qf, k, v, None, cu, 0, scale, False, True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_cross_attention_at_scale_sampled():
    """The cross workload at full size (65,536 keys, 16,408 queries over 64
    sequences, 16 x 128 bf16, non-causal) in the launch configuration the
    benchmark times, checked on sampled rows."""
    wl = workloads.make_workload(6)
    cq, ck = wl.cu_seqlens_q_host(), wl.cu_seqlens_host()
    out, lse = vlp.varlen_attn_fwd(wl.q.to(DEV), wl.k.to(DEV), wl.v.to(DEV), torch.from_numpy(cq).to(DEV),
                                   torch.from_numpy(ck).to(DEV), wl.max_len, wl.scale, False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(88)
    samples = [(int(rng.integers(0, wl.total_queries)), int(rng.integers(0, wl.heads))) for _ in range(64)]
    samples += [(int(cq[i]), 3) for i in (0, 17, 63)] + [(int(cq[i + 1]) - 1, 9) for i in (0, 40)]
    ref, ref_lse = oracle.varlen_attention_rows(wl.q, wl.k, wl.v, cq, ck, wl.scale, False, samples)
    rows = torch.tensor([r for r, _ in samples], device=DEV)
    heads = torch.tensor([h for _, h in samples], device=DEV)
    err = np.max(np.abs(out[rows, heads].float().cpu().numpy() - ref))
    lerr = np.max(np.abs(lse[heads, rows].cpu().numpy() - ref_lse))
    _say(f"[parity] cross at scale, {len(samples)} sampled rows: out {err:.3e} lse {lerr:.3e}")
    assert err <= TOL_OUT["bf16"] and lerr <= TOL_LSE


def test_causal_with_longer_keys():
    """Lq != Lk (cross-attention shapes): bottom-right causal alignment."""
    rng = np.random.default_rng(14)
    lq, lk = [5, 40, 1, 130], [9, 40, 7, 200]
    h, d = 2, 64
    for dtype in ("fp32", "bf16"):
        tdt = workloads.DTYPES[dtype]
        q = torch.from_numpy(rng.standard_normal((sum(lq), h, d), dtype=np.float32)).to(tdt)
        k = torch.from_numpy(rng.standard_normal((sum(lk), h, d), dtype=np.float32)).to(tdt)
        v = torch.from_numpy(rng.standard_normal((sum(lk), h, d), dtype=np.float32)).to(tdt)
        cq, ck = _cu(lq), _cu(lk)
        for causal in (False, True):
            out, lse = vlp.varlen_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV), ck.to(DEV), 0, 0.125,
                                           causal)
            torch.cuda.synchronize()
            ref, ref_lse = oracle.varlen_attention(q, k, v, cq.numpy(), ck.numpy(), 0.125, causal)
            assert np.max(np.abs(out.float().cpu().numpy() - ref)) <= TOL_OUT[dtype]
            assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= TOL_LSE


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_cross_lengths_causal_every_kernel(dtype, head_dim):
    """Lq != Lk in both directions, causal and not, at head dims that run the
    four-wave kernel (64) and, for 16-bit inputs, the two-group kernel (128):
    whole 256-row tiles and single waves with no visible key (their rows give
    0 and lse -inf), tiles whose key range ends inside a block, and key block
    counts of every residue modulo the three-slot ring."""
    lq = [600, 5, 300, 1, 257, 130]
    lk = [100, 9, 700, 1, 3, 200]
    h = 2
    rng = np.random.default_rng(100 + head_dim)
    tdt = workloads.DTYPES[dtype]
    q = torch.from_numpy(rng.standard_normal((sum(lq), h, head_dim), dtype=np.float32)).to(tdt)
    k = torch.from_numpy(rng.standard_normal((sum(lk), h, head_dim), dtype=np.float32)).to(tdt)
    v = torch.from_numpy(rng.standard_normal((sum(lk), h, head_dim), dtype=np.float32)).to(tdt)
    cq, ck = _cu(lq), _cu(lk)
    scale = float(np.float32(1.0 / np.sqrt(head_dim)))
    for causal in (False, True):
        _say(f"[parity] cross lengths {dtype} D={head_dim} causal={causal}")
        out, lse = vlp.varlen_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV), ck.to(DEV), 0, scale, causal)
        torch.cuda.synchronize()
        ref, ref_lse = oracle.varlen_attention(q, k, v, cq.numpy(), ck.numpy(), scale, causal)
        got_lse = lse.cpu().numpy()
        keyless = np.isneginf(ref_lse)
        assert np.array_equal(np.isneginf(got_lse), keyless)
        if causal:
            assert keyless.any()  # the case is exercised
        assert np.max(np.abs(got_lse[~keyless] - ref_lse[~keyless])) <= TOL_LSE
        assert np.max(np.abs(out.float().cpu().numpy() - ref)) <= TOL_OUT[dtype]


def test_causal_query_sees_no_key_gives_zero_and_neg_inf():
    """Lq > Lk with causal alignment leaves the first Lq - Lk queries keyless."""
    h, d = 1, 64
    q = torch.randn(6, h, d).to(torch.bfloat16)
    k = torch.randn(2, h, d).to(torch.bfloat16)
    v = torch.randn(2, h, d).to(torch.bfloat16)
    cq, ck = _cu([6]), _cu([2])
    out, lse = vlp.varlen_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), cq.to(DEV), ck.to(DEV), 0, 0.125, True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.varlen_attention(q, k, v, cq.numpy(), ck.numpy(), 0.125, True)
    assert np.all(out[:4].float().cpu().numpy() == 0) and np.all(np.isneginf(lse[:, :4].cpu().numpy()))
    assert np.max(np.abs(out.float().cpu().numpy() - ref)) <= 2e-2


# --------------------------------------------------------------------------
# invariants (bitwise on the GPU)
# --------------------------------------------------------------------------

def test_deterministic_and_schedule_independent():
    wl = workloads.make_workload(3)
    out1, lse1 = _gpu_forward(wl)
    out2, lse2 = _gpu_forward(wl)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    cu = torch.from_numpy(wl.cu_seqlens_host())
    bm = vlp.kernel_block_m(torch.bfloat16, wl.head_dim)
    host = vlp.build_ragged_grid(cu, bm)
    natural = vlp.RaggedGrid(host.grid_mapping.to(DEV), host.block_offsets.to(DEV), None, host.num_blocks, bm)
    lpt = vlp.RaggedGrid(host.grid_mapping.to(DEV), host.block_offsets.to(DEV), host.tile_order.to(DEV),
                         host.num_blocks, bm)
    out3, lse3 = _gpu_forward(wl, grid=natural)
    out4, lse4 = _gpu_forward(wl, grid=lpt)
    assert torch.equal(out1, out3) and torch.equal(lse1, lse3)
    assert torch.equal(out1, out4) and torch.equal(lse1, lse4)


def test_sequence_independence_bitwise():
    wl = workloads.make_workload(3)
    out1, lse1 = _gpu_forward(wl)
    cu = wl.cu_seqlens_host()
    j = 5
    wl.k[cu[j]:cu[j + 1]] += 1.0
    wl.v[cu[j]:cu[j + 1]] *= -1.0
    out2, lse2 = _gpu_forward(wl)
    keep = torch.ones(wl.total_tokens, dtype=torch.bool)
    keep[cu[j]:cu[j + 1]] = False
    keep = keep.to(DEV)
    assert torch.equal(out1[keep], out2[keep]) and torch.equal(lse1[:, keep], lse2[:, keep])
    assert not torch.equal(out1[~keep], out2[~keep])


def test_sequence_permutation_moves_output_blocks_bitwise():
    wl = workloads.make_workload(2)
    out1, _ = _gpu_forward(wl)
    cu = wl.cu_seqlens_host()
    order = np.random.default_rng(3).permutation(wl.num_seqs)
    idx = torch.from_numpy(np.concatenate([np.arange(cu[i], cu[i + 1]) for i in order])).long()
    wl2 = workloads.custom_workload(wl.lengths[order], wl.heads, wl.head_dim, wl.dtype, wl.causal, seed=0)
    wl2.q, wl2.k, wl2.v = wl.q[idx], wl.k[idx], wl.v[idx]
    out2, _ = _gpu_forward(wl2)
    assert torch.equal(out2, out1[idx.to(DEV)])


def test_host_grid_matches_device_grid_bitwise():
    wl = workloads.make_workload(4)
    out1, lse1 = _gpu_forward(wl)
    cu = torch.from_numpy(wl.cu_seqlens_host())
    bm = vlp.kernel_block_m(torch.bfloat16, wl.head_dim, True)
    host = vlp.build_ragged_grid(cu, bm)
    g = vlp.RaggedGrid(host.grid_mapping.to(DEV), host.block_offsets.to(DEV), host.tile_order.to(DEV),
                       host.num_blocks, bm)
    out2, lse2 = _gpu_forward(wl, grid=g)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


@pytest.mark.parametrize("dtype,head_dim", [("bf16", 128), ("fp16", 128), ("fp32", 64), ("bf16", 32), ("fp16", 16)])
def test_first_token_chunked_form(dtype, head_dim):
    """First-token mode over long sequences with a workspace takes the
    chunked form: 4096-key tiles, one workgroup per (tile, head), the partial
    states merged by the last workgroup of each (sequence, head).  Sequences
    on both sides of the tile boundaries (4095, 4096, 4097, 8192, 12289
    keys), short ones and a single key, in the static and persistent
    schedules and through the no-allocation entry point, against the oracle;
    repeated launches agree bit for bit (the merge order is fixed)."""
    lengths = [4095, 12289, 1, 4096, 70, 4097, 8192, 300, 5]
    wl = workloads.custom_workload(lengths, 3, head_dim, dtype, False, seed=61 + head_dim)
    cu = wl.cu_seqlens_host()
    q = wl.q[torch.from_numpy(cu[:-1]).long()].contiguous()
    ref, ref_lse = oracle.varlen_attention(q, wl.k, wl.v, None, cu, wl.scale, False, query_is_first_token=True)
    qd, kd, vd = q.to(DEV), wl.k.to(DEV), wl.v.to(DEV)
    cud = torch.from_numpy(cu).to(DEV)
    first = None
    for nw in (None, 0, 5):
        for rep in range(2):
            out, lse = vlp.varlen_attn_fwd(qd, kd, vd, None, cud, 12289, wl.scale, False, True, num_workers=nw)
            torch.cuda.synchronize()
            err = np.max(np.abs(out.float().cpu().numpy() - ref))
            lerr = np.max(np.abs(lse.cpu().numpy() - ref_lse))
            _say(f"[parity] first token, chunked {dtype} D={head_dim} workers={nw} rep={rep}: "
                 f"out {err:.3e} lse {lerr:.3e}")
            assert err <= TOL_OUT[dtype] and lerr <= TOL_LSE
            if first is None:
                first = (out.clone(), lse.clone())
            else:
                assert torch.equal(out, first[0]) and torch.equal(lse, first[1])
    import ctypes

    from variable_length_packed_pack_amd import _lib
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((3, len(lengths)), float("nan"), dtype=torch.float32, device=DEV)
    code = {"fp32": _lib.VLP_FP32, "fp16": _lib.VLP_FP16, "bf16": _lib.VLP_BF16}[dtype]
    st = _lib.load().vlp_varlen_attn_fwd_noalloc(
        code, ctypes.c_void_p(qd.data_ptr()), ctypes.c_void_p(kd.data_ptr()), ctypes.c_void_p(vd.data_ptr()), None,
        ctypes.c_void_p(cud.data_ptr()), len(lengths), len(lengths), kd.shape[0], 3, head_dim, 0, 0, 0, 12289,
        wl.scale, 0, 1, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _lib.VLP_OK
    torch.cuda.synchronize()
    assert torch.equal(out, first[0]) and torch.equal(lse, first[1])


@pytest.mark.parametrize("dtype,head_dim", [("bf16", 128), ("fp16", 64), ("fp32", 64), ("fp32", 128), ("bf16", 16)])
def test_first_token_key_split_for_long_sequences(dtype, head_dim):
    """Sequences of thousands of keys: first-token launches split each
    sequence's keys over eight wavefronts (max_seqlen >= 1024, or a mean
    length >= 1024 without the hint); every form against the oracle."""
    lengths = [5000, 3, 1200, 70, 1, 2048]
    wl = workloads.custom_workload(lengths, 3, head_dim, dtype, False, seed=44)
    cu = wl.cu_seqlens_host()
    q = wl.q[torch.from_numpy(cu[:-1]).long()].contiguous()
    cud = torch.from_numpy(cu).to(DEV)
    for causal in (False, True):
        ref, ref_lse = oracle.varlen_attention(q, wl.k, wl.v, None, cu, wl.scale, causal, query_is_first_token=True)
        for max_seqlen, nw in ((5000, None), (0, None), (5000, 0), (100, None)):
            out, lse = vlp.varlen_attn_fwd(q.to(DEV), wl.k.to(DEV), wl.v.to(DEV), None, cud, max_seqlen, wl.scale,
                                           causal, True, num_workers=nw)
            torch.cuda.synchronize()
            err = np.max(np.abs(out.float().cpu().numpy() - ref))
            lerr = np.max(np.abs(lse.cpu().numpy() - ref_lse))
            _say(f"[parity] first token, long sequences {dtype} D={head_dim} causal={causal} "
                 f"max_seqlen={max_seqlen} workers={nw}: out {err:.3e} lse {lerr:.3e}")
            assert err <= TOL_OUT[dtype] and lerr <= TOL_LSE
