"""Benchmark of the packed variable-length attention forward on one MI355X.

One step = one pass of the whole path over one synthetic packed batch:
  1. pack_sequences on the host (lengths -> cu_seqlens, flat_index) into a
     pinned buffer, then an asynchronous copy of cu_seqlens to the device;
  2. the device ragged-grid build (block_offsets, grid_mapping, tile_order,
     and the cleared work queues of the persistent schedule);
  3. the tiled attention forward: one launch of G_cap * heads workgroups,
     the surplus exiting at once (--schedule persistent: the resident number
     of workgroups, taking the G * heads active tile tasks from per-XCD work
     queues).
Q/K/V are resident in HBM before timing starts.  W warm-up steps, then K
timed steps bracketed by synchronisation; the host work of step i overlaps the
GPU work of step i-1.

Also measured in the same run:
  * the attention kernel alone, timed with HIP events on the stream it runs
    on (roofline "achieved"): K launches on a cached grid (static grid), or K
    calls of the entry point minus K grid builds timed alone (persistent);
  * the padded comparator: torch SDPA over [B, H, L_max, D] on the same GPU
    ("DanLing NestedTensor", Appendix C.8: padded attention is masked SDPA over
    the padded envelope), inputs scattered before timing;
  * the CPU oracle on a bounded sample of the same workload (cpu_baseline).
  * the ceilings as this GPU reaches them (measured_peak): the matrix-core
    rate of the element type's MFMA instruction from the library's
    calibration launch, and a plain device copy's streaming rate; the
    attainable rate min(MFMA peak, arithmetic intensity x HBM rate) from the
    datasheet figures and from the measured ones (attainable), with the
    kernel's fraction of each.

Prints ONE JSON line.  Default workload: the Zipf decoder batch (64 sequences,
Zipf s = 1 over 65,536 tokens, 16 heads x 128, causal, bf16).

``--backward`` measures the gradients instead: one step = pack_sequences, the
cu_seqlens copy, two device grid builds, the dq kernel and the dk/dv kernel,
with q, k, v, out, lse and dout resident; the rate counts 2.5x the forward's
algorithmic flops (the five products S, dP, dV, dK, dQ), the roofline is that
of the dk/dv kernel (its four products, 2x the forward's flops), and the
padded comparator is torch SDPA's backward over the padded envelope.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}   # dense MFMA, MI355X datasheet
HBM_PEAK_GBS = 8000.0
METRIC = "varlen attn fwd real-token TFLOP/s (% MFMA peak) + speedup vs padded, 1 GPU"
# Sources of the 16-bit tiled attention kernel (the roofline kernel of the
# bench line); a committed HBM-traffic profile is used only while they match.
KERNEL_SOURCES = ["attn_fwd_mfma.h", "attn_fwd_pingpong.h", "attn_h16.hip", "tile_config.h", "vlp_internal.h"]
# ... of the fp32 tiled kernel and of the first-token kernel (their own
# committed traffic profiles, attn_fwd_<workload> and attn_first_token_<workload>).
KERNEL_SOURCES_F32 = ["attn_fwd_mfma.h", "attn_f32.hip", "tile_config.h", "vlp_internal.h"]
KERNEL_SOURCES_FT = ["attn_first_token.hip", "vlp_internal.h"]
METRIC_BWD = "varlen attn bwd TFLOP/s (2.5x forward real-token flops; % MFMA peak) + speedup vs padded, 1 GPU"
# Sources of the 16-bit dk/dv kernel (the roofline kernel of the backward line).
KERNEL_SOURCES_BWD = ["attn_bwd_mfma.h", "attn_bwd_launch.h", "attn_bwd_h16.hip", "attn_fwd_mfma.h",
                      "tile_config.h", "vlp_internal.h"]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "variable_length_packed_pack_amd", "csrc")
    for name in sources:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_flops(lengths: np.ndarray, heads: int, head_dim: int, causal: bool,
                      first_token: bool = False) -> float:
    """4 * sum N_i^2 * H * D, halved when causal; 4 * sum N_i * H * D with
    one query per sequence (a causal first token sees one key)."""
    if first_token:
        keys = float(len(lengths)) if causal else float(np.sum(lengths.astype(np.float64)))
        return 4.0 * keys * heads * head_dim
    n2 = float(np.sum(lengths.astype(np.float64) ** 2))
    f = 4.0 * n2 * heads * head_dim
    return f / 2 if causal else f


def workload_flops(wl, heads: int, first_token: bool = False) -> float:
    """Algorithmic forward flops of a workload: 4 * sum Lq_i * Lk_i * H * D
    when query and key lengths differ (non-causal), else algorithmic_flops."""
    if wl.lengths_q is not None and not first_token:
        lq = wl.lengths_q.astype(np.float64)
        lk = wl.lengths.astype(np.float64)
        assert not wl.causal
        return 4.0 * float(np.sum(lq * lk)) * heads * wl.head_dim
    return algorithmic_flops(wl.lengths, heads, wl.head_dim, wl.causal, first_token=first_token)


def compulsory_bytes(rows_q: int, total_k: int, heads: int, head_dim: int, elt: int) -> float:
    """q, k, v read once, out written once, lse written once."""
    return (2.0 * rows_q + 2.0 * total_k) * heads * head_dim * elt + 4.0 * rows_q * heads


def measured_peaks(dev, dtype: str):
    """The two ceilings as this GPU reaches them now, each timed with HIP
    events on the stream the work runs on: the matrix-core rate of the
    element type's MFMA instruction (vlp_mfma_rate: one workgroup of eight
    waves per CU, four independent products per wave, no memory traffic) and
    the streaming rate of a plain 1 GiB device copy (bytes read + written)."""
    import torch
    import variable_length_packed_pack_amd as vlp

    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    iters = 8192 if dtype == "fp32" else 16384
    stream = torch.cuda.current_stream(dev)

    def timed(fn, warm, reps):
        for _ in range(warm):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    flops = vlp.mfma_rate(tdt, cus, iters, sink)
    mfma_s = timed(lambda: vlp.mfma_rate(tdt, cus, iters, sink), 2, 5)
    del sink
    nbytes = 1 << 30
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    copy_s = timed(lambda: dst.copy_(src), 2, 5)
    del src, dst
    return {"mfma_tflops": round(flops / mfma_s / 1e12, 1), "copy_gbs": round(2 * nbytes / copy_s / 1e9, 1),
            "method": f"vlp_mfma_rate ({dtype} MFMA, {cus} workgroups x 8 waves x {iters} rounds of 4 independent "
                      "products) and a 1 GiB device copy, HIP events, 5 launches each after 2 warm-ups"}


def attainable(flops: float, nbytes: float, achieved_tflops: float, peak_tflops: float, peaks):
    """Attainable rate = min(MFMA peak, arithmetic intensity x HBM rate), from
    the datasheet figures and, beside them, from the measured ones; and the
    kernel's fraction of each."""
    ai = flops / nbytes
    bound = min(peak_tflops, ai * HBM_PEAK_GBS / 1e3)
    out = {"ai_flop_per_byte": round(ai, 2), "datasheet_tflops": round(bound, 2),
           "frac": round(achieved_tflops / bound, 4)}
    if peaks is not None:
        mb = min(peaks["mfma_tflops"], ai * peaks["copy_gbs"] / 1e3)
        out.update({"measured_tflops": round(mb, 2), "frac_measured": round(achieved_tflops / mb, 4)})
    return out


def traffic_from_profile(workload: str, src_hash: str, kernel: str = "attn_fwd"):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, or None
    when no summary matches the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def trace_of_bench(workload: str, build: str, kernel: str = "attn_fwd"):
    """The committed rocprofv3 kernel trace of this very command (bench.py on
    the same workload, profiled), or None unless it was taken with the
    library build loaded now: its average attention-kernel duration gives the
    trace-derived roofline fraction reported next to the HIP-event one."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_bench_trace.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("library_build") != build:
        return None
    rec["path"] = os.path.relpath(path, ROOT)
    return rec


def cpu_oracle_baseline(wl, budget_s: float, first_token: bool = False):
    """Time the oracle on a bounded sample of the same batch: whole heads (every
    sequence of the batch for that head), one after another, until the
    elapsed time reaches the budget (at least one head)."""
    import oracle  # test infrastructure: used only for this reported baseline

    cu = wl.cu_seqlens_host()
    cu_q = wl.cu_seqlens_q_host()
    rows = cu[:-1].astype(np.int64)
    elapsed, heads_done = 0.0, 0
    while heads_done < wl.heads and (heads_done == 0 or elapsed < budget_s):
        hh = heads_done
        q = wl.q[:, hh:hh + 1].float().numpy()
        k = wl.k[:, hh:hh + 1].float().numpy()
        v = wl.v[:, hh:hh + 1].float().numpy()
        if first_token:
            q = q[rows]
        t0 = time.perf_counter()
        oracle.varlen_attention(q, k, v, None if first_token else cu_q, cu, wl.scale, wl.causal,
                                query_is_first_token=first_token)
        elapsed += time.perf_counter() - t0
        heads_done += 1
    flops = workload_flops(wl, heads_done, first_token=first_token)
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - informational only
        threads = len(os.sched_getaffinity(0))
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{heads_done} of {wl.heads} heads, all {wl.num_seqs} sequences "
                   f"({flops / 1e9:.1f} GFLOP real-token), fp64 numpy, {elapsed:.1f} s"),
        "seconds": elapsed,
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": platform.processor() or platform.machine(),
    }


def padded_comparator(wl, q, k, v, reps: int, first_token: bool = False):
    """torch SDPA over the padded envelope [B, H, L_max, D] (same data),
    chunked over the batch if the envelope is large; returns (ms, backend).
    In first-token mode q is [B, H, D] and the padded query is [B, H, 1, D]."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel

    b, h, d = wl.num_seqs, wl.heads, wl.head_dim
    lmax = wl.max_len
    cu = wl.cu_seqlens_host()
    cross = wl.lengths_q is not None and not first_token
    cu_q = wl.cu_seqlens_q_host()
    lqmax = int(wl.query_lengths().max())
    elt = q.element_size()
    per_seq = 4 * h * lmax * d * elt
    chunk = max(1, min(b, int(40e9 // per_seq)))
    total_ms = 0.0
    backend_used = None
    for c0 in range(0, b, chunk):
        c1 = min(b, c0 + chunk)
        nb = c1 - c0
        kp = torch.zeros(nb, h, lmax, d, dtype=q.dtype, device=q.device)
        vp = torch.zeros_like(kp)
        if first_token:
            qp = q[c0:c1].unsqueeze(2).contiguous()
        elif cross:
            qp = torch.zeros(nb, h, lqmax, d, dtype=q.dtype, device=q.device)
        else:
            qp = torch.zeros_like(kp)
        for j, i in enumerate(range(c0, c1)):
            s, e = int(cu[i]), int(cu[i + 1])
            if cross:
                qs, qe = int(cu_q[i]), int(cu_q[i + 1])
                qp[j, :, : qe - qs] = q[qs:qe].transpose(0, 1)
            elif not first_token:
                qp[j, :, : e - s] = q[s:e].transpose(0, 1)
            kp[j, :, : e - s] = k[s:e].transpose(0, 1)
            vp[j, :, : e - s] = v[s:e].transpose(0, 1)
        mask = None
        if not wl.causal:
            lens = torch.as_tensor(wl.lengths[c0:c1], device=q.device)
            mask = (torch.arange(lmax, device=q.device)[None, :] < lens[:, None])[:, None, None, :]
        ran = None
        for be in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
            if mask is not None and be == SDPBackend.FLASH_ATTENTION:
                continue
            try:
                with sdpa_kernel([be]):
                    torch.nn.functional.scaled_dot_product_attention(qp, kp, vp, attn_mask=mask,
                                                                     is_causal=wl.causal, scale=wl.scale)
                torch.cuda.synchronize()
                ran = be
                break
            except RuntimeError:
                continue
        if ran is None:
            del qp, kp, vp
            return None, "none (no fused SDPA backend accepted the envelope)"
        backend_used = str(ran).split(".")[-1]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with sdpa_kernel([ran]):
            torch.cuda.synchronize()
            start.record()
            for _ in range(reps):
                torch.nn.functional.scaled_dot_product_attention(qp, kp, vp, attn_mask=mask, is_causal=wl.causal,
                                                                 scale=wl.scale)
            end.record()
            torch.cuda.synchronize()
        total_ms += start.elapsed_time(end) / reps
        del qp, kp, vp
        torch.cuda.empty_cache()
    return total_ms, backend_used


def torch_varlen_comparator(wl, q, k, v, cu, ours, reps: int):
    """PyTorch's own variable-length flash-attention forward
    (torch.ops.aten._flash_attention_forward with cumulative sequence
    lengths; this build's ROCm backend) on the same packed q/k/v: the best
    per-kernel time of `reps` rounds of 5 launches (HIP events) and the
    largest absolute difference from this library's output.  Self-attention
    in 16-bit types only (the op takes one cu_seqlens per side and no fp32)."""
    import torch

    lmax = int(wl.max_len)

    def run():
        return torch.ops.aten._flash_attention_forward(q, k, v, cu, cu, lmax, lmax, 0.0, wl.causal, False,
                                                       scale=wl.scale)[0]

    out = run()
    torch.cuda.synchronize()
    diff = float((out.float() - ours.float()).abs().max().item())
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            run()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 5
        best = t if best is None else min(best, t)
    return best, diff


def envelope_own_comparator(wl, dev, reps: int, first_token: bool = False):
    """This library's own forward over the padded envelope: every sequence
    padded to L_max (queries to the longest query length), cu_seqlens =
    [0, L, 2L, ...], timing only (random values).  The padded run then costs
    the same kernel the same work as a rectangular B x L_max grid, which
    isolates the win of ragged scheduling from the quality of the SDPA
    backend.  Sequences are taken in equal chunks of at most ~40 GB of
    q/k/v/out; every chunk does the same work, so the time of one chunk is
    scaled by B / chunk.  Returns ms (or None if one padded sequence alone
    exceeds the budget)."""
    import torch
    import variable_length_packed_pack_amd as vlp

    b, h, d = wl.num_seqs, wl.heads, wl.head_dim
    lk = int(wl.max_len)
    lq = 1 if first_token else int(wl.query_lengths().max())
    tdt = workloads_dtype(wl.dtype)
    elt = torch.tensor([], dtype=tdt).element_size()
    per_seq = (2 * lq + 2 * lk) * h * d * elt
    chunk = min(b, int(40e9 // per_seq))
    if chunk < 1:
        return None
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    q = torch.randn(chunk * lq, h, d, generator=gen, device=dev, dtype=torch.float32).to(tdt)
    k = torch.randn(chunk * lk, h, d, generator=gen, device=dev, dtype=torch.float32).to(tdt)
    v = torch.randn(chunk * lk, h, d, generator=gen, device=dev, dtype=torch.float32).to(tdt)
    cu_k = (torch.arange(chunk + 1, dtype=torch.int32) * lk).to(dev)
    cu_q = None if first_token else (torch.arange(chunk + 1, dtype=torch.int32) * lq).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(h, q.shape[0], dtype=torch.float32, device=dev)
    # the grid runs over the query lengths (first-token mode: over the keys, one tile per sequence)
    grid_cu = torch.arange(chunk + 1, dtype=torch.int32) * (lk if first_token else lq)
    bm = vlp.kernel_block_m(tdt, d, wl.causal, first_token, chunk, q.shape[0], lk)
    gh = vlp.build_ragged_grid(grid_cu, bm)
    grid = vlp.RaggedGrid(gh.grid_mapping.to(dev), gh.block_offsets.to(dev), gh.tile_order.to(dev), gh.num_blocks, bm)
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        def call():
            vlp.varlen_attn_fwd(q, k, v, cu_q, cu_k, lk, wl.scale, wl.causal, first_token, out=out, lse=lse, grid=grid)
        call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        stream.synchronize()
    ms = e0.elapsed_time(e1) / reps * b / chunk
    del q, k, v, out, lse
    torch.cuda.empty_cache()
    return ms


def workloads_dtype(name: str):
    import workloads
    return workloads.DTYPES[name]


def cpu_oracle_baseline_bwd(wl, dout, budget_s: float):
    """The oracle's gradients on whole heads of the same batch until the
    budget is spent (at least one head); rate in 2.5x forward flops."""
    import oracle  # test infrastructure: used only for this reported baseline

    cu = wl.cu_seqlens_host()
    elapsed, heads_done = 0.0, 0
    while heads_done < wl.heads and (heads_done == 0 or elapsed < budget_s):
        hh = heads_done
        sl = slice(hh, hh + 1)
        q, k, v = (x[:, sl].float().numpy() for x in (wl.q, wl.k, wl.v))
        g = dout[:, sl].float().numpy()
        t0 = time.perf_counter()
        oracle.varlen_attention_bwd(q, k, v, g, cu, cu, wl.scale, wl.causal)
        elapsed += time.perf_counter() - t0
        heads_done += 1
    flops = 2.5 * algorithmic_flops(wl.lengths, heads_done, wl.head_dim, wl.causal)
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - informational only
        threads = len(os.sched_getaffinity(0))
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"gradients of {heads_done} of {wl.heads} heads, all {wl.num_seqs} sequences "
                   f"({flops / 1e9:.1f} GFLOP at 2.5x forward), fp64 numpy, {elapsed:.1f} s"),
        "seconds": elapsed,
    }


def padded_backward_comparator(wl, q, k, v, dout, reps: int):
    """torch SDPA's backward over the padded envelope (forward outside the
    timed region), chunked over the batch; returns (ms, backend)."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel

    b, h, d = wl.num_seqs, wl.heads, wl.head_dim
    lmax = wl.max_len
    cu = wl.cu_seqlens_host()
    per_seq = 10 * h * lmax * d * q.element_size()
    chunk = max(1, min(b, int(40e9 // per_seq)))
    total_ms, backend_used = 0.0, None
    for c0 in range(0, b, chunk):
        c1 = min(b, c0 + chunk)
        nb = c1 - c0
        pads = [torch.zeros(nb, h, lmax, d, dtype=q.dtype, device=q.device) for _ in range(4)]
        for j, i in enumerate(range(c0, c1)):
            s0, e0 = int(cu[i]), int(cu[i + 1])
            for src, dst in zip((q, k, v, dout), pads):
                dst[j, :, : e0 - s0] = src[s0:e0].transpose(0, 1)
        qp, kp, vp, dop = pads
        for t in (qp, kp, vp):
            t.requires_grad_(True)
        mask = None
        if not wl.causal:
            lens = torch.as_tensor(wl.lengths[c0:c1], device=q.device)
            mask = (torch.arange(lmax, device=q.device)[None, :] < lens[:, None])[:, None, None, :]
        ran, out = None, None
        for be in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
            if mask is not None and be == SDPBackend.FLASH_ATTENTION:
                continue
            try:
                with sdpa_kernel([be]):
                    out = torch.nn.functional.scaled_dot_product_attention(qp, kp, vp, attn_mask=mask,
                                                                           is_causal=wl.causal, scale=wl.scale)
                    torch.autograd.grad(out, (qp, kp, vp), dop, retain_graph=True)
                torch.cuda.synchronize()
                ran = be
                break
            except RuntimeError:
                out = None
                continue
        if ran is None:
            return None, "none (no fused SDPA backend accepted the envelope)"
        backend_used = str(ran).split(".")[-1]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            torch.autograd.grad(out, (qp, kp, vp), dop, retain_graph=True)
        end.record()
        torch.cuda.synchronize()
        total_ms += start.elapsed_time(end) / reps
        del qp, kp, vp, dop, out, pads
        torch.cuda.empty_cache()
    return total_ms, backend_used


def bench_backward(args, wl, dev) -> int:
    """The gradient step; see the module docstring."""
    import torch

    if wl.lengths_q is not None:
        print("--backward runs on workloads whose query and key lengths agree", file=sys.stderr)
        return 2

    import variable_length_packed_pack_amd as vlp
    import workloads

    k_idx = workloads.WORKLOAD_NAMES[args.workload]
    t, h, d, b = wl.total_tokens, wl.heads, wl.head_dim, wl.num_seqs
    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    dout_host = workloads.random_dout(t, h, d, wl.dtype, workloads.GRAD_SEED_BASE + k_idx)
    dout = dout_host.to(dev)
    cu_host = torch.from_numpy(wl.cu_seqlens_host())
    cu_dev = cu_host.to(dev)
    out, lse = vlp.varlen_attn_fwd(q, k, v, cu_dev, cu_dev, wl.max_len, wl.scale, wl.causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bm = vlp.bwd_block_m(q.dtype, d, wl.causal)
    ws = torch.empty(vlp.bwd_workspace_size(b, t, t, h, bm), dtype=torch.uint8, device=dev)
    fwd_flops = algorithmic_flops(wl.lengths, h, d, wl.causal)
    flops = 2.5 * fwd_flops
    lengths_host = wl.lengths.copy()
    n_steps = args.warmup + args.steps
    pinned = [torch.empty(b + 1, dtype=torch.int32).pin_memory() for _ in range(n_steps)]
    cu_step = torch.empty(b + 1, dtype=torch.int32, device=dev)

    def step(i: int) -> None:
        _, cu = vlp.pack_sequences(lengths_host, wl.max_len)
        pinned[i].copy_(cu)
        cu_step.copy_(pinned[i], non_blocking=True)
        vlp.varlen_attn_bwd(q, k, v, out, dout, lse, cu_step, cu_step, wl.max_len, wl.scale, wl.causal, dq, dk, dv,
                            workspace=ws)

    log(f"[bench] backward: warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] backward: timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.warmup, n_steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # each kernel alone: cached grids, HIP events on the stream they run on
    def dev_grid(block):
        gh = vlp.build_ragged_grid(cu_host, block)
        return vlp.RaggedGrid(gh.grid_mapping.to(dev), gh.block_offsets.to(dev), gh.tile_order.to(dev),
                              gh.num_blocks, block)
    grids = (dev_grid(bm), dev_grid(vlp.VLP_BWD_BLOCK_K))
    stats = torch.empty(2, h, t, dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    reps = args.kernel_only_reps or args.steps
    torch.cuda.synchronize()
    kernel_ms = {}
    with torch.cuda.stream(stream):
        vlp.varlen_attn_bwd(q, k, v, out, dout, lse, cu_dev, cu_dev, wl.max_len, wl.scale, wl.causal, dq, dk, dv,
                            grids=grids, row_stats=stats, phases=vlp.VLP_BWD_DQ | vlp.VLP_BWD_DKDV)
        for name, ph in (("dkdv", vlp.VLP_BWD_DKDV), ("dq", vlp.VLP_BWD_DQ)):
            for _ in range(2):
                vlp.varlen_attn_bwd(q, k, v, out, dout, lse, cu_dev, cu_dev, wl.max_len, wl.scale, wl.causal, dq, dk,
                                    dv, grids=grids, row_stats=stats, phases=ph)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(reps):
                vlp.varlen_attn_bwd(q, k, v, out, dout, lse, cu_dev, cu_dev, wl.max_len, wl.scale, wl.causal, dq, dk,
                                    dv, grids=grids, row_stats=stats, phases=ph)
            ev1.record(stream)
            stream.synchronize()
            kernel_ms[name] = ev0.elapsed_time(ev1) / reps
    torch.cuda.synchronize()

    value = flops / (ms_per_step * 1e-3) / 1e12
    dkdv_flops = 2.0 * fwd_flops
    roof = {"bound": "mfma", "achieved": round(dkdv_flops / (kernel_ms["dkdv"] * 1e-3) / 1e12, 3),
            "peak": PEAK_TFLOPS[wl.dtype], "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    src_hash = kernel_source_hash(KERNEL_SOURCES_BWD)
    traffic = traffic_from_profile(args.workload, src_hash, kernel="attn_bwd_dkdv")
    log(f"[bench] backward step {ms_per_step:.3f} ms  dkdv {kernel_ms['dkdv']:.3f} ms  dq {kernel_ms['dq']:.3f} ms")
    peaks = None if args.no_peaks else measured_peaks(dev, wl.dtype)
    if peaks is not None:
        peaks["frac_mfma"] = round(roof["achieved"] / peaks["mfma_tflops"], 4)

    padded_ms, padded_backend = (None, "skipped")
    if not args.no_padded:
        log("[bench] padded SDPA backward comparator")
        padded_ms, padded_backend = padded_backward_comparator(wl, q, k, v, dout, reps=3)
    torch.cuda.synchronize()
    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline (gradients)")
        cpu = cpu_oracle_baseline_bwd(wl, dout_host, args.cpu_budget)

    rec = {
        "metric": METRIC_BWD,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; no dataset)",
        "config": {"workload": wl.name, "pass": "backward", "num_seqs": b, "total_tokens": t,
                   "max_seqlen": wl.max_len, "heads": h, "head_dim": d, "causal": wl.causal, "block_m": bm},
        "roofline": {**roof, "traffic": traffic},
        "measured_peak": peaks,
        "cpu_baseline": None if cpu is None else {k2: cpu[k2] for k2 in ("value", "unit", "cores", "kind", "sample")},
        "speedup_vs_padded": None if padded_ms is None else round(padded_ms / ms_per_step, 3),
        "padded_ms": None if padded_ms is None else round(padded_ms, 3),
        "padded_backend": padded_backend,
        "kernel_ms": {kk: round(vv, 4) for kk, vv in kernel_ms.items()},
        "dkdv_kernel_tflops": roof["achieved"],
        "dq_kernel_tflops": round(1.5 * fwd_flops / (kernel_ms["dq"] * 1e-3) / 1e12, 3),
        "kernel_source_hash": src_hash,
        "library_build": vlp.build_info(),
        "algorithmic_gflop": round(flops / 1e9, 3),
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_overcapture(args, wl, dev) -> int:
    """Graph replays under overcapture ("So you wanna CUDA Graph", "Graph
    overcapture: bound capacity-sized launches"): the forward (with
    --backward, forward and gradients) is captured once in a HIP graph for a
    token capacity and a sequence-slot capacity R times the workload's (the
    tail of cu_seqlens holds zero-length sequences, the unused rows hold
    zeros) and replayed on the workload's real lengths, under the static grid
    (one workgroup per capacity tile and head, the surplus exiting at once)
    and under the persistent schedule (the resident worker count striding
    over the active tiles).  Prints one JSON line with the replay times."""
    import torch

    import variable_length_packed_pack_amd as vlp
    import workloads

    if wl.lengths_q is not None:
        print("--overcapture runs on workloads whose query and key lengths agree", file=sys.stderr)
        return 2
    ratios = [float(x) for x in args.overcapture.split(",")]
    if any(r < 1.0 for r in ratios):
        print("--overcapture ratios must be >= 1", file=sys.stderr)
        return 2
    k_idx = workloads.WORKLOAD_NAMES[args.workload]
    t, h, d, b = wl.total_tokens, wl.heads, wl.head_dim, wl.num_seqs
    tdt = workloads.DTYPES[wl.dtype]
    bm = vlp.kernel_block_m(tdt, d, wl.causal, False, b, t, wl.max_len)
    dout_host = workloads.random_dout(t, h, d, wl.dtype, workloads.GRAD_SEED_BASE + k_idx) if args.backward else None
    reps = args.steps
    rows = []
    for r in ratios:
        cap_rows, cap_seqs = int(round(r * t)), int(round(r * b))
        q, k, v = (torch.zeros(cap_rows, h, d, dtype=tdt, device=dev) for _ in range(3))
        q[:t].copy_(wl.q.to(dev))
        k[:t].copy_(wl.k.to(dev))
        v[:t].copy_(wl.v.to(dev))
        lengths = np.concatenate([wl.lengths, np.zeros(cap_seqs - b, dtype=np.int32)])
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).to(dev)
        out, lse = torch.zeros_like(q), torch.zeros(h, cap_rows, device=dev)
        ws_f = torch.empty(vlp.workspace_size(cap_seqs, cap_rows, bm), dtype=torch.uint8, device=dev)
        if args.backward:
            dout = torch.zeros_like(q)
            dout[:t].copy_(dout_host.to(dev))
            grads = tuple(torch.zeros_like(q) for _ in range(3))
            ws_b = torch.empty(vlp.bwd_workspace_size(cap_seqs, cap_rows, cap_rows, h,
                                                      vlp.bwd_block_m(tdt, d, wl.causal)), dtype=torch.uint8,
                               device=dev)
        rec = {"capacity_ratio": r, "capacity_tokens": cap_rows, "capacity_seqs": cap_seqs,
               "capacity_tiles": vlp.grid_capacity(cap_rows, cap_seqs, bm),
               "active_tiles": int(np.sum((wl.lengths.astype(np.int64) + bm - 1) // bm))}
        graphs = {}
        for name, nw in (("static", None), ("persistent", 0)):
            def step(nw=nw):
                vlp.varlen_attn_fwd(q, k, v, cu, cu, 0, wl.scale, wl.causal, False, out=out, lse=lse, workspace=ws_f,
                                    num_workers=nw)
                if args.backward:
                    vlp.varlen_attn_bwd(q, k, v, out, dout, lse, cu, cu, 0, wl.scale, wl.causal, *grads,
                                        workspace=ws_b, num_workers=nw)
            step()
            torch.cuda.synchronize()
            graphs[name] = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graphs[name]):
                step()
        # both warmed up alike, then timed in alternating rounds (clocks
        # settle over the first launches of a run): the median round counts
        for _ in range(max(args.warmup, 1)):
            for name in graphs:
                graphs[name].replay()
        torch.cuda.synchronize()
        rounds = {name: [] for name in graphs}
        for rnd in range(5):
            for name in (("static", "persistent") if rnd % 2 == 0 else ("persistent", "static")):
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ev0.record()
                for _ in range(reps):
                    graphs[name].replay()
                ev1.record()
                torch.cuda.synchronize()
                rounds[name].append(ev0.elapsed_time(ev1) / reps)
        for name, vals in rounds.items():
            rec[f"{name}_ms"] = round(sorted(vals)[len(vals) // 2], 4)
        del graphs
        log(f"[bench] overcapture x{r:g}: static {rec['static_ms']:.4f} ms, persistent {rec['persistent_ms']:.4f} ms")
        rows.append(rec)
        del q, k, v, out, lse, ws_f
        if args.backward:
            del dout, grads, ws_b
        torch.cuda.empty_cache()
    print(json.dumps({"mode": "overcapture", "workload": wl.name, "dtype": wl.dtype,
                      "pass": "forward+backward" if args.backward else "forward", "replays": reps, "rounds": 5,
                      "num_seqs": b, "total_tokens": t, "heads": h, "head_dim": d, "causal": wl.causal,
                      "block_m": bm, "rows": rows}), flush=True)
    return 0


def bench_order_ablation(args, wl, dev) -> int:
    """Tile-order ablation: the attention kernel alone on cached grids, tiles
    in longest-first order against the natural (sequence) order, the same
    kernel either way (a NULL tile_order).  On the skewed batch the long
    sequence sits last as drawn (the worst case for the natural order) and
    is also moved first.  Prints one JSON line."""
    import torch

    import variable_length_packed_pack_amd as vlp

    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    t, h, d, b = wl.total_tokens, wl.heads, wl.head_dim, wl.num_seqs
    bm = vlp.kernel_block_m(q.dtype, d, wl.causal, False, b, t, wl.max_len)
    out = torch.empty_like(q)
    lse = torch.empty(h, t, dtype=torch.float32, device=dev)
    arrangements = [("as drawn", wl.lengths)]
    if int(np.argmax(wl.lengths)) != 0:
        i = int(np.argmax(wl.lengths))
        arrangements.append(("longest first", np.concatenate([wl.lengths[i:i + 1], wl.lengths[:i],
                                                               wl.lengths[i + 1:]])))
    flops = algorithmic_flops(wl.lengths, h, d, wl.causal)
    stream = torch.cuda.Stream(device=dev)
    rows = []
    for name, lengths in arrangements:
        cu_host = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
        cu = cu_host.to(dev)
        gh = vlp.build_ragged_grid(cu_host, bm)
        grids = {"longest-first": vlp.RaggedGrid(gh.grid_mapping.to(dev), gh.block_offsets.to(dev),
                                                 gh.tile_order.to(dev), gh.num_blocks, bm),
                 "natural": vlp.RaggedGrid(gh.grid_mapping.to(dev), gh.block_offsets.to(dev), None,
                                           gh.num_blocks, bm)}
        times = {o: [] for o in grids}
        with torch.cuda.stream(stream):
            for o in grids:
                for _ in range(max(args.warmup, 3)):
                    vlp.varlen_attn_fwd(q, k, v, cu, cu, wl.max_len, wl.scale, wl.causal, out=out, lse=lse,
                                        grid=grids[o])
            for rnd in range(5):
                for o in (grids if rnd % 2 == 0 else reversed(list(grids))):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    for _ in range(args.steps):
                        vlp.varlen_attn_fwd(q, k, v, cu, cu, wl.max_len, wl.scale, wl.causal, out=out, lse=lse,
                                            grid=grids[o])
                    e1.record(stream)
                    stream.synchronize()
                    times[o].append(e0.elapsed_time(e1) / args.steps)
        rec = {"arrangement": name}
        for o, vals in times.items():
            ms = sorted(vals)[len(vals) // 2]
            rec[f"{o}_ms"] = round(ms, 4)
            rec[f"{o}_tflops"] = round(flops / (ms * 1e-3) / 1e12, 2)
        log(f"[bench] tile order, {name}: longest-first {rec['longest-first_ms']:.4f} ms, "
            f"natural {rec['natural_ms']:.4f} ms")
        rows.append(rec)
    print(json.dumps({"mode": "tile-order ablation", "workload": wl.name, "dtype": wl.dtype, "heads": h,
                      "head_dim": d, "causal": wl.causal, "block_m": bm, "launches_per_round": args.steps,
                      "rounds": 5, "rows": rows}), flush=True)
    return 0


def bench_matmul(args, wl, dev) -> int:
    """Ragged matrix multiplication on the workload's token split: the packed
    QKV projection (hidden = heads x head_dim -> 3 x hidden, one shared
    weight) or, with --matmul per-seq, one [hidden, hidden] weight per
    sequence ("PyCoRa", "Ragged Matrix Multiplication")."""
    import torch

    import variable_length_packed_pack_amd as vlp

    t, b = wl.total_tokens, wl.num_seqs
    hidden = wl.heads * wl.head_dim
    per_seq = args.matmul == "per-seq"
    n_out = hidden if per_seq else 3 * hidden
    g = torch.Generator(device="cpu").manual_seed(77)
    tdt = torch.bfloat16
    x = torch.randn(t, hidden, generator=g).to(tdt).to(dev)
    wshape = (b, n_out, hidden) if per_seq else (n_out, hidden)
    w = (torch.randn(*wshape, generator=g) / math.sqrt(hidden)).to(tdt).to(dev)
    cu_host = torch.from_numpy(wl.cu_seqlens_host())
    cu = cu_host.to(dev)
    y = torch.empty(t, n_out, dtype=tdt, device=dev)
    nb = vlp._lib.load()  # noqa: F841  (loads the library before timing)
    ws_bytes = __import__("ctypes").c_size_t(0)
    vlp._lib.check(vlp._lib.load().vlp_ragged_matmul_workspace_size(b, t, __import__("ctypes").addressof(ws_bytes)),
                   "workspace")
    ws = torch.empty(max(int(ws_bytes.value), 256), dtype=torch.uint8, device=dev)
    flops = 2.0 * t * hidden * n_out
    nbytes = 2.0 * (t * hidden + (b if per_seq else 1) * n_out * hidden + t * n_out)

    def run():
        vlp.ragged_matmul(x, w, cu, None, out=y, workspace=ws)

    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            run()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(args.steps):
            run()
        ev1.record(stream)
    stream.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps

    # library reference on the same packed rows (hipBLASLt through torch)
    lib_ms = None
    with torch.cuda.stream(stream):
        if per_seq:
            def ref():
                for i in range(b):
                    s0, e0 = int(cu_host[i]), int(cu_host[i + 1])
                    torch.matmul(x[s0:e0], w[i].t(), out=y[s0:e0])
        else:
            def ref():
                torch.matmul(x, w.t(), out=y)
        for _ in range(3):
            ref()
        ev0.record(stream)
        for _ in range(args.steps):
            ref()
        ev1.record(stream)
    stream.synchronize()
    lib_ms = ev0.elapsed_time(ev1) / args.steps

    cpu = None
    if not args.no_cpu:
        import oracle  # test infrastructure: used only for this reported baseline
        xs, ws_ = x.float().cpu(), w.float().cpu()
        elapsed, done, fl = 0.0, 0, 0.0
        order = np.argsort(-wl.lengths)[::-1]  # shortest sequences first, until the budget is spent
        for i in order:
            s0, e0 = int(cu_host[i]), int(cu_host[i + 1])
            cu1 = np.array([0, e0 - s0], dtype=np.int32)
            t0 = time.perf_counter()
            oracle.ragged_matmul(xs[s0:e0], ws_[i:i + 1] if per_seq else ws_, cu1, shared_weight=not per_seq)
            elapsed += time.perf_counter() - t0
            done += 1
            fl += 2.0 * (e0 - s0) * hidden * n_out
            if elapsed > args.cpu_budget:
                break
        cpu = {"value": fl / elapsed / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
               "kind": "oracle",
               "sample": f"{done} of {b} sequences (shortest first), fp64 numpy, {fl / 1e9:.1f} GFLOP, {elapsed:.1f} s"}

    achieved = flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": "ragged matmul TFLOP/s (% MFMA peak), 1 GPU",
        "value": round(achieved, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; no dataset)",
        "config": {"workload": wl.name + (" per-sequence weights" if per_seq else " shared QKV projection"),
                   "rows": t, "num_seqs": b, "in_features": hidden, "out_features": n_out,
                   "weights": b if per_seq else 1},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4), "traffic": None},
        "cpu_baseline": cpu,
        "library_gemm_ms": round(lib_ms, 4),
        "library_gemm_tflops": round(flops / (lib_ms * 1e-3) / 1e12, 3),
        "vs_library_gemm": round(lib_ms / ms, 3),
        "algorithmic_gflop": round(flops / 1e9, 3),
        "compulsory_gb": round(nbytes / 1e9, 4),
        "library_build": vlp.build_info(),
        "note": "each timed call includes the device grid build (~10 us)",
    }
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="zipf", help="tiny | graph | encoder | zipf | skewed | cross")
    ap.add_argument("--no-padded", action="store_true", help="skip the padded SDPA comparator")
    ap.add_argument("--torch-varlen", action="store_true",
                    help="also time PyTorch's own varlen flash-attention forward on the same packed batch "
                         "(16-bit self-attention workloads; off by default)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured MFMA and device-copy ceilings (measured_peak, attainable.*measured)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work (approx.)")
    ap.add_argument("--kernel-only-reps", type=int, default=0, help="attention-kernel launches (0 = steps)")
    ap.add_argument("--first-token", action="store_true",
                    help="query_is_first_token mode: one query per sequence (its first token)")
    ap.add_argument("--no-causal", action="store_true",
                    help="run the workload without its causal mask (e.g. first-token mode over all keys of the "
                         "Zipf batch's long sequences)")
    ap.add_argument("--backward", action="store_true",
                    help="measure the gradients (dq, dk, dv) instead of the forward")
    ap.add_argument("--matmul", choices=["shared", "per-seq"], default=None,
                    help="measure the ragged matrix multiplication on the workload's token split instead")
    ap.add_argument("--schedule", choices=["static", "persistent"], default="static",
                    help="forward launch schedule: the static grid (G_cap * heads workgroups) or persistent workers")
    ap.add_argument("--order-ablation", action="store_true",
                    help="kernel time with longest-first against natural tile order (skewed: also long first)")
    ap.add_argument("--overcapture", default=None, metavar="R1,R2,...",
                    help="graph replays captured for R times the workload's token and sequence capacity, "
                         "static grid against persistent schedule (with --backward: forward and gradients)")
    ap.add_argument("--hbm-reference", action="store_true",
                    help="only time a 4 GiB device-to-device copy (torch) and print the achieved bandwidth: the "
                         "streaming rate a plain library kernel reaches on this GPU, beside the 8 TB/s datasheet "
                         "peak that the HBM-bound rooflines are quoted against")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (3 times) and exit: the "
                         "reference point that scales the FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the forward needs no exchange; see the design notes on sharding).", file=sys.stderr)
        return 2

    import torch

    import variable_length_packed_pack_amd as vlp
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    if args.hbm_reference:
        nbytes = 4 << 30
        src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        print(json.dumps({"hbm_reference": "torch device copy", "bytes_read": nbytes, "bytes_written": nbytes,
                          "ms": round(ms, 4), "GB_per_s": round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
                          "frac_of_8TBps": round(2 * nbytes / (ms * 1e-3) / 8e12, 4)}), flush=True)
        return 0
    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": nbytes, "launches": 3}), flush=True)
        return 0
    vlp.load_library()
    lib_hash = vlp.check_library_current()  # refuses a libvlp.so built from other sources
    k_idx = workloads.WORKLOAD_NAMES[args.workload]
    log(f"[bench] generating workload {args.workload}")
    wl = workloads.make_workload(k_idx)
    if args.no_causal:
        wl.causal = False
    if args.matmul:
        return bench_matmul(args, wl, dev)
    if args.overcapture:
        return bench_overcapture(args, wl, dev)
    if args.order_ablation:
        if wl.lengths_q is not None:
            print("--order-ablation runs on workloads whose query and key lengths agree", file=sys.stderr)
            return 2
        return bench_order_ablation(args, wl, dev)
    if args.backward:
        if args.first_token:
            print("--backward has no first-token mode", file=sys.stderr)
            return 2
        return bench_backward(args, wl, dev)
    ft = args.first_token
    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    t, h, d = wl.total_tokens, wl.heads, wl.head_dim
    b = wl.num_seqs
    if ft:
        # one query per sequence: the row cu_seqlens[i] of the packed batch
        q = q[torch.from_numpy(wl.cu_seqlens_host()[:-1]).long().to(dev)].contiguous()
    rows_q = q.shape[0]
    schedule = args.schedule
    workers = 0 if schedule == "persistent" else None
    flops = workload_flops(wl, h, first_token=ft)
    out = torch.empty_like(q)
    lse = torch.empty(h, rows_q, dtype=torch.float32, device=dev)
    bm = vlp.kernel_block_m(q.dtype, d, wl.causal, ft, b, rows_q, wl.max_len)
    ws = torch.empty(vlp.fwd_workspace_size(q.dtype, b, rows_q, t, h, d, wl.max_len, wl.causal, ft),
                     dtype=torch.uint8, device=dev)
    cu_dev = torch.empty(b + 1, dtype=torch.int32, device=dev)
    lengths_host = wl.lengths.copy()
    cross = wl.lengths_q is not None and not ft
    cu_q_dev = torch.empty(b + 1, dtype=torch.int32, device=dev) if cross else cu_dev
    lengths_q_host = wl.query_lengths().copy()
    n_steps = args.warmup + args.steps
    pinned = [torch.empty(b + 1, dtype=torch.int32).pin_memory() for _ in range(n_steps)]
    pinned_q = [torch.empty(b + 1, dtype=torch.int32).pin_memory() for _ in range(n_steps)] if cross else None

    def step(i: int) -> None:
        flat, cu = vlp.pack_sequences(lengths_host, wl.max_len)
        pinned[i].copy_(cu)
        cu_dev.copy_(pinned[i], non_blocking=True)
        if cross:  # query boundaries of their own
            _, cuq = vlp.pack_sequences(lengths_q_host, int(lengths_q_host.max()))
            pinned_q[i].copy_(cuq)
            cu_q_dev.copy_(pinned_q[i], non_blocking=True)
        vlp.varlen_attn_fwd(q, k, v, cu_q_dev, cu_dev, wl.max_len, wl.scale, wl.causal, ft, out=out, lse=lse,
                            workspace=ws, num_workers=workers)

    log(f"[bench] warmup {args.warmup} steps ({schedule} schedule)")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.warmup, n_steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # host cost of pack_sequences alone (for the record)
    tp = time.perf_counter()
    for _ in range(20):
        vlp.pack_sequences(lengths_host, wl.max_len)
    pack_us = (time.perf_counter() - tp) * 1e6 / 20

    # Attention kernel alone, HIP events on the launch stream.  Static grid:
    # launches on a cached device grid.  Persistent schedule (its queues are
    # cleared by the grid build of each call): calls through the device-grid
    # entry point minus the same number of grid builds timed alone.
    cu_host = torch.from_numpy(wl.cu_seqlens_host())
    grid_host = vlp.build_ragged_grid(cu_host if ft else torch.from_numpy(wl.cu_seqlens_q_host()), bm)
    grid = vlp.RaggedGrid(grid_host.grid_mapping.to(dev), grid_host.block_offsets.to(dev),
                          grid_host.tile_order.to(dev), grid_host.num_blocks, bm)
    stream = torch.cuda.Stream(device=dev)
    reps = args.kernel_only_reps or args.steps
    torch.cuda.synchronize()

    def timed(fn) -> float:
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        stream.synchronize()
        return e0.elapsed_time(e1) / reps

    grid_build_ms = None
    # first-token mode over long sequences runs the chunked form, whose grid
    # (over the keys, VLP_FIRST_TOKEN_CHUNK_KEYS per tile) only the
    # device-grid entry points build
    chunked = ft and not wl.causal and wl.max_len >= vlp.VLP_FIRST_TOKEN_CHUNK_MIN
    with torch.cuda.stream(stream):
        if schedule == "persistent" or chunked:
            lib = vlp._lib.load()
            gbm = vlp.VLP_FIRST_TOKEN_CHUNK_KEYS if chunked else bm
            cap = vlp.grid_capacity(t if chunked else (b if ft else rows_q), b, gbm)
            g_bo, g_gm, g_to = (torch.empty(n, dtype=torch.int32, device=dev) for n in (b + 1, cap, cap))
            grid_cu = cu_dev if ft else cu_q_dev
            nw = 0 if schedule == "persistent" else None
            call_ms = timed(lambda: vlp.varlen_attn_fwd(q, k, v, cu_q_dev, cu_dev, wl.max_len, wl.scale, wl.causal,
                                                        ft, out=out, lse=lse, workspace=ws, num_workers=nw))
            grid_build_ms = timed(lambda: vlp._lib.check(lib.vlp_build_ragged_grid_device(
                grid_cu.data_ptr(), b, gbm, g_bo.data_ptr(), g_gm.data_ptr(), g_to.data_ptr(), cap,
                stream.cuda_stream), "grid build"))
            kernel_ms = call_ms - grid_build_ms
        else:
            kernel_ms = timed(lambda: vlp.varlen_attn_fwd(q, k, v, cu_q_dev, cu_dev, wl.max_len, wl.scale, wl.causal,
                                                          ft, out=out, lse=lse, grid=grid))
    torch.cuda.synchronize()

    value = flops / (ms_per_step * 1e-3) / 1e12
    elt = q.element_size()
    # first-token mode reads the visible keys only: one per sequence when causal
    nbytes = compulsory_bytes(rows_q, b if (ft and wl.causal) else t, h, d, elt)
    if ft:
        # one query per sequence streams all of K and V: bandwidth-bound
        roof = {"bound": "hbm", "achieved": round(nbytes / (kernel_ms * 1e-3) / 1e9, 3), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(flops / (kernel_ms * 1e-3) / 1e12, 3),
                "peak": PEAK_TFLOPS[wl.dtype], "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    if ft:
        src_hash = kernel_source_hash(KERNEL_SOURCES_FT)
        traffic = traffic_from_profile(args.workload, src_hash, kernel="attn_first_token")
    else:
        src_hash = kernel_source_hash(KERNEL_SOURCES_F32 if wl.dtype == "fp32" else KERNEL_SOURCES)
        traffic = traffic_from_profile(args.workload, src_hash)
    log(f"[bench] step {ms_per_step:.3f} ms  kernel {kernel_ms:.3f} ms  {achieved:.1f} TFLOP/s kernel-only")
    peaks = None if args.no_peaks else measured_peaks(dev, wl.dtype)
    if peaks is not None:
        if ft:
            peaks["frac_copy"] = round(roof["achieved"] / peaks["copy_gbs"], 4)
        else:
            peaks["frac_mfma"] = round(achieved / peaks["mfma_tflops"], 4)
    trace = trace_of_bench(args.workload + ("_first_token" if ft else ""), vlp.build_info(),
                           kernel="attn_first_token" if ft else "attn_fwd")
    if trace is not None and not ft:
        # the same roofline from the profiled run of this command: per-launch
        # algorithmic flops over the trace's average kernel duration
        t_us = trace["timed_loop_avg_us"]
        roof["trace"] = {"source": trace["path"], "kernel_avg_us": t_us,
                         "achieved": round(flops / (t_us * 1e-6) / 1e12, 3),
                         "frac": round(flops / (t_us * 1e-6) / 1e12 / roof["peak"], 4),
                         "profiled_run": {"kernel_ms": trace["bench_kernel_ms"],
                                          "ms_per_step": trace["bench_ms_per_step"]}}

    padded_ms, padded_backend = (None, "skipped")
    envelope_ms = None
    if not args.no_padded:
        log("[bench] padded SDPA comparator")
        padded_ms, padded_backend = padded_comparator(wl, q, k, v, reps=3, first_token=ft)
        log("[bench] own kernel over the padded envelope")
        envelope_ms = envelope_own_comparator(wl, dev, reps=3, first_token=ft)
    torch.cuda.synchronize()
    varlen_ms = varlen_diff = None
    if args.torch_varlen:
        if ft or wl.lengths_q is not None or wl.dtype not in ("bf16", "fp16"):
            log("[bench] --torch-varlen applies to 16-bit self-attention without first-token mode; skipped")
        else:
            log("[bench] torch varlen flash-attention comparator")
            varlen_ms, varlen_diff = torch_varlen_comparator(wl, q, k, v, cu_dev, out, reps=3)

    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        cpu = cpu_oracle_baseline(wl, args.cpu_budget, first_token=ft)

    lmax = wl.max_len
    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; no dataset)",
        "config": {
            "workload": wl.name,
            "description": {
                "zipf": "64 sequences, Zipf (s=1) lengths over 65,536 tokens, 16 heads x 128, causal, bf16",
                "skewed": "255 x U[64,256] + one 32,768-token sequence, 32 heads x 128, causal, bf16",
                "encoder": "128 sequences, gamma(2,75) lengths clipped to [8,384], 12 heads x 64, bf16",
                "graph": "512 sequences, lognormal(ln 80, 0.6) lengths clipped to [1,256], 8 heads x 64, fp32",
                "tiny": "8 sequences, U[1,64] lengths, 2 heads x 16, fp32",
                "cross": "cross-attention: the zipf key lengths (65,536 keys over 64 sequences), ceil(len/4) "
                         "queries each (16,408), 16 heads x 128, non-causal, bf16",
            }[wl.name] + ("; run without the causal mask" if args.no_causal else ""),
            "num_seqs": b,
            "total_tokens": t,
            "total_queries": rows_q,
            "max_seqlen": lmax,
            "heads": h,
            "head_dim": d,
            "causal": wl.causal,
            "query_is_first_token": ft,
            # first-token mode has one query per sequence and no query tiles
            "block_m": None if ft else bm,
            "schedule": schedule,
        },
        "roofline": {**roof, "traffic": traffic},
        "measured_peak": peaks,
        "attainable": attainable(flops, nbytes, achieved, PEAK_TFLOPS[wl.dtype], peaks),
        "cpu_baseline": None if cpu is None else {k2: cpu[k2] for k2 in ("value", "unit", "cores", "kind", "sample")},
        "speedup_vs_padded": None if padded_ms is None else round(padded_ms / ms_per_step, 3),
        "padded_ms": None if padded_ms is None else round(padded_ms, 3),
        "padded_backend": padded_backend,
        "envelope_own_ms": None if envelope_ms is None else round(envelope_ms, 3),
        "speedup_vs_envelope_own": None if envelope_ms is None else round(envelope_ms / kernel_ms, 3),
        **({} if varlen_ms is None else {"torch_varlen_flash_ms": round(varlen_ms, 4),
                                         "speedup_vs_torch_varlen": round(varlen_ms / kernel_ms, 3),
                                         "torch_varlen_max_abs_diff": varlen_diff}),
        "kernel_ms": round(kernel_ms, 4),
        "kernel_timing": ("device-grid calls minus grid builds timed alone (grid build "
                          f"{grid_build_ms:.4f} ms)" if grid_build_ms is not None else "cached-grid launches"),
        "kernel_tflops": round(achieved, 3),
        "kernel_source_hash": src_hash,
        "library_build": vlp.build_info(),
        "algorithmic_gflop": round(flops / 1e9, 3),
        "compulsory_gb": round(nbytes / 1e9, 4),
        "rho_seq": round(t / (b * lmax), 4),
        "work_ratio": round(float(np.sum(wl.query_lengths().astype(np.float64) * wl.lengths))
                            / (b * int(wl.query_lengths().max()) * lmax), 5),
        "pack_sequences_host_us": round(pack_us, 1),
        "cpu_baseline_detail": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
