"""GPU tier: the largest inputs -- byte offsets past 4 GiB.

One packed batch of 2^25 tokens (8,192 sequences of 4,096; two heads of 64,
bf16, causal) makes every q, k, v, out, dout, dq, dk, dv tensor 8 GiB, so
the rows of the second half of the batch sit more than 2^32 bytes into
their buffers and the lse / row-statistic arrays hold 2^26 entries: every address the
kernels form (row index times token stride, buffer-descriptor bases, lse
offsets) is exercised beyond 32 bits.  The values are drawn on the device by
seeded generators; the oracle computes whole sampled sequences (the first,
the two on either side of the 4 GiB mark, the last) from host copies of their
rows.  Tolerances as in the forward and gradient parity tests: out 2e-2 and
lse 1e-3 absolute; gradients per row 2e-2 + 2^-7 * max |oracle| over the
row (the derivation is in the gradient tests' module docstring).
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
SEQ, NSEQ, H, D = 4096, 8192, 2, 64
T = SEQ * NSEQ  # 2^25 tokens x 2 heads x 64: 8 GiB per bf16 tensor
SAMPLED = (0, NSEQ // 2 - 1, NSEQ // 2, NSEQ - 1)  # the first, those at the 4 GiB mark, the last


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def batch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vlp.load_library()
    vlp.check_library_current()
    free, _ = torch.cuda.mem_get_info()
    if free < 96 << 30:
        pytest.skip(f"needs 96 GiB of free device memory, {free >> 30} GiB free")
    _say(f"[large] drawing {T} tokens x {H} x {D} bf16 on the device (8 GiB per tensor)")
    q, k, v, dout = (workloads.random_rows_device(T, H, D, "bf16", 5000 + i, DEV) for i in range(4))
    cu = torch.arange(0, T + 1, SEQ, dtype=torch.int32)
    yield q, k, v, dout, cu
    del q, k, v, dout
    torch.cuda.empty_cache()


def _rows(t, i):
    return t[i * SEQ:(i + 1) * SEQ].float().cpu()


def test_forward_beyond_4gib(batch):
    q, k, v, _, cu = batch
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out, lse = vlp.varlen_attn_fwd(q, k, v, cu.to(DEV), cu.to(DEV), SEQ, scale, True)
    torch.cuda.synchronize()
    one = np.array([0, SEQ], dtype=np.int32)
    for i in SAMPLED:
        ref, ref_lse = oracle.varlen_attention(_rows(q, i), _rows(k, i), _rows(v, i), one, one, scale, True)
        got = _rows(out, i).numpy()
        got_lse = lse[:, i * SEQ:(i + 1) * SEQ].cpu().numpy()
        err, lerr = np.max(np.abs(got - ref)), np.max(np.abs(got_lse - ref_lse))
        _say(f"[large] forward, sequence {i} (byte offset {i * SEQ * H * D * 2:#x}): out {err:.3e} lse {lerr:.3e}")
        assert err <= 2e-2 and lerr <= 1e-3
    del out, lse


def test_first_token_beyond_4gib(batch):
    q, k, v, _, cu = batch
    scale = float(np.float32(1.0 / np.sqrt(D)))
    qf = q[cu[:-1].long().to(DEV)].contiguous()
    out, lse = vlp.varlen_attn_fwd(qf, k, v, None, cu.to(DEV), SEQ, scale, False, True)
    torch.cuda.synchronize()
    one = np.array([0, SEQ], dtype=np.int32)
    for i in SAMPLED:
        ref, ref_lse = oracle.varlen_attention(qf[i:i + 1].float().cpu(), _rows(k, i), _rows(v, i), None, one,
                                               scale, False, query_is_first_token=True)
        err = np.max(np.abs(out[i:i + 1].float().cpu().numpy() - ref))
        lerr = np.max(np.abs(lse[:, i:i + 1].cpu().numpy() - ref_lse))
        _say(f"[large] first token, sequence {i}: out {err:.3e} lse {lerr:.3e}")
        assert err <= 2e-2 and lerr <= 1e-3


def test_backward_beyond_4gib(batch):
    q, k, v, dout, cu = batch
    scale = float(np.float32(1.0 / np.sqrt(D)))
    cud = cu.to(DEV)
    out, lse = vlp.varlen_attn_fwd(q, k, v, cud, cud, SEQ, scale, True)
    dq, dk, dv = vlp.varlen_attn_bwd(q, k, v, out, dout, lse, cud, cud, SEQ, scale, True)
    torch.cuda.synchronize()
    one = np.array([0, SEQ], dtype=np.int32)
    for i in SAMPLED:
        refs = oracle.varlen_attention_bwd(_rows(q, i), _rows(k, i), _rows(v, i), _rows(dout, i), one, one, scale,
                                           True)
        excess = []
        for got, ref in zip((dq, dk, dv), refs):
            g = _rows(got, i).numpy().astype(np.float64)
            err = np.max(np.abs(g - ref), axis=-1)
            excess.append(float(np.max(err - (2e-2 + 2.0 ** -7 * np.max(np.abs(ref), axis=-1)))))
        _say(f"[large] backward, sequence {i}: excess over tolerance dq {excess[0]:.3e} dk {excess[1]:.3e} "
             f"dv {excess[2]:.3e}")
        assert max(excess) <= 0.0
    del out, lse, dq, dk, dv


def test_ragged_matmul_beyond_4gib():
    """x [2^26, 64] (8 GiB) times one [64, 64] weight per sequence (16,384
    sequences of 4,096 rows); sampled sequences on both sides of the 4 GiB
    byte offset and the last one against the oracle, with the matmul tests'
    per-element bound rel * |y| + 2^-14 * (|x| |W|^T) (rel = 2^-8, bf16)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vlp.load_library()
    vlp.check_library_current()
    free, _ = torch.cuda.mem_get_info()
    if free < 24 << 30:
        pytest.skip(f"needs 24 GiB of free device memory, {free >> 30} GiB free")
    rows, nseq, kdim = 1 << 26, 1 << 14, 64
    seq = rows // nseq
    x = workloads.random_rows_device(rows, 1, kdim, "bf16", 5100, DEV).view(rows, kdim)
    w = (workloads.random_rows_device(nseq, kdim, kdim, "bf16", 5101, DEV).float() / 8).to(torch.bfloat16)
    cu = torch.arange(0, rows + 1, seq, dtype=torch.int32)
    y = vlp.ragged_matmul(x, w, cu.to(DEV))
    torch.cuda.synchronize()
    one = np.array([0, seq], dtype=np.int32)
    assert (nseq // 2) * seq * kdim * 2 == 1 << 32  # the sampled sequences straddle the 4 GiB mark
    for i in (0, nseq // 2 - 1, nseq // 2, nseq - 1):
        xs = x[i * seq:(i + 1) * seq].float().cpu()
        ws = w[i:i + 1].float().cpu()
        ref = oracle.ragged_matmul(xs, ws, one)
        mag = oracle.ragged_matmul(xs.abs(), ws.abs(), one)
        got = y[i * seq:(i + 1) * seq].float().cpu().numpy()
        excess = np.max(np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * mag))
        _say(f"[large] ragged matmul, sequence {i} (byte offset {i * seq * kdim * 2:#x}): max excess {excess:.3e}")
        assert excess <= 0.0
    del x, w, y
    torch.cuda.empty_cache()
