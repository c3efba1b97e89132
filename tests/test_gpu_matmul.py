"""GPU tier: ragged matrix multiplication through the C ABI against the oracle.

Tolerance (derived; the pages give none): an output element passes if
|gpu - oracle| <= rel * |oracle| + 2^-14 * (|x| |W|^T + |b|) for that element,
with rel = 2^-8 for bf16 and 2^-11 for fp16: the result is rounded once to
the element type (at most half an ulp), and the fp32 accumulation of the
K products in another order than the oracle's fp64 sum moves it by far less
than 2^-14 of the sum of the products' magnitudes.
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
REL = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


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


def _check(x, w, b, cu, dtype, shared_w, shared_b, label):
    tdt = workloads.DTYPES[dtype]
    xd, wd = x.to(tdt).to(DEV), w.to(tdt).to(DEV)
    bd = None if b is None else b.to(tdt).to(DEV)
    rows, n = x.shape[0], w.shape[-2]
    y = torch.full((rows, n), float("nan"), dtype=tdt, device=DEV)
    vlp.ragged_matmul(xd, wd, cu.to(DEV), bd, out=y)
    torch.cuda.synchronize()
    xr, wr = xd.cpu(), wd.cpu()
    br = None if bd is None else bd.cpu()
    ref = oracle.ragged_matmul(xr, wr, cu.numpy(), br, shared_weight=shared_w, shared_bias=shared_b)
    mag = oracle.ragged_matmul(xr.float().abs(), wr.float().abs(), cu.numpy(),
                               None if br is None else br.float().abs(), shared_weight=shared_w,
                               shared_bias=shared_b)
    t = int(cu[-1])
    got = y[:t].float().cpu().numpy()
    excess = np.abs(got - ref[:t]) - (REL[dtype] * np.abs(ref[:t]) + 2.0 ** -14 * mag[:t])
    _say(f"[matmul] {label} {dtype} rows={t} K={x.shape[1]} N={n}: max excess {np.max(excess, initial=-1):.3e}")
    assert np.max(excess, initial=-1.0) <= 0.0
    assert torch.isnan(y[t:].float()).all().item()  # capacity rows are never written
    return y


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("k,n", [(64, 4), (128, 100), (512, 128), (256, 260)])
def test_per_sequence_weights_edge_lengths(dtype, k, n):
    lengths = [1, 127, 128, 129, 0, 300, 5]
    cu = _cu(lengths)
    rows = int(cu[-1]) + 9
    x = _rand((rows, k), 1 + k)
    x[int(cu[-1]):] = float("nan")  # capacity rows: must not leak into anything
    w = _rand((len(lengths), n, k), 2 + n) / np.sqrt(k)
    b = _rand((len(lengths), n), 3)
    _check(x, w, b, cu, dtype, False, False, "per-sequence weights + bias")
    _check(x, w, None, cu, dtype, False, False, "per-sequence weights")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_shared_weight_projection(dtype):
    """The packed linear layer: one [N, K] weight and [N] bias for all rows."""
    lengths = workloads.draw_lengths(3)  # encoder batch: 128 gamma lengths
    cu = _cu(lengths)
    x = _rand((int(cu[-1]), 768), 4)
    w = _rand((3 * 768, 768), 5) / np.sqrt(768)
    b = _rand((3 * 768,), 6)
    y = _check(x, w, b, cu, dtype, True, True, "shared projection 768 -> 2304")
    # the packed result equals one plain product of all rows, bit for bit on
    # the GPU, whatever the split into sequences
    y2 = vlp.ragged_matmul(x.to(workloads.DTYPES[dtype]).to(DEV), w.to(workloads.DTYPES[dtype]).to(DEV),
                           _cu([int(cu[-1])]).to(DEV), b.to(workloads.DTYPES[dtype]).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


def test_zipf_batch_per_sequence_weights():
    """The Zipf token split (64 sequences over 65,536 tokens), 512 -> 512 with
    one weight per sequence, every row checked."""
    lengths = workloads.draw_lengths(4)
    cu = _cu(lengths)
    x = _rand((int(cu[-1]), 512), 7)
    w = _rand((len(lengths), 512, 512), 8) / np.sqrt(512)
    _check(x, w, None, cu, "bf16", False, False, "zipf split, per-sequence 512 -> 512")


def test_sequence_independence_bitwise():
    lengths = [200, 17, 129]
    cu = _cu(lengths)
    x = _rand((int(cu[-1]), 256), 9).to(torch.bfloat16).to(DEV)
    w = (_rand((3, 128, 256), 10) / 16).to(torch.bfloat16).to(DEV)
    y1 = vlp.ragged_matmul(x, w, cu.to(DEV))
    x2, w2 = x.clone(), w.clone()
    x2[200:217] *= -4
    w2[1] += 1
    y2 = vlp.ragged_matmul(x2, w2, cu.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y1[:200], y2[:200]) and torch.equal(y1[217:], y2[217:])
    assert not torch.equal(y1[200:217], y2[200:217])
