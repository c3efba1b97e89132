"""GPU tier: document ids -> cu_seqlens on the device, and attention under the
sample-id mask of one packed sequence through it.

The run boundaries are integers: bit-exact against ``oracle.cu_seqlens_from_ids``.
The attention is checked against ``oracle.document_masked_attention``, the
dense [T, T] definition of the mask, at the forward's tolerances (out 1e-4
fp32 / 2e-2 bf16, lse 1e-3); the gradients against the oracle's gradients on
the runs at the backward's row-wise tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
import variable_length_packed_pack_amd as vlp

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vlp.load_library()
    vlp.check_library_current()
    yield
    torch.cuda.synchronize()


def _ids(rng, runs, max_len):
    vals = rng.integers(0, 1 << 20, size=runs)
    vals[1:][vals[1:] == vals[:-1]] += 1  # neighbouring runs differ
    return np.repeat(vals, rng.integers(1, max_len + 1, size=runs)).astype(np.int32)


@pytest.mark.parametrize("seed,runs,max_len,cap", [(0, 1, 1, 1), (1, 7, 5, 7), (2, 300, 40, 512),
                                                   (3, 2000, 200, 4096), (4, 50, 20000, 64)])
def test_boundaries_bit_exact(seed, runs, max_len, cap):
    rng = np.random.default_rng(seed)
    ids = _ids(rng, runs, max_len)
    cu, n = vlp.cu_seqlens_from_ids(torch.from_numpy(ids).to(DEV), cap)
    torch.cuda.synchronize()
    ref, nref = oracle.cu_seqlens_from_ids(ids, cap)
    assert int(n.item()) == nref == runs
    assert np.array_equal(cu.cpu().numpy(), ref)


def test_over_capacity_reports_the_count_and_empty_input():
    ids = torch.arange(100, dtype=torch.int32, device=DEV)
    cu, n = vlp.cu_seqlens_from_ids(ids, 10)
    torch.cuda.synchronize()
    assert int(n.item()) == 100
    assert cu.cpu().tolist() == list(range(10)) + [100]
    cu, n = vlp.cu_seqlens_from_ids(torch.empty(0, dtype=torch.int32, device=DEV), 3)
    torch.cuda.synchronize()
    assert int(n.item()) == 0 and cu.cpu().tolist() == [0, 0, 0, 0]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_sample_id_masked_attention(dtype, causal):
    """One packed sequence of ~2,000 tokens in 23 documents: device ids ->
    cu_seqlens (capacity 64, zero-length tail) -> varlen forward, against the
    dense sample-id mask; then the gradients through the same boundaries."""
    rng = np.random.default_rng(5 + causal)
    ids = _ids(rng, 23, 170)
    t, h, d = len(ids), 2, 64
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16}[dtype]
    q, k, v, do = (torch.from_numpy(rng.standard_normal((t, h, d), dtype=np.float32)).to(tdt) for _ in range(4))
    cu, n = vlp.cu_seqlens_from_ids(torch.from_numpy(ids).to(DEV), 64)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    out, lse = vlp.varlen_attn_fwd(qd, kd, vd, cu, cu, 0, 0.125, causal)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.document_masked_attention(q, k, v, ids, 0.125, causal)
    tol = 1e-4 if dtype == "fp32" else 2e-2
    assert np.max(np.abs(out.float().cpu().numpy() - ref)) <= tol
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 1e-3
    dq, dk, dv = vlp.varlen_attn_bwd(qd, kd, vd, out, dod, lse, cu, cu, 0, 0.125, causal)
    torch.cuda.synchronize()
    cu_h = cu.cpu().numpy()
    refs = oracle.varlen_attention_bwd(q, k, v, do, cu_h, cu_h, 0.125, causal)
    atol, rtol = (1e-4, 2.0 ** -14) if dtype == "fp32" else (2e-2, 2.0 ** -7)
    for got, r in zip((dq, dk, dv), refs):
        err = np.max(np.abs(got.float().cpu().numpy() - r), axis=-1)
        assert np.all(err <= atol + rtol * np.max(np.abs(r), axis=-1))
