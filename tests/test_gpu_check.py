"""GPU tier: the VLP_CHECK=1 debug validation of device cu_seqlens contents.

With VLP_CHECK=1 the entry points check cu_seqlens on the device before any
other kernel reads it and refuse broken contents with VLP_ERR_INVALID; valid
contents give the same results, to the bit, as the unchecked path.  Every
tensor passed is a view of the first 20 rows of a 64-row allocation (lse:
of a 64-row allocation per head), and every broken case stays inside 64
rows, so nothing could be read or written out of bounds even if the check
were skipped.
"""

import sys

import pytest
import torch

import variable_length_packed_pack_amd as vlp
from variable_length_packed_pack_amd import _lib
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"
H, D, ROWS, ALLOC = 2, 64, 20, 64


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


@pytest.fixture
def checks(monkeypatch):
    monkeypatch.setenv("VLP_CHECK", "1")
    yield monkeypatch


def _view(t):
    return t.to(DEV)[:ROWS]


def _inputs(seed=41):
    q, k, v = workloads.random_qkv(ALLOC, H, D, "bf16", seed)
    dout = workloads.random_dout(ALLOC, H, D, "bf16", seed + 1)
    return tuple(_view(t) for t in (q, k, v, dout))


def _outs():
    """out-like views and an lse view [H, ROWS] whose rows stay inside the
    allocation for any row index below ALLOC."""
    big = torch.empty(ALLOC, H, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(H * ALLOC, dtype=torch.float32, device=DEV)[:H * ROWS].view(H, ROWS)
    return big[:ROWS], lse


def _grads():
    return tuple(torch.empty(ALLOC, H, D, dtype=torch.bfloat16, device=DEV)[:ROWS] for _ in range(3))


def _cu(vals):
    return torch.tensor(vals, dtype=torch.int32, device=DEV)


def _status(fn):
    try:
        fn()
        torch.cuda.synchronize()
        return _lib.VLP_OK
    except _lib.VlpError as e:
        return e.status


BROKEN = {
    "cu[0] != 0": [3, 10, 20],
    "decreasing": [0, 12, 8, 20],
    "total beyond the rows": [0, 10, 30],
}


def _good(case):
    return _cu([0, ROWS] + [ROWS] * (len(BROKEN[case]) - 2))


def test_check_is_active_and_valid_contents_pass(checks):
    q, k, v, _ = _inputs()
    out, lse = _outs()
    bad = _cu([1, 10, 20])
    assert _status(lambda: vlp.varlen_attn_fwd(q, k, v, bad, bad, out=out, lse=lse)) == _lib.VLP_ERR_INVALID
    good = _cu([0, 7, 7, 20])
    out1, lse1 = vlp.varlen_attn_fwd(q, k, v, good, good, causal=True)
    checks.delenv("VLP_CHECK")
    out2, lse2 = vlp.varlen_attn_fwd(q, k, v, good, good, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


@pytest.mark.parametrize("case", sorted(BROKEN))
def test_forward_refuses_broken_cu_seqlens(checks, case):
    q, k, v, _ = _inputs()
    out, lse = _outs()
    cu, good = _cu(BROKEN[case]), _good(case)
    _say(f"[check] forward, {case}: cu_seqlens {BROKEN[case]}")
    for cq, ck in ((cu, cu), (cu, good), (good, cu)):
        for nw in (None, 0):
            assert _status(lambda: vlp.varlen_attn_fwd(q, k, v, cq, ck, out=out, lse=lse, num_workers=nw)) == \
                _lib.VLP_ERR_INVALID


def test_first_token_refuses_an_empty_sequence(checks):
    q, k, v, _ = _inputs()
    big, lse_all = torch.empty(ALLOC, H, D, dtype=torch.bfloat16, device=DEV), torch.empty(
        H * ALLOC, dtype=torch.float32, device=DEV)
    q2, out2, lse2 = q[:2].contiguous(), big[:2], lse_all[:2 * H].view(H, 2)
    status = _status(lambda: vlp.varlen_attn_fwd(q2, k, v, None, _cu([0, 0, 20]), out=out2, lse=lse2,
                                                 query_is_first_token=True))
    assert status == _lib.VLP_ERR_INVALID
    assert _status(lambda: vlp.varlen_attn_fwd(q2, k, v, None, _cu([0, 5, 20]), out=out2, lse=lse2,
                                               query_is_first_token=True)) == _lib.VLP_OK


@pytest.mark.parametrize("case", sorted(BROKEN))
def test_backward_and_matmul_refuse_broken_cu_seqlens(checks, case):
    q, k, v, dout = _inputs()
    cu, good = _cu(BROKEN[case]), _good(case)
    out, lse = _outs()
    vlp.varlen_attn_fwd(q, k, v, good, good, out=out, lse=lse)
    dq, dk, dv = _grads()
    for cq, ck in ((cu, good), (good, cu)):
        assert _status(lambda: vlp.varlen_attn_bwd(q, k, v, out, dout, lse, cq, ck, dq=dq, dk=dk, dv=dv)) == \
            _lib.VLP_ERR_INVALID
    assert _status(lambda: vlp.varlen_attn_bwd(q, k, v, out, dout, lse, good, good, dq=dq, dk=dk, dv=dv)) == \
        _lib.VLP_OK
    g = torch.Generator().manual_seed(43)
    x = torch.randn(ALLOC, 64, generator=g).to(torch.bfloat16).to(DEV)[:ROWS]
    w = (torch.randn(64, 64, generator=g) / 8).to(torch.bfloat16).to(DEV)
    y = torch.empty(ALLOC, 64, dtype=torch.bfloat16, device=DEV)[:ROWS]
    assert _status(lambda: vlp.ragged_matmul(x, w, cu, out=y)) == _lib.VLP_ERR_INVALID
    assert _status(lambda: vlp.ragged_matmul(x, w, good, out=y)) == _lib.VLP_OK
