"""The inline-metadata forward (vlp_varlen_attn_fwd_inline): host boundaries
and host-built tile metadata carried in the kernel's argument block.  Same
kernels and tile order as the device-grid forward, so the results must be
bit-identical to it, and within tolerance of the oracle.

SKIPPED, and the entry point is not in the library.  These tests passed on
the GPU, but the Zipf forward step run back to back through this entry point
(about 25 launches of a 1.3 ms kernel in flight, each with a 4 KB argument
block that its late workgroups read) left the GPU faulted, and no mistake in
the library's code was found that would cause it: the single calls above give
the device-grid forward's bits at full size.  Until a cause is shown, the
entry point stays out and these tests do not run."""
import numpy as np
import pytest
import torch

import variable_length_packed_pack_amd as vlp
import workloads
from variable_length_packed_pack_amd import _lib
from oracle import varlen_oracle as oracle

pytestmark = [pytest.mark.gpu,
              pytest.mark.skip(reason="inline-metadata entry point withdrawn: a back-to-back run faulted the GPU "
                                      "with no cause found in the library")]

TOL_OUT = {"fp32": 1e-4, "fp16": 2e-2, "bf16": 2e-2}
TOL_LSE = 1e-3
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _cu(lengths):
    return torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))


@pytest.mark.parametrize("dtype,head_dim", [("bf16", 128), ("fp16", 128), ("bf16", 64), ("fp16", 32),
                                            ("bf16", 16), ("fp32", 64), ("fp32", 128)])
@pytest.mark.parametrize("cross", [False, True])
def test_inline_matches_device_grid_and_oracle(dtype, head_dim, cross):
    """Every kernel family (two-group at 16-bit head dim 128, four-wave, fp32),
    self- and cross-attention (Lq != Lk in both directions), causal and not,
    a negative scale: bit-identical to varlen_attn_fwd, and the oracle."""
    lk = [300, 1, 129, 70, 513, 2, 64]
    lq = [100, 7, 700, 1, 3, 2, 64] if cross else lk
    h = 2
    rng = np.random.default_rng(7 + head_dim + (1000 if cross else 0))
    tdt = workloads.DTYPES[dtype]
    q = torch.from_numpy(rng.standard_normal((sum(lq), h, head_dim), dtype=np.float32)).to(tdt)
    k = torch.from_numpy(rng.standard_normal((sum(lk), h, head_dim), dtype=np.float32)).to(tdt)
    v = torch.from_numpy(rng.standard_normal((sum(lk), h, head_dim), dtype=np.float32)).to(tdt)
    cq, ck = _cu(lq), _cu(lk)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    base = float(np.float32(1.0 / np.sqrt(head_dim)))
    for causal in (False, True):
        for scale in (base, -base):
            _say(f"[inline] {dtype} D={head_dim} cross={cross} causal={causal} scale={scale:+.4f}")
            out, lse = vlp.varlen_attn_fwd(qd, kd, vd, cq.to(DEV), ck.to(DEV), 0, scale, causal)
            out2, lse2 = vlp.varlen_attn_fwd_inline(qd, kd, vd, cq, ck, 0, scale, causal)
            torch.cuda.synchronize()
            assert torch.equal(out, out2) and torch.equal(lse, lse2)
            ref, ref_lse = oracle.varlen_attention(q, k, v, cq.numpy(), ck.numpy(), scale, causal)
            got_lse = lse2.cpu().numpy()
            keyless = np.isneginf(ref_lse)
            assert np.array_equal(np.isneginf(got_lse), keyless)
            assert np.max(np.abs(got_lse[~keyless] - ref_lse[~keyless])) <= TOL_LSE
            assert np.max(np.abs(out2.float().cpu().numpy() - ref)) <= TOL_OUT[dtype]


@pytest.mark.parametrize("name", ["encoder", "zipf"])
def test_inline_on_full_size_batches(name):
    """The encoder batch (128 sequences, bf16 12x64) and the Zipf batch (64
    sequences, bf16 16x128, causal) fit the argument block; both give the
    device-grid forward's bits."""
    wl = workloads.make_workload(workloads.WORKLOAD_NAMES[name])
    cu = torch.from_numpy(wl.cu_seqlens_host())
    q, k, v = wl.q.to(DEV), wl.k.to(DEV), wl.v.to(DEV)
    _say(f"[inline] full-size {name}: {wl.num_seqs} sequences")
    out, lse = vlp.varlen_attn_fwd(q, k, v, cu.to(DEV), cu.to(DEV), wl.max_len, wl.scale, wl.causal)
    out2, lse2 = vlp.varlen_attn_fwd_inline(q, k, v, cu, cu, wl.max_len, wl.scale, wl.causal)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_inline_capacity_and_argument_errors():
    """Metadata beyond VLP_INLINE_META_INTS is refused before any launch (the
    caller then uses the device-grid forward); device or non-int32 boundaries
    are refused by the binding; bad host boundaries by the library."""
    lengths = [300] * 400  # 2 * 401 boundary ints + 2 * 800 tiles > 983
    h, d = 1, 128
    n = sum(lengths)
    q = torch.zeros(n, h, d, dtype=torch.bfloat16, device=DEV)
    cu = _cu(lengths)
    with pytest.raises(_lib.VlpError) as e:
        vlp.varlen_attn_fwd_inline(q, q, q, cu, cu, 0, 0.1, True)
    assert e.value.status == _lib.VLP_ERR_CAPACITY
    with pytest.raises(ValueError):
        vlp.varlen_attn_fwd_inline(q, q, q, cu.to(DEV), cu.to(DEV), 0, 0.1, True)
    with pytest.raises(TypeError):
        vlp.varlen_attn_fwd_inline(q, q, q, cu.long(), cu.long(), 0, 0.1, True)
    bad = cu.clone()
    bad[-1] = n + 1  # beyond the rows of q
    with pytest.raises(_lib.VlpError) as e:
        vlp.varlen_attn_fwd_inline(q, q, q, bad, bad, 0, 0.1, True)
    assert e.value.status == _lib.VLP_ERR_INVALID
