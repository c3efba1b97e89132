"""vlp_varlen_attn_fwd_noalloc: the forward entry point that allocates
nothing (its tile metadata lives in a library-owned device array).

Called through the C ABI and compared with vlp_varlen_attn_fwd (same kernels:
the results must be bit-identical) on two calls in a row, the second with a
smaller batch, for every dtype and in first-token mode.  The size limit is
checked on the host before any HIP call (CPU tier).
"""

import ctypes
import os
import sys

import numpy as np
import pytest
import torch

import variable_length_packed_pack_amd as vlp
from variable_length_packed_pack_amd import _lib
import workloads

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libvlp.so not built")

_CODES = {"fp32": _lib.VLP_FP32, "fp16": _lib.VLP_FP16, "bf16": _lib.VLP_BF16}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(q, k, v, cu_q, cu_k, b, max_seqlen, scale, causal, ft, out, lse):
    lib = _lib.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.vlp_varlen_attn_fwd_noalloc(_CODES[{torch.float32: "fp32", torch.float16: "fp16",
                                                   torch.bfloat16: "bf16"}[q.dtype]],
                                           _p(q), _p(k), _p(v), _p(cu_q), _p(cu_k), b, q.shape[0], k.shape[0],
                                           q.shape[1], q.shape[2], 0, 0, 0, max_seqlen, scale, int(causal),
                                           int(ft), _p(out), _p(lse), stream)


def test_noalloc_refuses_metadata_beyond_its_scratch_on_the_host():
    """Refused before any HIP call (no GPU needed): with block_m 256 rows and
    a million one-token sequences the grid metadata exceeds the scratch."""
    lib = _lib.load()
    fake = ctypes.c_void_p(1 << 20)  # aligned dummy pointers; never dereferenced
    b = 1 << 20
    st = lib.vlp_varlen_attn_fwd_noalloc(_lib.VLP_BF16, fake, fake, fake, fake, fake, b, b, b, 1, 128,
                                         0, 0, 0, 0, 0.125, 1, 0, fake, None, None)
    assert st == _lib.VLP_ERR_CAPACITY
    # the other checks of vlp_varlen_attn_fwd come first
    st = lib.vlp_varlen_attn_fwd_noalloc(_lib.VLP_BF16, None, fake, fake, fake, fake, 4, 16, 16, 1, 128,
                                         0, 0, 0, 0, 0.125, 1, 0, fake, None, None)
    assert st == _lib.VLP_ERR_NULL
    st = lib.vlp_varlen_attn_fwd_noalloc(_lib.VLP_BF16, fake, fake, fake, fake, fake, 4, 16, 16, 1, 128,
                                         0, 0, 0, 0, float("nan"), 1, 0, fake, None, None)
    assert st == _lib.VLP_ERR_INVALID


def _case(lengths, heads, head_dim, dtype, causal, ft, seed):
    wl = workloads.custom_workload(lengths, heads, head_dim, dtype, causal, seed=seed)
    dev = "cuda"
    cu_h = wl.cu_seqlens_host()
    cu = torch.from_numpy(cu_h).to(dev)
    q = wl.q.to(dev)
    if ft:
        q = q[torch.from_numpy(cu_h[:-1]).long().to(dev)].contiguous()
    k, v = wl.k.to(dev), wl.v.to(dev)
    b = wl.num_seqs
    # reference: the entry point with a caller-supplied workspace
    ref_out, ref_lse = vlp.varlen_attn_fwd(q, k, v, None if ft else cu, cu, wl.max_len, wl.scale, causal, ft)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((heads, q.shape[0]), float("nan"), dtype=torch.float32, device=dev)
    st = _noalloc(q, k, v, None if ft else cu, cu, b, wl.max_len, wl.scale, causal, ft, out, lse)
    assert st == _lib.VLP_OK, _lib.load().vlp_status_string(st)
    torch.cuda.synchronize()
    same = torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    _say(f"[noalloc] {dtype} D={head_dim} H={heads} B={b} T={wl.total_tokens} causal={causal} first_token={ft}: "
         f"bit-identical={same}")
    assert same


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,head_dim,causal,ft", [
    ("bf16", 128, True, False), ("fp16", 64, False, False), ("fp32", 64, False, False),
    ("bf16", 128, False, True), ("fp32", 16, True, False),
])
def test_noalloc_matches_workspace_entry_point_twice(dtype, head_dim, causal, ft):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vlp.load_library()
    vlp.check_library_current()
    rng = np.random.default_rng(5 + head_dim)
    big = [int(x) for x in rng.integers(1, 1500, size=40)] + [3000]
    small = [int(x) for x in rng.integers(1, 200, size=7)]
    _case(big, 4, head_dim, dtype, causal, ft, seed=71)
    _case(small, 2, head_dim, dtype, causal, ft, seed=72)  # second call, smaller batch: same scratch
