"""Packed variable-length attention forward for AMD Instinct MI355X (gfx950).

A thin Python layer over the C ABI of ``libvlp.so`` (``include/vlp.h``).  It
only marshals arguments: torch supplies device memory and the current stream;
every step of the computation runs in the library's C++ and HIP code.

Functions mirror the pages' calls:

* ``pack_sequences(lengths, max_seq_len) -> (flat_index, cu_seqlens)``
  ("gigl.nn.packed_attention", "Data flow of a packed forward", "Example").
* ``build_ragged_grid(cu_seqlens, block_m) -> RaggedGrid`` with grid_mapping,
  block_offsets and the longest-first tile_order ("PyCoRa", "CoRa Metadata").
* ``varlen_attn_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen, scale,
  causal, query_is_first_token, out, lse) -> (out, lse)``
  ("gigl.nn.packed_attention", packed_attention).
* ``varlen_attn_bwd(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k,
  max_seqlen, scale, causal) -> (dq, dk, dv)``, the gradients of the same
  attention ("gigl.nn.packed_attention", "Why this exists").
* ``cu_seqlens_from_ids(ids, max_seqs) -> (cu_seqlens, num_seqs)``: the runs
  of document ids in one packed sequence, on the device.
* ``ragged_matmul(x, weight, cu_seqlens, bias) -> y``: every sequence times its
  own weight matrix, or one shared weight ("PyCoRa", "Ragged Matrix
  Multiplication").
"""

from __future__ import annotations

import ctypes
import math
from typing import NamedTuple, Optional

import numpy as np
import torch

from . import _lib
from ._lib import (  # noqa: F401
    VLP_BF16,
    VLP_BWD_BLOCK_K,
    VLP_BWD_DKDV,
    VLP_BWD_DQ,
    VLP_DEVICE_SORT_MAX_SEQS,
    VLP_FIRST_TOKEN_BLOCK_M,
    VLP_FIRST_TOKEN_CHUNK_KEYS,
    VLP_FIRST_TOKEN_CHUNK_MIN,
    VLP_FP16,
    VLP_FP32,
    VLP_MATMUL_BLOCK_M,
    VlpError,
)

_DTYPE_CODES = {torch.float32: VLP_FP32, torch.float16: VLP_FP16, torch.bfloat16: VLP_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _token_stride(t: torch.Tensor, name: str) -> int:
    """Elements between consecutive tokens of a [rows, H, D] tensor whose
    heads are D apart and whose head rows are contiguous (a contiguous tensor
    or a view such as qkv.view(T, 3, H, D).unbind(1)); raises otherwise."""
    if t.dim() != 3 or t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != t.shape[2]):
        raise ValueError(f"{name}: heads must be head_dim apart and each head row contiguous")
    if t.shape[0] > 1 and t.stride(0) < t.shape[1] * t.shape[2]:
        raise ValueError(f"{name}: tokens overlap")
    return int(t.stride(0)) if t.shape[0] > 1 else int(t.shape[1] * t.shape[2])  # one row: any stride


def _stream_handle(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def library_path() -> str:
    return _lib.LIB_PATH


def load_library():
    """Load libvlp.so (raises if it is not built)."""
    return _lib.load()


def build_info() -> str:
    """The library's own record of its sources: "csrc=<hash> arch=gfx950"."""
    return _lib.load().vlp_build_info().decode()


def mfma_rate(dtype: torch.dtype, blocks: int, iters: int, sink: torch.Tensor) -> float:
    """One calibration launch on the current stream: ``blocks`` workgroups
    each running ``iters`` rounds of independent MFMA products of ``dtype``'s
    instruction.  ``sink``: float32 device tensor of at least blocks * 512
    elements (overwritten).  Returns the launch's flop count; the caller
    times the launch."""
    if sink.dtype != torch.float32 or not sink.is_cuda or not sink.is_contiguous():
        raise TypeError("sink must be a contiguous float32 device tensor")
    if sink.numel() < int(blocks) * 512:
        raise ValueError("sink needs blocks * 512 elements")
    flops = ctypes.c_double(0.0)
    _lib.check(_lib.load().vlp_mfma_rate(_DTYPE_CODES.get(dtype, -1), int(blocks), int(iters), _ptr(sink),
                                         ctypes.addressof(flops), _stream_handle(sink.device)), "mfma_rate")
    return float(flops.value)


def check_library_current() -> str:
    """Raise unless the loaded libvlp.so was built from the sources in this
    tree (its compiled-in hash equals build.source_hash()); returns the hash."""
    from .build import source_hash

    want = source_hash()
    info = build_info()
    if f"csrc={want}" not in info.split():
        raise RuntimeError(f"{_lib.LIB_PATH} is stale: it reports '{info}', the sources hash to {want}; "
                           "rebuild with `python -m variable_length_packed_pack_amd.build`")
    return want


# ---------------------------------------------------------------------------
# host metadata
# ---------------------------------------------------------------------------

def pack_sequences(lengths, max_seq_len: int):
    """lengths (host, int) -> (flat_index int64 [T], cu_seqlens int32 [B+1]), CPU tensors."""
    lib = _lib.load()
    lens = np.asarray(lengths)
    if lens.dtype != np.int32:
        wide = lens.astype(np.int64).reshape(-1)
        if wide.size and (wide.min() < -2**31 or wide.max() > 2**31 - 1):
            raise _lib.VlpError(_lib.VLP_ERR_INVALID, "pack_sequences")
        lens = wide.astype(np.int32)
    lens = np.ascontiguousarray(lens.reshape(-1))
    b = int(lens.size)
    cu = np.empty(b + 1, dtype=np.int32)
    total = ctypes.c_int64(0)
    # One call: the buffer is sized by the lengths' sum; the library validates
    # the lengths (and the sum) and fills both outputs, or reports the error.
    cap = int(lens.sum(dtype=np.int64)) if b else 0
    flat = np.empty(max(cap, 1), dtype=np.int64)
    st = lib.vlp_pack_sequences(lens.ctypes.data, b, int(max_seq_len), flat.ctypes.data, cap, cu.ctypes.data,
                                ctypes.addressof(total))
    _lib.check(st, "pack_sequences")
    return torch.from_numpy(flat if cap else flat[:0]), torch.from_numpy(cu)


def grid_capacity(total_tokens: int, num_seqs: int, block_m: int) -> int:
    return int(_lib.load().vlp_grid_capacity(int(total_tokens), int(num_seqs), int(block_m)))


class RaggedGrid(NamedTuple):
    """Tile metadata of one batch.  On the host the arrays have exactly
    ``num_blocks`` entries; built on the device they have ``grid_cap``
    entries (-1 past the active tiles) and ``num_blocks`` is None because
    it is known only on the device (block_offsets[-1])."""

    grid_mapping: torch.Tensor
    block_offsets: torch.Tensor
    tile_order: torch.Tensor
    num_blocks: Optional[int]
    block_m: int


def build_ragged_grid(cu_seqlens: torch.Tensor, block_m: int, grid_cap: Optional[int] = None) -> RaggedGrid:
    """CoRa-style metadata for ``cu_seqlens`` with ``block_m`` rows per tile.

    A CPU tensor is processed on the host; a CUDA tensor on the device (no
    host read; ``grid_cap`` defaults to G_cap(total capacity, B, block_m)
    which needs ``grid_cap`` or a host total, so it must be given).
    """
    lib = _lib.load()
    b = int(cu_seqlens.numel()) - 1
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if cu_seqlens.is_cuda:
        if grid_cap is None:
            raise ValueError("grid_cap is required for a device build (use grid_capacity)")
        dev = cu_seqlens.device
        bo = torch.empty(b + 1, dtype=torch.int32, device=dev)
        gm = torch.empty(max(grid_cap, 1), dtype=torch.int32, device=dev)
        to = torch.empty(max(grid_cap, 1), dtype=torch.int32, device=dev)
        st = lib.vlp_build_ragged_grid_device(_ptr(cu_seqlens.contiguous()), b, int(block_m), _ptr(bo), _ptr(gm),
                                              _ptr(to), int(grid_cap), _stream_handle(dev))
        _lib.check(st, "build_ragged_grid (device)")
        return RaggedGrid(gm[:grid_cap], bo, to[:grid_cap], None, int(block_m))
    cu = np.ascontiguousarray(cu_seqlens.numpy().astype(np.int32))
    bo = np.zeros(b + 1, dtype=np.int32)
    nb = ctypes.c_int64(0)
    st = lib.vlp_build_ragged_grid(cu.ctypes.data, b, int(block_m), bo.ctypes.data, None, None, 0,
                                   ctypes.addressof(nb))
    _lib.check(st, "build_ragged_grid")
    g = nb.value
    gm = np.zeros(max(g, 1), dtype=np.int32)
    to = np.zeros(max(g, 1), dtype=np.int32)
    st = lib.vlp_build_ragged_grid(cu.ctypes.data, b, int(block_m), bo.ctypes.data, gm.ctypes.data,
                                   to.ctypes.data, g, ctypes.addressof(nb))
    _lib.check(st, "build_ragged_grid")
    return RaggedGrid(torch.from_numpy(gm[:g].copy()), torch.from_numpy(bo), torch.from_numpy(to[:g].copy()),
                      g, int(block_m))


def kernel_block_m(dtype: torch.dtype, head_dim: int, causal: bool = False, query_is_first_token: bool = False,
                   num_seqs: int = 1, rows_q: int = 0, max_seqlen: int = 0) -> int:
    code = _DTYPE_CODES.get(dtype, -1)
    return int(_lib.load().vlp_kernel_block_m(code, int(head_dim), int(causal), int(query_is_first_token),
                                              int(num_seqs), int(rows_q), int(max_seqlen)))


def bwd_block_m(dtype: torch.dtype, head_dim: int, causal: bool = False) -> int:
    """Query rows per tile of the backward's dq phase (its query grid's block_m)."""
    code = _DTYPE_CODES.get(dtype, -1)
    return int(_lib.load().vlp_bwd_block_m(code, int(head_dim), int(causal)))


def workspace_size(num_seqs: int, rows_q: int, block_m: int) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().vlp_varlen_attn_workspace_size(int(num_seqs), int(rows_q), int(block_m),
                                                          ctypes.addressof(n)), "workspace_size")
    return int(n.value)


def fwd_workspace_size(dtype: torch.dtype, num_seqs: int, rows_q: int, total_k: int, heads: int, head_dim: int,
                       max_seqlen: int = 0, causal: bool = False, query_is_first_token: bool = False) -> int:
    """Bytes of workspace varlen_attn_fwd needs for these arguments (every
    form, including first-token mode over long sequences)."""
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().vlp_varlen_attn_fwd_workspace_size(
        _DTYPE_CODES.get(dtype, -1), int(num_seqs), int(rows_q), int(total_k), int(heads), int(head_dim),
        int(max_seqlen), int(bool(causal)), int(bool(query_is_first_token)), ctypes.addressof(n)),
        "fwd_workspace_size")
    return int(n.value)


# ---------------------------------------------------------------------------
# attention forward
# ---------------------------------------------------------------------------

def _check_cu(cu: torch.Tensor, name: str, device: torch.device) -> None:
    if cu.device != device:
        raise ValueError(f"{name} must be on {device} (it is on {cu.device})")
    if cu.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    if cu.dim() != 1 or cu.numel() < 2 or not cu.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 vector [num_seqs + 1]")


def check_fwd_args(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: Optional[torch.Tensor],
                   cu_seqlens_k: torch.Tensor, out: Optional[torch.Tensor], lse: Optional[torch.Tensor],
                   query_is_first_token: bool = False):
    """Validate the tensors of ``varlen_attn_fwd`` before anything is launched
    (the caller checks that q is a device tensor).  Every tensor must sit on
    q's device; cu_seqlens are contiguous int32 [num_seqs + 1] (cu_seqlens_q
    may be None in first-token mode, where it is not read); ``out`` (if
    given) has q's dtype and shape and token-major head rows; ``lse`` (if
    given) is float32 [H, rows_q] and contiguous.  Returns the token strides
    of q, k/v and out.  Raises ValueError or TypeError."""
    dev = q.device
    for name, t in (("k", k), ("v", v)):
        if t.device != dev:
            raise ValueError(f"{name} must be on {dev} (it is on {t.device})")
    if q.dtype not in _DTYPE_CODES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one of float32 / float16 / bfloat16")
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or k.shape != v.shape or q.shape[1:] != k.shape[1:]:
        raise ValueError("q [rows, H, D] and k, v [T, H, D] with matching H, D")
    _check_cu(cu_seqlens_k, "cu_seqlens_k", dev)
    if cu_seqlens_q is None:
        if not query_is_first_token:
            raise ValueError("cu_seqlens_q is required unless query_is_first_token")
    else:
        _check_cu(cu_seqlens_q, "cu_seqlens_q", dev)
        if cu_seqlens_q.numel() != cu_seqlens_k.numel():
            raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same number of entries")
    if query_is_first_token and q.shape[0] != cu_seqlens_k.numel() - 1:
        raise ValueError("first-token mode takes one query row per sequence")
    q_st, k_st, v_st = _token_stride(q, "q"), _token_stride(k, "k"), _token_stride(v, "v")
    if k_st != v_st and k.shape[0] > 1:
        raise ValueError("k and v must share one token stride")
    o_st = None
    if out is not None:
        if out.device != dev or out.dtype != q.dtype or out.shape != q.shape:
            raise ValueError("out must be a tensor of q's dtype and shape on q's device")
        o_st = _token_stride(out, "out")
    if lse is not None:
        if lse.device != dev:
            raise ValueError(f"lse must be on {dev}")
        if lse.dtype != torch.float32:
            raise TypeError("lse must be float32")
        if tuple(lse.shape) != (q.shape[1], q.shape[0]) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [H, rows_q] tensor")
    return q_st, k_st, o_st


def varlen_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    cu_seqlens_q: Optional[torch.Tensor], cu_seqlens_k: torch.Tensor,
                    max_seqlen: int = 0, scale: Optional[float] = None, causal: bool = False,
                    query_is_first_token: bool = False, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, *, return_lse: bool = True,
                    workspace: Optional[torch.Tensor] = None, grid: Optional[RaggedGrid] = None,
                    num_workers: Optional[int] = None):
    """Packed attention forward on the current stream; returns (out, lse).

    q [rows_q, H, D] (first-token mode: [num_seqs, H, D]), k/v [T_k, H, D],
    cu_seqlens int32 [B+1] on the same device.  ``grid``: cached device
    metadata from ``build_ragged_grid`` (host-built arrays moved to the
    device) to skip the device grid build.  ``num_workers``: None launches
    the static grid (one workgroup per capacity tile and head); an int
    launches the persistent schedule with that many workgroups at most (0 =
    as many as the device holds at once), which take the active tiles from
    work queues.
    """
    lib = _lib.load()
    if not q.is_cuda:
        raise ValueError("q, k, v and cu_seqlens must be device tensors")
    q_st, k_st, o_st = check_fwd_args(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse, query_is_first_token)
    rows_q, heads, head_dim = (int(x) for x in q.shape)
    total_k = int(k.shape[0])
    b = int(cu_seqlens_k.numel()) - 1
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    dev = q.device
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
        o_st = _token_stride(out, "out")
    if lse is None and return_lse:
        lse = torch.empty(heads, rows_q, dtype=torch.float32, device=dev)
    for name, t in (("workspace", workspace),) + (() if grid is None else (
            ("grid.grid_mapping", grid.grid_mapping), ("grid.block_offsets", grid.block_offsets),
            ("grid.tile_order", grid.tile_order))):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} must be on {dev}")
    code = _DTYPE_CODES[q.dtype]
    ft = int(bool(query_is_first_token))
    cu_q_ptr = None if (ft and cu_seqlens_q is None) else _ptr(cu_seqlens_q)
    stream = _stream_handle(dev)
    if grid is not None and num_workers is not None:
        raise ValueError("the persistent schedule builds its grid on the device: pass grid or num_workers")
    if grid is not None:
        nb = grid.num_blocks if grid.num_blocks is not None else int(grid.grid_mapping.numel())
        st = lib.vlp_varlen_attn_fwd_grid(code, _ptr(q), _ptr(k), _ptr(v), cu_q_ptr, _ptr(cu_seqlens_k), b,
                                          rows_q, total_k, heads, head_dim, q_st, k_st, o_st, int(max_seqlen),
                                          float(scale),
                                          int(bool(causal)), ft, _ptr(out), _ptr(lse), _ptr(grid.grid_mapping),
                                          _ptr(grid.block_offsets), _ptr(grid.tile_order), nb, grid.block_m,
                                          stream)
        _lib.check(st, "varlen_attn_fwd_grid")
        return out, lse
    if workspace is None:
        nbytes = fwd_workspace_size(q.dtype, b, rows_q, total_k, heads, head_dim, max_seqlen, causal, ft)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    args = (code, _ptr(q), _ptr(k), _ptr(v), cu_q_ptr, _ptr(cu_seqlens_k), b, rows_q, total_k, heads, head_dim,
            q_st, k_st, o_st, int(max_seqlen), float(scale), int(bool(causal)), ft, _ptr(out), _ptr(lse),
            _ptr(workspace), int(workspace.numel()))
    if num_workers is None:
        _lib.check(lib.vlp_varlen_attn_fwd(*args, stream), "varlen_attn_fwd")
    else:
        _lib.check(lib.vlp_varlen_attn_fwd_persistent(*args, int(num_workers), stream), "varlen_attn_fwd_persistent")
    return out, lse


# ---------------------------------------------------------------------------
# attention gradients
# ---------------------------------------------------------------------------

def bwd_workspace_size(num_seqs: int, rows_q: int, total_k: int, heads: int, block_m: int) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().vlp_varlen_attn_bwd_workspace_size(int(num_seqs), int(rows_q), int(total_k), int(heads),
                                                              int(block_m), ctypes.addressof(n)),
               "bwd_workspace_size")
    return int(n.value)


def varlen_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                    lse: torch.Tensor, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                    max_seqlen: int = 0, scale: Optional[float] = None, causal: bool = False,
                    dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                    dv: Optional[torch.Tensor] = None, *, workspace: Optional[torch.Tensor] = None,
                    grids: Optional[tuple] = None, row_stats: Optional[torch.Tensor] = None,
                    phases: int = 3, num_workers: Optional[int] = None):
    """Gradients (dq, dk, dv) of ``varlen_attn_fwd`` on the current stream.

    ``out`` and ``lse`` are the forward's results for the same arguments;
    ``dout`` has the shape of ``out``.  Rows owned by no sequence are never
    written (fresh outputs are allocated with ``torch.empty``).
    ``grids``: cached device metadata ``(query_grid, key_grid)`` from
    ``build_ragged_grid`` over cu_seqlens_q with ``bwd_block_m`` and over
    cu_seqlens_k with VLP_BWD_BLOCK_K; then ``row_stats`` (fp32 [2, H, rows_q]) carries the row
    statistics from the dq phase to the dk/dv phase and ``phases`` selects
    VLP_BWD_DQ, VLP_BWD_DKDV or both.  ``num_workers``: as for
    ``varlen_attn_fwd`` (device-built grids only), per gradient launch.
    """
    lib = _lib.load()
    tensors = (q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k) + tuple(
        t for t in (dq, dk, dv, workspace, row_stats) if t is not None)
    if not q.is_cuda or any(t.device != q.device for t in tensors):
        raise ValueError("all inputs must be device tensors on q's device")
    _check_cu(cu_seqlens_q, "cu_seqlens_q", q.device)
    _check_cu(cu_seqlens_k, "cu_seqlens_k", q.device)
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same number of entries")
    if q.dtype not in _DTYPE_CODES or any(t.dtype != q.dtype for t in (k, v, out, dout)):
        raise TypeError("q, k, v, out, dout must share one of float32 / float16 / bfloat16")
    if q.dim() != 3 or k.shape != v.shape or q.shape[1:] != k.shape[1:] or out.shape != q.shape \
            or dout.shape != q.shape:
        raise ValueError("q/out/dout [rows, H, D] and k, v [T, H, D] with matching H, D")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[1], q.shape[0]):
        raise ValueError("lse must be float32 [H, rows]")
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous")
    q_st, k_st, v_st = _token_stride(q, "q"), _token_stride(k, "k"), _token_stride(v, "v")
    o_st, do_st = _token_stride(out, "out"), _token_stride(dout, "dout")
    if k_st != v_st and k.shape[0] > 1:
        raise ValueError("k and v must share one token stride")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    rows_q, heads, head_dim = (int(x) for x in q.shape)
    total_k = int(k.shape[0])
    b = int(cu_seqlens_k.numel()) - 1
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    dq = torch.empty(q.shape, dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=k.dtype, device=k.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=v.dtype, device=v.device) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.dtype != ref.dtype or t.shape != ref.shape:
            raise ValueError(f"{name} must match the dtype and shape of its input")
    if row_stats is not None and (row_stats.dtype != torch.float32 or not row_stats.is_contiguous()
                                  or tuple(row_stats.shape) != (2, heads, rows_q)):
        raise ValueError("row_stats must be a contiguous float32 [2, H, rows_q] tensor")
    dq_st, dk_st, dv_st = _token_stride(dq, "dq"), _token_stride(dk, "dk"), _token_stride(dv, "dv")
    if dk_st != dv_st and dk.shape[0] > 1:
        raise ValueError("dk and dv must share one token stride")
    strides = (q_st, k_st, o_st, do_st, dq_st, dk_st)
    code = _DTYPE_CODES[q.dtype]
    if grids is not None and num_workers is not None:
        raise ValueError("the persistent schedule builds its grids on the device: pass grids or num_workers")
    if grids is not None:
        gq, gk = grids
        if row_stats is None:
            row_stats = torch.empty(2, heads, rows_q, dtype=torch.float32, device=q.device)

        def nblocks(g):
            return g.num_blocks if g.num_blocks is not None else int(g.grid_mapping.numel())
        st = lib.vlp_varlen_attn_bwd_grid(code, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                          _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), b, rows_q, total_k, heads,
                                          head_dim, *strides, int(max_seqlen), float(scale), int(bool(causal)),
                                          _ptr(dq),
                                          _ptr(dk), _ptr(dv), _ptr(gq.grid_mapping), _ptr(gq.block_offsets),
                                          _ptr(gq.tile_order), nblocks(gq), _ptr(gk.grid_mapping),
                                          _ptr(gk.block_offsets), _ptr(gk.tile_order), nblocks(gk), gq.block_m,
                                          _ptr(row_stats), int(phases), _stream_handle(q.device))
        _lib.check(st, "varlen_attn_bwd_grid")
        return dq, dk, dv
    if workspace is None:
        bm = lib.vlp_bwd_block_m(code, head_dim, int(bool(causal)))
        if bm < 1:
            raise _lib.VlpError(_lib.VLP_ERR_UNSUPPORTED, "varlen_attn_bwd")
        nbytes = bwd_workspace_size(b, rows_q, total_k, heads, bm)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    args = (code, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(cu_seqlens_q),
            _ptr(cu_seqlens_k), b, rows_q, total_k, heads, head_dim, *strides, int(max_seqlen), float(scale),
            int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), int(workspace.numel()))
    stream = _stream_handle(q.device)
    if num_workers is None:
        _lib.check(lib.vlp_varlen_attn_bwd(*args, stream), "varlen_attn_bwd")
    else:
        _lib.check(lib.vlp_varlen_attn_bwd_persistent(*args, int(num_workers), stream), "varlen_attn_bwd_persistent")
    return dq, dk, dv


# ---------------------------------------------------------------------------
# ragged matrix multiplication
# ---------------------------------------------------------------------------

def ragged_matmul(x: torch.Tensor, weight: torch.Tensor, cu_seqlens: torch.Tensor,
                  bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, *,
                  workspace: Optional[torch.Tensor] = None, num_workers: Optional[int] = None) -> torch.Tensor:
    """y = x_i @ weight_i^T (+ bias_i) for the rows of every sequence i.

    x [rows, K] contiguous; weight [B, N, K] (one linear-layer weight per
    sequence) or [N, K] (shared); bias None, [B, N] or [N]; cu_seqlens int32
    [B+1] on the device.  Returns y [rows, N]; rows owned by no sequence are
    left as they were (fresh outputs come from ``torch.empty``).
    ``num_workers``: as for ``varlen_attn_fwd``.
    """
    lib = _lib.load()
    if not (x.is_cuda and weight.is_cuda and cu_seqlens.is_cuda):
        raise ValueError("x, weight and cu_seqlens must be device tensors")
    if x.dtype not in _DTYPE_CODES or weight.dtype != x.dtype or (bias is not None and bias.dtype != x.dtype):
        raise TypeError("x, weight and bias must share one of float16 / bfloat16")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    for t in (x, weight) + (() if bias is None else (bias,)):
        if not t.is_contiguous():
            raise ValueError("x, weight and bias must be contiguous")
    b = int(cu_seqlens.numel()) - 1
    rows, k = (int(d) for d in x.shape)
    if weight.dim() == 2:
        n, w_stride = int(weight.shape[0]), 0
    elif weight.dim() == 3 and weight.shape[0] == b:
        n, w_stride = int(weight.shape[1]), int(weight.shape[1] * weight.shape[2])
    else:
        raise ValueError("weight must be [N, K] or [num_seqs, N, K]")
    if int(weight.shape[-1]) != k:
        raise ValueError("weight's last dimension must equal x's")
    b_stride = 0
    if bias is not None:
        if bias.dim() == 2 and bias.shape[0] == b and bias.shape[1] == n:
            b_stride = n
        elif not (bias.dim() == 1 and bias.shape[0] == n):
            raise ValueError("bias must be [N] or [num_seqs, N]")
    if out is None:
        out = torch.empty(rows, n, dtype=x.dtype, device=x.device)
    elif out.shape != (rows, n) or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [rows, N] tensor of x's dtype")
    if workspace is None:
        nb = ctypes.c_size_t(0)
        _lib.check(lib.vlp_ragged_matmul_workspace_size(b, rows, ctypes.addressof(nb)), "ragged_matmul")
        workspace = torch.empty(max(int(nb.value), 256), dtype=torch.uint8, device=x.device)
    args = (_DTYPE_CODES[x.dtype], _ptr(x), _ptr(weight), _ptr(bias), _ptr(cu_seqlens), b, rows, k, n, w_stride,
            b_stride, _ptr(out), _ptr(workspace), int(workspace.numel()))
    if num_workers is None:
        _lib.check(lib.vlp_ragged_matmul(*args, _stream_handle(x.device)), "ragged_matmul")
    else:
        _lib.check(lib.vlp_ragged_matmul_persistent(*args, int(num_workers), _stream_handle(x.device)),
                   "ragged_matmul_persistent")
    return out


def cu_seqlens_from_ids(ids: torch.Tensor, max_seqs: int):
    """Device cu_seqlens [max_seqs + 1] of the runs of equal ids in ``ids``
    (int32 [T] on the device) and a device int32 [1] holding the run count;
    unused slots hold T (zero-length sequences).  Enqueued on the current
    stream, no host read."""
    if not ids.is_cuda or ids.dtype != torch.int32 or ids.dim() != 1 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous int32 device vector")
    cu = torch.empty(int(max_seqs) + 1, dtype=torch.int32, device=ids.device)
    n = torch.empty(1, dtype=torch.int32, device=ids.device)
    st = _lib.load().vlp_cu_seqlens_from_ids(_ptr(ids) if ids.numel() else None, int(ids.numel()), int(max_seqs),
                                             _ptr(cu), _ptr(n), _stream_handle(ids.device))
    _lib.check(st, "cu_seqlens_from_ids")
    return cu, n
