"""CPU tier: the C ABI loads, exports what include/vlp.h declares, and its host
functions agree bit for bit with the oracle.  Argument validation of the
device entry points is exercised with dummy pointers: every case here fails
on the host before any HIP call, so no GPU is needed.
"""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
import variable_length_packed_pack_amd as vlp
from variable_length_packed_pack_amd import _lib
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vlp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libvlp.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vlp_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for must in ("vlp_pack_sequences", "vlp_build_ragged_grid", "vlp_varlen_attn_fwd",
                 "vlp_varlen_attn_fwd_grid", "vlp_build_ragged_grid_device", "vlp_grid_capacity",
                 "vlp_kernel_block_m", "vlp_varlen_attn_workspace_size", "vlp_status_string",
                 "vlp_varlen_attn_bwd", "vlp_varlen_attn_bwd_workspace_size", "vlp_ragged_matmul",
                 "vlp_varlen_attn_fwd_persistent", "vlp_varlen_attn_bwd_persistent", "vlp_ragged_matmul_persistent",
                 "vlp_bwd_block_m"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_declared_functions()) == set(_lib.SIGNATURES)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert f"#define VLP_DEVICE_SORT_MAX_SEQS {_lib.VLP_DEVICE_SORT_MAX_SEQS}" in text
    assert "#define VLP_FIRST_TOKEN_BLOCK_M (1 << 30)" in text
    assert f"#define VLP_BWD_DQ {_lib.VLP_BWD_DQ}" in text and f"#define VLP_BWD_DKDV {_lib.VLP_BWD_DKDV}" in text
    assert f"#define VLP_BWD_BLOCK_K {_lib.VLP_BWD_BLOCK_K}" in text
    assert f"#define VLP_MATMUL_BLOCK_M {_lib.VLP_MATMUL_BLOCK_M}" in text
    assert f"#define VLP_FIRST_TOKEN_CHUNK_KEYS {_lib.VLP_FIRST_TOKEN_CHUNK_KEYS}" in text
    assert f"#define VLP_FIRST_TOKEN_CHUNK_MIN {_lib.VLP_FIRST_TOKEN_CHUNK_MIN}" in text
    for name in ("VLP_FP32 = 0", "VLP_FP16 = 1", "VLP_BF16 = 2", "VLP_OK = 0", "VLP_ERR_HIP = 6"):
        assert name in text


# --------------------------------------------------------------------------
# pack_sequences
# --------------------------------------------------------------------------

def test_pack_worked_example():
    flat, cu = vlp.pack_sequences([3, 1, 2], 3)
    assert flat.tolist() == [0, 1, 2, 3, 6, 7]
    assert cu.tolist() == [0, 3, 4, 6]
    assert flat.dtype == torch.int64 and cu.dtype == torch.int32


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_pack_matches_oracle_on_workloads(k):
    lengths = workloads.draw_lengths(k)
    max_len = int(lengths.max())
    flat, cu = vlp.pack_sequences(lengths, max_len)
    oflat, ocu = oracle.pack_sequences(lengths, max_len)
    assert np.array_equal(flat.numpy(), oflat)
    assert np.array_equal(cu.numpy(), ocu)


@pytest.mark.parametrize("seed", range(10))
def test_pack_fuzz_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    b = int(rng.integers(1, 200))
    max_len = int(rng.integers(1, 500))
    lengths = rng.integers(1, max_len + 1, size=b)
    flat, cu = vlp.pack_sequences(lengths, max_len)
    oflat, ocu = oracle.pack_sequences(lengths, max_len)
    assert np.array_equal(flat.numpy(), oflat) and np.array_equal(cu.numpy(), ocu)


def test_pack_errors():
    lib = _lib.load()
    lens = np.asarray([3, 0, 2], dtype=np.int32)
    cu = np.zeros(4, dtype=np.int32)
    tot = ctypes.c_int64(0)
    assert lib.vlp_pack_sequences(lens.ctypes.data, 3, 3, None, 0, cu.ctypes.data, ctypes.addressof(tot)) == 2
    lens = np.asarray([3, 4], dtype=np.int32)
    assert lib.vlp_pack_sequences(lens.ctypes.data, 2, 3, None, 0, cu.ctypes.data, ctypes.addressof(tot)) == 2
    assert lib.vlp_pack_sequences(None, 2, 3, None, 0, cu.ctypes.data, ctypes.addressof(tot)) == 1
    assert lib.vlp_pack_sequences(lens.ctypes.data, 0, 3, None, 0, cu.ctypes.data, ctypes.addressof(tot)) == 2
    big = np.asarray([2**30 + 1, 2**30 + 1], dtype=np.int32)
    assert lib.vlp_pack_sequences(big.ctypes.data, 2, 2**30 + 1, None, 0, cu.ctypes.data,
                                  ctypes.addressof(tot)) == 5
    lens = np.asarray([3, 1, 2], dtype=np.int32)
    flat = np.zeros(5, dtype=np.int64)
    st = lib.vlp_pack_sequences(lens.ctypes.data, 3, 3, flat.ctypes.data, 5, cu.ctypes.data, ctypes.addressof(tot))
    assert st == 4 and tot.value == 6 and cu.tolist() == [0, 3, 4, 6]
    with pytest.raises(vlp.VlpError):
        vlp.pack_sequences([1, 0], 4)


# --------------------------------------------------------------------------
# ragged grid (host)
# --------------------------------------------------------------------------

def test_grid_worked_example():
    g = vlp.build_ragged_grid(torch.tensor([0, 65, 128], dtype=torch.int32), 64)
    assert g.block_offsets.tolist() == [0, 2, 3]
    assert g.grid_mapping.tolist() == [0, 0, 1]
    assert g.tile_order.tolist() == [1, 0, 2]
    assert g.num_blocks == 3


def _cu(lengths):
    return torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))


@pytest.mark.parametrize("block_m", [1, 7, 32, 64, 128, 1 << 30])
@pytest.mark.parametrize("seed", range(6))
def test_grid_matches_oracle(seed, block_m):
    rng = np.random.default_rng(seed)
    b = int(rng.integers(1, 300))
    lengths = rng.integers(0 if seed % 2 else 1, 700, size=b)
    if seed % 3 == 0:
        lengths[rng.integers(0, b, size=b // 3)] = 64  # many ties
    cu = _cu(lengths)
    g = vlp.build_ragged_grid(cu, block_m)
    bo, gm, to = oracle.build_ragged_grid(cu.numpy(), block_m)
    assert np.array_equal(g.block_offsets.numpy(), bo)
    assert np.array_equal(g.grid_mapping.numpy(), gm)
    assert np.array_equal(g.tile_order.numpy(), to)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_grid_matches_oracle_on_workloads(k):
    lengths = workloads.draw_lengths(k)
    cu = _cu(lengths)
    for bm in (32, 64, 128):
        g = vlp.build_ragged_grid(cu, bm)
        bo, gm, to = oracle.build_ragged_grid(cu.numpy(), bm)
        assert np.array_equal(g.block_offsets.numpy(), bo)
        assert np.array_equal(g.grid_mapping.numpy(), gm)
        assert np.array_equal(g.tile_order.numpy(), to)


def test_grid_capacity_matches_oracle():
    rng = np.random.default_rng(3)
    for _ in range(200):
        t = int(rng.integers(0, 10**6))
        n = int(rng.integers(0, 5000))
        c = int(rng.integers(1, 300))
        assert vlp.grid_capacity(t, n, c) == oracle.grid_capacity(t, n, c)
    assert vlp.grid_capacity(-1, 3, 4) == -1 and vlp.grid_capacity(3, 3, 0) == -1


def test_grid_errors():
    lib = _lib.load()
    bo = np.zeros(3, dtype=np.int32)
    gm = np.zeros(8, dtype=np.int32)
    nb = ctypes.c_int64(0)
    bad = np.asarray([1, 65, 128], dtype=np.int32)
    assert lib.vlp_build_ragged_grid(bad.ctypes.data, 2, 64, bo.ctypes.data, None, None, 0,
                                     ctypes.addressof(nb)) == 2
    dec = np.asarray([0, 65, 60], dtype=np.int32)
    assert lib.vlp_build_ragged_grid(dec.ctypes.data, 2, 64, bo.ctypes.data, None, None, 0,
                                     ctypes.addressof(nb)) == 2
    ok = np.asarray([0, 65, 128], dtype=np.int32)
    assert lib.vlp_build_ragged_grid(ok.ctypes.data, 2, 0, bo.ctypes.data, None, None, 0,
                                     ctypes.addressof(nb)) == 2
    st = lib.vlp_build_ragged_grid(ok.ctypes.data, 2, 64, bo.ctypes.data, gm.ctypes.data, None, 2,
                                   ctypes.addressof(nb))
    assert st == 4 and nb.value == 3 and bo.tolist() == [0, 2, 3]
    assert lib.vlp_build_ragged_grid(None, 2, 64, bo.ctypes.data, None, None, 0, ctypes.addressof(nb)) == 1


def test_kernel_block_m_and_workspace():
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        for d in (16, 32, 64, 128):
            bm = vlp.kernel_block_m(dt, d)
            assert bm >= 32 and bm % 32 == 0
            assert vlp.kernel_block_m(dt, d, query_is_first_token=True) == vlp.VLP_FIRST_TOKEN_BLOCK_M
        assert vlp.kernel_block_m(dt, 48) == -1
        assert vlp.kernel_block_m(dt, 256) == -1
    assert vlp.kernel_block_m(torch.int32, 64) == -1
    # 16-bit head_dim 128 runs the two-group forward (256-row tiles); the
    # backward's dq phase keeps 128-row tiles.
    assert vlp.kernel_block_m(torch.bfloat16, 128, True) == 256
    assert vlp.kernel_block_m(torch.float16, 128) == 256
    assert vlp.kernel_block_m(torch.float32, 128) == 64
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        for d in (16, 32, 64, 128):
            bb = vlp.bwd_block_m(dt, d, True)
            assert bb >= 32 and bb % 32 == 0
        assert vlp.bwd_block_m(dt, 48) == -1
    assert vlp.bwd_block_m(torch.bfloat16, 128) == 128
    assert vlp.bwd_block_m(torch.int32, 64) == -1
    ws = vlp.workspace_size(64, 65536, 128)
    cap = vlp.grid_capacity(65536, 64, 128)
    assert ws >= 4 * (65 + 2 * cap)


def test_forward_workspace_size_query():
    """vlp_varlen_attn_fwd_workspace_size: the grid workspace of
    vlp_varlen_attn_workspace_size for every tiled launch; first-token mode
    over sequences of 8192+ keys (the chunked form) adds a grid over the keys
    in 4096-key tiles, one arrival counter per (sequence, head) and one
    partial state of head_dim + 4 floats per (tile, head)."""
    lib = _lib.load()
    for dt, d in ((torch.bfloat16, 128), (torch.float32, 64), (torch.float16, 16)):
        for causal in (False, True):
            bm = vlp.kernel_block_m(dt, d, causal)
            assert vlp.fwd_workspace_size(dt, 64, 65536, 65536, 16, d, 13802, causal) == vlp.workspace_size(
                64, 65536, bm)
    # first-token mode: short sequences, or causal (one key), use the one-tile-per-sequence grid
    short = vlp.fwd_workspace_size(torch.bfloat16, 64, 64, 65536, 16, 128, 8191, False, True)
    assert short == vlp.workspace_size(64, 64, vlp.kernel_block_m(torch.bfloat16, 128, False, True))
    assert vlp.fwd_workspace_size(torch.bfloat16, 64, 64, 65536, 16, 128, 13802, True, True) == short
    # chunked form: every part of the layout fits
    ws = vlp.fwd_workspace_size(torch.bfloat16, 64, 64, 65536, 16, 128, 13802, False, True)
    cap = vlp.grid_capacity(65536, 64, 4096)
    assert ws >= 4 * (65 + 2 * cap) + 4 * 64 * 16 + 4 * cap * 16 * (128 + 4)
    # without the hint the mean length (1024 here) decides: not chunked
    assert vlp.fwd_workspace_size(torch.bfloat16, 64, 64, 65536, 16, 128, 0, False, True) == short
    n = ctypes.c_size_t(0)
    fws = lib.vlp_varlen_attn_fwd_workspace_size
    assert fws(2, 4, 10, 10, 1, 64, 0, 0, 0, None) == _lib.VLP_ERR_NULL
    assert fws(7, 4, 10, 10, 1, 64, 0, 0, 0, ctypes.addressof(n)) == _lib.VLP_ERR_UNSUPPORTED
    assert fws(2, 4, 10, 10, 1, 48, 0, 0, 0, ctypes.addressof(n)) == _lib.VLP_ERR_UNSUPPORTED
    assert fws(2, 0, 10, 10, 1, 64, 0, 0, 0, ctypes.addressof(n)) == _lib.VLP_ERR_INVALID
    assert fws(2, 4, 10, 10, 0, 64, 0, 0, 0, ctypes.addressof(n)) == _lib.VLP_ERR_INVALID
    assert fws(2, 4, 10, 10, 1, 64, 0, 2, 0, ctypes.addressof(n)) == _lib.VLP_ERR_INVALID
    assert fws(2, 4, 1 << 31, 10, 1, 64, 0, 0, 0, ctypes.addressof(n)) == _lib.VLP_ERR_OVERFLOW


def test_chunked_first_token_refuses_a_grid_only_workspace():
    """The chunked form needs more than vlp_varlen_attn_workspace_size gives:
    a workspace sized that way is refused with VLP_ERR_CAPACITY before any
    HIP call."""
    lib = _lib.load()
    bm = vlp.kernel_block_m(torch.bfloat16, 128, False, True)
    small = vlp.workspace_size(4, 4, bm)
    st = lib.vlp_varlen_attn_fwd(2, FAKE, FAKE, FAKE, None, FAKE, 4, 4, 40000, 2, 128, 0, 0, 0, 20000, 0.125, 0, 1,
                                 FAKE, None, FAKE, small, None)
    assert st == _lib.VLP_ERR_CAPACITY


# --------------------------------------------------------------------------
# forward argument validation (host only; no HIP call is reached)
# --------------------------------------------------------------------------

FAKE = 0x10000  # aligned, never dereferenced: each case fails validation first


# Which entry point the validation helpers call: None = the static grid,
# an int = the persistent schedule with that num_workers.
_WORKERS = [None]


@pytest.fixture(params=[None, 0, 24], ids=["static", "persistent-resident", "persistent-24"], autouse=False)
def schedule(request):
    _WORKERS[0] = request.param
    yield request.param
    _WORKERS[0] = None


def _fwd(**kw):
    lib = _lib.load()
    a = dict(dtype=2, q=FAKE, k=FAKE, v=FAKE, cu_q=FAKE, cu_k=FAKE, b=4, rows_q=100, total_k=100, heads=2,
             head_dim=64, qs=0, kvs=0, os=0, max_seqlen=0, scale=0.125, causal=0, ft=0, out=FAKE, lse=None, ws=FAKE,
             ws_bytes=1 << 20, workers=_WORKERS[0])
    a.update(kw)
    args = (a["dtype"], a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"], a["b"], a["rows_q"], a["total_k"], a["heads"],
            a["head_dim"], a["qs"], a["kvs"], a["os"], a["max_seqlen"], a["scale"], a["causal"], a["ft"], a["out"],
            a["lse"], a["ws"], a["ws_bytes"])
    if a["workers"] is None:
        return lib.vlp_varlen_attn_fwd(*args, None)
    return lib.vlp_varlen_attn_fwd_persistent(*args, a["workers"], None)


def test_persistent_entry_points_reject_negative_worker_counts():
    assert _fwd(workers=-1) == 2
    assert _fwd(workers=-1, ws_bytes=16) == 2       # checked before anything else of the launch
    assert _bwd(workers=-5) == 2
    assert _mm(workers=-1) == 2
    assert _fwd(workers=1, ws_bytes=16) == 4         # a positive count reaches the usual checks
    assert _bwd(workers=7, ws_bytes=64) == 4
    assert _mm(workers=3, ws_bytes=8) == 4


@pytest.mark.usefixtures("schedule")
def test_forward_validation_errors():
    assert _fwd(q=None) == 1
    assert _fwd(cu_k=None) == 1
    assert _fwd(cu_q=None) == 1
    assert _fwd(ws=None) == 1
    assert _fwd(dtype=7) == 3
    assert _fwd(head_dim=48) == 3
    assert _fwd(head_dim=256) == 3
    assert _fwd(b=0) == 2
    assert _fwd(heads=0) == 2
    assert _fwd(rows_q=-1) == 2
    assert _fwd(scale=float("nan")) == 2
    assert _fwd(scale=float("inf")) == 2
    assert _fwd(scale=-0.125, ws_bytes=16) == 4  # any finite scale passes (runs as |scale| on -q)
    assert _fwd(scale=-0.0, ws_bytes=16) == 4
    assert _fwd(scale=0.0) != 2
    assert _fwd(q=FAKE + 8) == 2
    assert _fwd(out=FAKE + 4) == 2
    assert _fwd(ws=FAKE + 16) == 2
    assert _fwd(causal=2) == 2
    assert _fwd(ft=1, rows_q=100) == 2          # first-token: one query per sequence
    assert _fwd(rows_q=2**31) == 5
    assert _fwd(rows_q=2**30, heads=4) == 5
    assert _fwd(ws_bytes=16) == 4
    # token strides: 0 = contiguous; >= heads*head_dim; 16-byte rows; <= 2^24 bytes
    assert _fwd(qs=128, kvs=384, os=128, ws_bytes=16) == 4   # valid strides reach the workspace check
    assert _fwd(qs=127) == 2                    # below heads * head_dim
    assert _fwd(kvs=132) == 2                   # 264-byte rows: not 16-byte aligned
    assert _fwd(os=-1) == 2
    assert _fwd(dtype=0, qs=130) == 2           # fp32: 520-byte rows are not 16-byte aligned
    assert _fwd(qs=(1 << 23) + 8) == 5          # beyond 2^24 bytes per token


def test_grid_forward_validation_errors():
    lib = _lib.load()

    def call(**kw):
        a = dict(gm=FAKE, bo=FAKE, to=None, nb=3, bm=lib.vlp_kernel_block_m(2, 128, 0, 0, 4, 100, 0), head_dim=128)
        a.update(kw)
        return lib.vlp_varlen_attn_fwd_grid(2, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 100, 100, 2, a["head_dim"], 0, 0,
                                            a.get("os", 0), 0, 0.1, 0, 0, FAKE, None, a["gm"], a["bo"], a["to"],
                                            a["nb"], a["bm"], None)
    assert call(gm=None) == 1
    assert call(bo=None) == 1
    assert call(nb=-1) == 2
    assert call(bm=64) == 2                      # must equal vlp_kernel_block_m
    assert call(nb=2**31) == 5
    assert call(os=100) == 2


def _bwd(**kw):
    lib = _lib.load()
    a = dict(dtype=2, q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, lse=FAKE, cu_q=FAKE, cu_k=FAKE, b=4, rows_q=100,
             total_k=100, heads=2, head_dim=64, strides=(0, 0, 0, 0, 0, 0), max_seqlen=0, scale=0.125, causal=0,
             dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE, ws_bytes=1 << 20, workers=_WORKERS[0])
    a.update(kw)
    args = (a["dtype"], a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["cu_q"], a["cu_k"], a["b"],
            a["rows_q"], a["total_k"], a["heads"], a["head_dim"], *a["strides"], a["max_seqlen"], a["scale"],
            a["causal"], a["dq"], a["dk"], a["dv"], a["ws"], a["ws_bytes"])
    if a["workers"] is None:
        return lib.vlp_varlen_attn_bwd(*args, None)
    return lib.vlp_varlen_attn_bwd_persistent(*args, a["workers"], None)


@pytest.mark.usefixtures("schedule")
def test_backward_validation_errors():
    for name in ("q", "k", "v", "out", "dout", "lse", "cu_q", "cu_k", "dq", "dk", "dv", "ws"):
        assert _bwd(**{name: None}) == 1, name
    assert _bwd(dtype=7) == 3
    assert _bwd(head_dim=48) == 3
    assert _bwd(b=0) == 2
    assert _bwd(heads=0) == 2
    assert _bwd(total_k=-1) == 2
    assert _bwd(scale=float("nan")) == 2
    assert _bwd(scale=-1.0, ws_bytes=16) == 4  # any finite scale passes validation
    assert _bwd(causal=3) == 2
    for name in ("dout", "dq", "dk", "dv"):
        assert _bwd(**{name: FAKE + 8}) == 2, name
    assert _bwd(lse=FAKE + 2) == 2
    assert _bwd(ws=FAKE + 64) == 2
    assert _bwd(rows_q=2**31) == 5
    assert _bwd(total_k=2**30, heads=4) == 5
    assert _bwd(ws_bytes=64) == 4
    assert _bwd(strides=(384, 384, 128, 128, 384, 384), ws_bytes=64) == 4   # fused q/k/v and dq/dk/dv views
    for i in range(6):
        bad = [0] * 6
        bad[i] = 120
        assert _bwd(strides=tuple(bad)) == 2, i


def test_grid_backward_validation_errors():
    lib = _lib.load()
    bm = lib.vlp_bwd_block_m(2, 64, 0)

    def call(**kw):
        a = dict(qgm=FAKE, qbo=FAKE, qn=3, kgm=FAKE, kbo=FAKE, kn=3, bm=bm, stats=FAKE, phases=3, dq=FAKE)
        a.update(kw)
        return lib.vlp_varlen_attn_bwd_grid(2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 100, 100, 2, 64,
                                            0, 0, 0, 0, 0, 0, 0, 0.1, 0, a["dq"], FAKE, FAKE, a["qgm"], a["qbo"], None,
                                            a["qn"],
                                            a["kgm"], a["kbo"], None, a["kn"], a["bm"], a["stats"], a["phases"],
                                            None)
    assert call(dq=None) == 1
    assert call(stats=None) == 1
    assert call(qgm=None) == 1
    assert call(kbo=None) == 1
    assert call(qgm=None, phases=2) != 1        # the dq grid is not needed for the dk/dv phase alone
    assert call(kgm=None, phases=1) != 1
    assert call(phases=0) == 2
    assert call(phases=4) == 2
    assert call(bm=bm // 2) == 2
    assert call(qn=-1) == 2
    assert call(stats=FAKE + 2) == 2
    assert call(kn=2**31) == 5


def test_backward_workspace_size():
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    assert lib.vlp_varlen_attn_bwd_workspace_size(64, 65536, 65536, 16, 128, None) == 1
    assert lib.vlp_varlen_attn_bwd_workspace_size(0, 10, 10, 1, 128, ctypes.addressof(n)) == 2
    assert lib.vlp_varlen_attn_bwd_workspace_size(4, 10, 10, 0, 128, ctypes.addressof(n)) == 2
    assert lib.vlp_varlen_attn_bwd_workspace_size(4, 10, 10, 1, 0, ctypes.addressof(n)) == 2
    assert lib.vlp_varlen_attn_bwd_workspace_size(64, 65536, 70000, 16, 128, ctypes.addressof(n)) == 0
    cq = vlp.grid_capacity(65536, 64, 128)
    ck = vlp.grid_capacity(70000, 64, vlp.VLP_BWD_BLOCK_K)
    assert n.value >= 2 * 4 * 16 * 65536 + 4 * (2 * 65 + 2 * cq + 2 * ck)
    assert n.value == vlp.bwd_workspace_size(64, 65536, 70000, 16, 128)


def _mm(**kw):
    lib = _lib.load()
    a = dict(dtype=2, x=FAKE, w=FAKE, bias=None, cu=FAKE, b=4, rows=100, k=512, n=256, ws_=0, bs=0, y=FAKE, ws=FAKE,
             ws_bytes=1 << 20, workers=_WORKERS[0])
    a.update(kw)
    args = (a["dtype"], a["x"], a["w"], a["bias"], a["cu"], a["b"], a["rows"], a["k"], a["n"], a["ws_"], a["bs"],
            a["y"], a["ws"], a["ws_bytes"])
    if a["workers"] is None:
        return lib.vlp_ragged_matmul(*args, None)
    return lib.vlp_ragged_matmul_persistent(*args, a["workers"], None)


@pytest.mark.usefixtures("schedule")
def test_ragged_matmul_validation_errors():
    for name in ("x", "w", "cu", "y", "ws"):
        assert _mm(**{name: None}) == 1, name
    assert _mm(dtype=0) == 3 and _mm(dtype=9) == 3
    assert _mm(b=0) == 2 and _mm(rows=-1) == 2
    assert _mm(k=96) == 2 and _mm(k=0) == 2 and _mm(k=65600) == 2   # multiples of 64 up to 65536
    assert _mm(n=6) == 2 and _mm(n=0) == 2
    assert _mm(ws_=-8) == 2 and _mm(ws_=12) == 2
    assert _mm(bias=FAKE, bs=2) == 2
    assert _mm(x=FAKE + 8) == 2 and _mm(bias=FAKE + 4) == 2 and _mm(ws=FAKE + 64) == 2
    assert _mm(rows=2**31) == 5
    assert _mm(ws_bytes=8) == 4
    lib = _lib.load()
    nb = ctypes.c_size_t(0)
    assert lib.vlp_ragged_matmul_workspace_size(64, 65536, ctypes.addressof(nb)) == 0
    assert nb.value >= 4 * (65 + 2 * vlp.grid_capacity(65536, 64, vlp.VLP_MATMUL_BLOCK_M))
    assert lib.vlp_ragged_matmul_workspace_size(0, 10, ctypes.addressof(nb)) == 2


def test_cu_seqlens_from_ids_validation_errors():
    lib = _lib.load()
    assert lib.vlp_cu_seqlens_from_ids(None, 10, 4, FAKE, FAKE, None) == 1
    assert lib.vlp_cu_seqlens_from_ids(FAKE, 10, 4, None, FAKE, None) == 1
    assert lib.vlp_cu_seqlens_from_ids(FAKE, 10, 4, FAKE, None, None) == 1
    assert lib.vlp_cu_seqlens_from_ids(FAKE, -1, 4, FAKE, FAKE, None) == 2
    assert lib.vlp_cu_seqlens_from_ids(FAKE, 10, 0, FAKE, FAKE, None) == 2
    assert lib.vlp_cu_seqlens_from_ids(FAKE, 2**31, 4, FAKE, FAKE, None) == 5


def test_device_grid_validation_errors():
    lib = _lib.load()
    assert lib.vlp_build_ragged_grid_device(None, 2, 64, FAKE, FAKE, FAKE, 4, None) == 1
    assert lib.vlp_build_ragged_grid_device(FAKE, 0, 64, FAKE, FAKE, FAKE, 4, None) == 2
    assert lib.vlp_build_ragged_grid_device(FAKE, 2, 0, FAKE, FAKE, FAKE, 4, None) == 2
    assert lib.vlp_build_ragged_grid_device(FAKE, 2, 64, FAKE, FAKE, FAKE, -1, None) == 2


def test_status_strings():
    lib = _lib.load()
    for code in range(7):
        assert lib.vlp_status_string(code)
    assert b"unknown" in lib.vlp_status_string(99)


def test_sources_never_bit_cast_a_vector_subscript():
    """hipcc (clang 22, ROCm 7.2) reads element 0 when __builtin_bit_cast is
    applied directly to an ext_vector_type subscript such as v[i]; the
    kernels bit-cast whole vectors instead.  Keep the pattern out."""
    csrc = os.path.join(ROOT, "variable_length_packed_pack_amd", "csrc")
    pat = re.compile(r"__builtin_bit_cast\s*\([^,()]+,\s*[A-Za-z_]\w*\s*\[")
    for name in os.listdir(csrc):
        text = open(os.path.join(csrc, name)).read()
        assert not pat.search(text), name


def _fwd_tensors(rows=6, heads=2, dim=16, dtype=torch.bfloat16, b=3):
    q = torch.zeros(rows, heads, dim, dtype=dtype)
    k = torch.zeros(rows, heads, dim, dtype=dtype)
    v = torch.zeros(rows, heads, dim, dtype=dtype)
    cu = torch.tensor([0, 3, 4, 6][: b + 1], dtype=torch.int32)
    return q, k, v, cu


def test_binding_forward_checks_accept_valid_arguments():
    q, k, v, cu = _fwd_tensors()
    out = torch.empty_like(q)
    lse = torch.empty(2, 6, dtype=torch.float32)
    assert vlp.check_fwd_args(q, k, v, cu, cu, out, lse) == (32, 32, 32)
    assert vlp.check_fwd_args(q, k, v, cu, cu, None, None)[2] is None
    qf = torch.zeros(3, 2, 16, dtype=torch.bfloat16)  # first-token mode: one query per sequence
    assert vlp.check_fwd_args(qf, k, v, None, cu, None, None, query_is_first_token=True)[0] == 32


@pytest.mark.parametrize("case", [
    "cu_q_int64", "cu_k_int64", "cu_q_short", "cu_q_strided", "cu_q_2d", "cu_q_missing", "out_dtype", "out_shape",
    "out_transposed", "lse_dtype", "lse_shape", "lse_transposed", "kv_dtype", "kv_shape", "first_token_rows",
])
def test_binding_forward_checks_reject_bad_arguments(case):
    """Every tensor argument of varlen_attn_fwd is checked in Python before
    the library sees a pointer: a wrong cu_seqlens, out or lse would otherwise
    be read or written out of bounds on the device."""
    q, k, v, cu = _fwd_tensors()
    cu_q, cu_k = cu, cu
    out = torch.empty_like(q)
    lse = torch.empty(2, 6, dtype=torch.float32)
    ft = False
    if case == "cu_q_int64":
        cu_q = cu.long()
    elif case == "cu_k_int64":
        cu_k = cu.long()
    elif case == "cu_q_short":
        cu_q = cu[:3].clone()
    elif case == "cu_q_strided":
        cu_q = torch.zeros(8, dtype=torch.int32)[::2]
    elif case == "cu_q_2d":
        cu_q = cu.view(1, 4)
    elif case == "cu_q_missing":
        cu_q = None
    elif case == "out_dtype":
        out = torch.empty(q.shape, dtype=torch.float16)
    elif case == "out_shape":
        out = torch.empty(5, 2, 16, dtype=q.dtype)
    elif case == "out_transposed":
        out = torch.empty(16, 2, 6, dtype=q.dtype).permute(2, 1, 0)
    elif case == "lse_dtype":
        lse = torch.empty(2, 6, dtype=torch.float16)
    elif case == "lse_shape":
        lse = torch.empty(6, 2, dtype=torch.float32)
    elif case == "lse_transposed":
        lse = torch.empty(6, 2, dtype=torch.float32).t()
    elif case == "kv_dtype":
        v = v.float()
    elif case == "kv_shape":
        v = v[:5]
    elif case == "first_token_rows":
        ft = True
    with pytest.raises((ValueError, TypeError)):
        vlp.check_fwd_args(q, k, v, cu_q, cu_k, out, lse, query_is_first_token=ft)


def test_binding_forward_rejects_host_tensors_before_any_launch():
    q, k, v, cu = _fwd_tensors()
    with pytest.raises(ValueError):
        vlp.varlen_attn_fwd(q, k, v, cu, cu, 4, None, False)


def test_loaded_library_matches_sources():
    """The library reports the hash of the sources it was built from; it must
    be the hash of the sources in this tree (a stale prebuilt library fails)."""
    from variable_length_packed_pack_amd.build import source_hash

    info = vlp.build_info()
    assert info == f"csrc={source_hash()} arch=gfx950", info
    assert vlp.check_library_current() == source_hash()


def test_mfma_rate_validates_before_any_launch():
    """The calibration entry point checks every argument on the host: bad
    values return their status without a HIP call (safe without a GPU)."""
    lib = _lib.load()
    flops = ctypes.c_double(-1.0)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its checks first
    fp = ctypes.addressof(flops)
    assert lib.vlp_mfma_rate(7, 256, 10, fake, fp, None) == _lib.VLP_ERR_UNSUPPORTED
    assert lib.vlp_mfma_rate(-1, 256, 10, fake, fp, None) == _lib.VLP_ERR_UNSUPPORTED
    assert lib.vlp_mfma_rate(_lib.VLP_BF16, 256, 10, None, fp, None) == _lib.VLP_ERR_NULL
    assert lib.vlp_mfma_rate(_lib.VLP_BF16, 256, 10, fake, None, None) == _lib.VLP_ERR_NULL
    assert lib.vlp_mfma_rate(_lib.VLP_BF16, 0, 10, fake, fp, None) == _lib.VLP_ERR_INVALID
    assert lib.vlp_mfma_rate(_lib.VLP_FP16, (1 << 16) + 1, 10, fake, fp, None) == _lib.VLP_ERR_INVALID
    assert lib.vlp_mfma_rate(_lib.VLP_FP32, 256, 0, fake, fp, None) == _lib.VLP_ERR_INVALID
    assert lib.vlp_mfma_rate(_lib.VLP_FP32, 256, (1 << 20) + 1, fake, fp, None) == _lib.VLP_ERR_INVALID
    assert flops.value == -1.0  # nothing written on a failed check
