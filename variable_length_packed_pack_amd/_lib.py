"""ctypes declarations for libvlp.so (the C ABI in include/vlp.h).

Loading is lazy and loud: if the library has not been built, every call
raises ``RuntimeError`` -- there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvlp.so")

VLP_OK = 0
VLP_ERR_NULL = 1
VLP_ERR_INVALID = 2
VLP_ERR_UNSUPPORTED = 3
VLP_ERR_CAPACITY = 4
VLP_ERR_OVERFLOW = 5
VLP_ERR_HIP = 6

VLP_FP32 = 0
VLP_FP16 = 1
VLP_BF16 = 2

VLP_FIRST_TOKEN_BLOCK_M = 1 << 30
VLP_DEVICE_SORT_MAX_SEQS = 4096
VLP_BWD_DQ = 1
VLP_BWD_DKDV = 2
VLP_BWD_BLOCK_K = 64
VLP_MATMUL_BLOCK_M = 128
VLP_FIRST_TOKEN_CHUNK_KEYS = 4096
VLP_FIRST_TOKEN_CHUNK_MIN = 8192

_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p

# name -> (restype, argtypes), in the order of include/vlp.h
SIGNATURES = {
    "vlp_pack_sequences": (ctypes.c_int32, [_vp, ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int64, _vp, _vp]),
    "vlp_grid_capacity": (ctypes.c_int64, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]),
    "vlp_build_ragged_grid": (ctypes.c_int32, [_vp, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp,
                                               ctypes.c_int64, _vp]),
    "vlp_build_ragged_grid_device": (ctypes.c_int32, [_vp, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp,
                                                      ctypes.c_int64, _vp]),
    "vlp_kernel_block_m": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]),
    "vlp_bwd_block_m": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "vlp_varlen_attn_workspace_size": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _vp]),
    "vlp_varlen_attn_fwd_workspace_size": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                                            ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp]),
    "vlp_varlen_attn_fwd": (ctypes.c_int32, [ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                             *[ctypes.c_int64] * 3,
                                             ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                                             _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "vlp_varlen_attn_fwd_noalloc": (ctypes.c_int32, [ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                     *[ctypes.c_int64] * 3,
                                                     ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                                                     _vp, _vp, _vp]),
    "vlp_varlen_attn_fwd_persistent": (ctypes.c_int32, [ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                                        ctypes.c_int32, *[ctypes.c_int64] * 3,
                                                        ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                                        ctypes.c_int32, _vp, _vp, _vp, ctypes.c_size_t,
                                                        ctypes.c_int32, _vp]),
    "vlp_varlen_attn_fwd_grid": (ctypes.c_int32, [ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                  *[ctypes.c_int64] * 3,
                                                  ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                                                  _vp, _vp, _vp, _vp, _vp, ctypes.c_int64, ctypes.c_int32, _vp]),
    "vlp_varlen_attn_bwd_workspace_size": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                                           ctypes.c_int32, ctypes.c_int32, _vp]),
    "vlp_varlen_attn_bwd": (ctypes.c_int32, [ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                             ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_int32, *[ctypes.c_int64] * 6,
                                             ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                             _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "vlp_varlen_attn_bwd_persistent": (ctypes.c_int32, [ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                        ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                                        ctypes.c_int32, ctypes.c_int32, *[ctypes.c_int64] * 6,
                                                        ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                                        _vp, _vp, _vp, _vp, ctypes.c_size_t, ctypes.c_int32,
                                                        _vp]),
    "vlp_varlen_attn_bwd_grid": (ctypes.c_int32, [ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                  ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                                  ctypes.c_int32, *[ctypes.c_int64] * 6,
                                                  ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                                  _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int64, _vp, _vp, _vp,
                                                  ctypes.c_int64, ctypes.c_int32, _vp, ctypes.c_int32, _vp]),
    "vlp_ragged_matmul_workspace_size": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int64, _vp]),
    "vlp_ragged_matmul": (ctypes.c_int32, [ctypes.c_int32, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, _vp,
                                           _vp, ctypes.c_size_t, _vp]),
    "vlp_ragged_matmul_persistent": (ctypes.c_int32, [ctypes.c_int32, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                                      ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                      ctypes.c_int64, ctypes.c_int64, _vp, _vp, ctypes.c_size_t,
                                                      ctypes.c_int32, _vp]),
    "vlp_cu_seqlens_from_ids": (ctypes.c_int32, [_vp, ctypes.c_int64, ctypes.c_int32, _vp, _vp, _vp]),
    "vlp_mfma_rate": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp]),
    "vlp_build_info": (ctypes.c_char_p, []),
    "vlp_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
}

_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """Load libvlp.so once; raise if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is not built: run `python -m variable_length_packed_pack_amd.build` "
                    "(hipcc, gfx950). There is no non-HIP fallback.")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


class VlpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = load().vlp_status_string(status).decode()
        super().__init__(f"{where}: {msg}")


def check(status: int, where: str) -> None:
    if status != VLP_OK:
        raise VlpError(status, where)
