"""ctypes loader for libcsa_hip.so (the C ABI declared in include/csa_hip.h).

There is no fallback: if the library is missing or cannot be loaded, every
call raises. Build it with ``python -m long_context_attention_csa_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa_hip.so")

CSA_F32, CSA_BF16, CSA_FP8_E4M3, CSA_FP4_E2M1 = 0, 1, 2, 3
STATUS = {0: "CSA_OK", 1: "CSA_ERR_NULL", 2: "CSA_ERR_SHAPE", 3: "CSA_ERR_UNSUPPORTED",
          4: "CSA_ERR_WORKSPACE", 5: "CSA_ERR_HIP"}
ATTN_WIN_RING, ATTN_BATCH_INVARIANT = 1, 2
KID = {"compress": 1, "hca_compress": 2, "quantize": 3, "index_score": 4, "topk": 5,
       "sparse_attn": 6, "dense_attn": 7, "attn_merge": 8, "attn_bwd": 9, "gemm": 10}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_U32 = ctypes.c_uint32

# name -> (restype, argtypes); mirrors include/csa_hip.h and include/csa_hip_timer.h
SIGNATURES = {
    "csa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "csa_last_error": (ctypes.c_char_p, []),
    "csa_version": (ctypes.c_char_p, []),
    "csa_quantize_rows": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I32, _P, ctypes.c_int, _P, _P]),
    "csa_compress": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I32, _I32, _P, ctypes.c_int, _P, _P]),
    "hca_compress": (ctypes.c_int, [_P, _P, ctypes.c_int, _I64, _I64, _I32, _I32, _P, ctypes.c_int, _P]),
    "csa_compress_append": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int, _I64, _I32, _I32, _P, _P, _I64, _P,
                                           ctypes.c_int, _P, _P]),
    "hca_compress_append": (ctypes.c_int, [_P, _P, ctypes.c_int, _I64, _I32, _I32, _P, _P, _I64, _P, ctypes.c_int,
                                           _P]),
    "indexer_topk_workspace_size": (_SZ, [_I64, _I64, _I64, _I32, _I32, _I32, ctypes.c_int]),
    "indexer_topk": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int, _P, _I64, _I64, _I64, _I32, _I32, _I32,
                                    _I32, _P, _P, _P, _SZ, _P]),
    "indexer_scores": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int, _P, _I64, _I64, _I64, _I32, _I32, _I32, _P,
                                      _P]),
    "indexer_topk_bf16_scores_workspace_size": (_SZ, [_I64, _I64, _I64, _I32, _I32, _I32, ctypes.c_int]),
    "indexer_topk_bf16_scores": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int, _P, _I64, _I64, _I64, _I32, _I32,
                                                _I32, _I32, _P, _P, _P, _SZ, _P]),
    "sparse_attn_workspace_size": (_SZ, [_I64, _I64, _I32, _I32, _I32, _I32, _U32]),
    "sparse_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64, _I32, _I32,
                                       _I32, _I32, _F, _P, _P, _P, _SZ, _U32, _P]),
    "sparse_attn_noalloc_scratch_bytes": (_SZ, []),
    "sparse_attn_fwd_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64,
                                               _I32, _I32, _I32, _I32, _F, _P, _P, _U32, _P]),
    "csa_state_checkpoint": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _P, _I64, _P]),
    "csa_state_restore": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "csa_ring_fill": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _I64, _P, _P]),
    "csa_linear_bf16": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _I64, _P, ctypes.c_int, _I64, _I64, _I64, _I64,
                                       _I64, _I64, _P]),
    "csa_grouped_out_proj_workspace_size": (_SZ, [_I64, _I32, _I32]),
    "csa_grouped_out_proj": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "csa_query_proj_shared_workspace_size": (_SZ, [_I64, _I32]),
    "csa_query_proj_shared": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "csa_kv_proj": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _I32, _P, _I32, _P]),
    "sparse_attn_bwd_workspace_size": (_SZ, [_I64, _I64, _I64, _I64, _I32, _I32, _I32, _I32]),
    "sparse_attn_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64, _I32, _I32,
                                       _I32, _I32, _F, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dense_attn_bwd_workspace_size": (_SZ, [_I64, _I64, _I64, _I64, _I32, _I32, _I32]),
    "dense_compressed_attn_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64, _I32,
                                                 _I32, _I32, _I32, _F, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dense_attn_workspace_size": (_SZ, [_I64, _I64, _I64, _I32, _I32, _I32, _U32]),
    "dense_compressed_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64, _I32,
                                                 _I32, _I32, _I32, _F, _P, _P, _P, _SZ, _U32, _P]),
    "csa_window_append": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I32, _P, _P, _I64, _P]),
    "csa_kernel_timer_start": (ctypes.c_int, [_I32, _I32]),
    "csa_kernel_timer_read": (_I32, [ctypes.POINTER(ctypes.c_float), _I32]),
}

_lib = None


class CsaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_attention_csa_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def check(fn: str, status: int) -> None:
    if status != 0:
        raise CsaError(fn, status, lib().csa_last_error().decode())
