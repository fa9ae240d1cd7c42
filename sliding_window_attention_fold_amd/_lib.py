"""ctypes loader for libnbattn.so (the C-ABI declared in include/nbattn.h,
include/nbexchange.h and include/nbring.h).

The library is built in-tree by ``sliding_window_attention_fold_amd.build``.  If it
is missing, loading fails loudly: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

# NBATTN_LIB selects another build of the same library (the host-AddressSanitizer
# debug build, libnbattn_asan.so, in its CPU test); by default the in-tree one.
LIB_PATH = os.environ.get("NBATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnbattn.so")

NB_OK, NB_ERR_INVALID_ARG, NB_ERR_UNSUPPORTED, NB_ERR_WORKSPACE, NB_ERR_LAUNCH, NB_ERR_DEVICE = range(6)
NB_BF16, NB_F32 = 0, 1
NB_SEG_HEADER = 16
HDR = dict(n_seg=0, max_q=1, max_k=2, status=3, lo=4, B=5, L=6, S=7, window=8, n_real=9)

# name -> (restype, argtypes); every symbol include/*.h declares
_c = ctypes
_P, _I, _F, _Z, _L = _c.c_void_p, _c.c_int, _c.c_float, _c.c_size_t, _c.c_int64
SIGNATURES = {
    "nb_status_string": (_c.c_char_p, [_I]),
    "nb_version": (_I, []),
    "nb_segment_offset_cu_q": (_Z, [_I, _I]),
    "nb_segment_offset_cu_k": (_Z, [_I, _I]),
    "nb_segment_offset_q_row0": (_Z, [_I, _I]),
    "nb_segment_offset_k_row0": (_Z, [_I, _I]),
    "nb_segment_offset_row_seg": (_Z, [_I, _I]),
    "nb_segment_offset_row_klo": (_Z, [_I, _I]),
    "nb_segment_offset_kcov_lo": (_Z, [_I, _I]),
    "nb_segment_offset_fwd_order": (_Z, [_I, _I]),
    "nb_segment_buffer_elems": (_Z, [_I, _I, _I]),
    "nb_segment_build": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _Z, _P]),
    "nb_segment_header": (_I, [_P, _P, _P]),
    "nb_attn_fwd_workspace_bytes": (_Z, [_I] * 7),
    "nb_attn_fwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _F, _I, _P, _Z, _P]),
    "nb_attn_bwd_workspace_bytes": (_Z, [_I] * 7),
    "nb_attn_bwd_workspace_bytes_window": (_Z, [_I] * 8),
    "nb_ring_chunk_bwd_workspace_bytes": (_Z, [_I] * 7),
    "nb_attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I,
                         _P, _P, _P, _P, _I, _P, _P, _Z, _P]),
    "nb_attn_bwd_dq": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _P, _Z, _P]),
    "nb_attn_bwd_dkdv": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _P, _P, _Z, _P]),
    "nb_attn_bwd_prep": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _Z, _P]),
    "nb_attn_bwd_main": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _P, _P, _P, _Z, _P]),
    "nb_owner_attended": (_I, [_P, _P, _I, _I, _I, _P, _I, _P, _P]),
    "nb_attn_bwd_noalloc_max_workspace_bytes": (_Z, []),
    "nb_attn_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I,
                                 _P, _P, _P, _P, _I, _P, _P]),
    "nb_attn_fwd_chunks": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _F,
                                _I, _P, _Z, _P]),
    "nb_attn_bwd_chunks": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F,
                                _I, _I, _P, _P, _P, _P, _P, _Z, _P]),
    # include/nbexchange.h
    "nb_exchange_plan_elems": (_Z, [_I]),
    "nb_exchange_plan": (_I, [_P, _P, _I, _I, _I, _P, _Z, _P]),
    "nb_exchange_send_index_elems": (_Z, [_I, _I]),
    "nb_exchange_send_index": (_I, [_P, _I, _I, _P, _Z, _P]),
    "nb_exchange_gather": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "nb_exchange_scatter_add": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "nb_ring_chunk_fwd": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "nb_ring_merge": (_I, [_P, _P, _P, _P, _L, _I, _I, _I, _P]),
    "nb_ring_live_rows": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "nb_ring_merge_live": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "nb_ring_finalize": (_I, [_P, _P, _P, _L, _I, _I, _P]),
    "nb_ring_chunk_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                               _P, _P, _P, _I, _P, _Z, _P]),
    "nb_ring_grad_add": (_I, [_P, _P, _L, _I, _I, _P]),
}
NB_XCH_MAX_RANKS = 64
NB_RING_DELTA_READY, NB_RING_DQ_F32_SET, NB_RING_DQ_F32_ADD = 1, 2, 4

_LIB = None


class NbError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -m sliding_window_attention_fold_amd.build` "
                "(the HIP library is required; there is no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def status_string(status: int) -> str:
    return load().nb_status_string(status).decode()


def check(status: int, where: str) -> None:
    if status != NB_OK:
        raise NbError(status, where)
