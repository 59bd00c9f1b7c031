"""ctypes declarations of the C ABI in include/sag.h (libsag.so).

Loading fails loudly when the library has not been built: there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsag.so")

i32, i64, u32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
vp, cint = ctypes.c_void_p, ctypes.c_int
P = ctypes.POINTER

# status codes
SAG_OK, SAG_E_INVALID, SAG_E_ALIGN, SAG_E_WORKSPACE = 0, -1, -2, -3
SAG_E_RANGE, SAG_E_HIP, SAG_E_UNSUPPORTED = -4, -5, -6
SAG_F32, SAG_BF16 = 0, 1
SAG_NORM_GCN, SAG_NORM_MEAN, SAG_NORM_NONE = 0, 1, 2
SAG_SYMMETRIZE, SAG_SELF_LOOPS = 1, 2
SAG_LAYER_FUSED = 1


class SagCsr(ctypes.Structure):
    _fields_ = [
        ("n_rows", i64), ("n_cols", i64), ("nnz", i64),
        ("indptr", vp), ("indices", vp), ("values", vp),
        ("sched", vp),
        ("n_short", i64), ("n_medium", i64), ("n_long", i64), ("n_seg", i64),
        ("seg_len", i32), ("row_mean", i32),
        ("hub_part", vp), ("cold_part", vp),
        ("col_slices", i32),
    ]


PCSR = P(SagCsr)

# name -> (restype, argtypes)
SIGNATURES = {
    "sag_csr_build_workspace_bytes": (sz, [i64, i64, i64, i64, u32]),
    "sag_csr_build_normalize_query": (cint, [vp, vp, i64, i64, i64, i64, u32, P(i64), P(i64), vp, sz, vp]),
    "sag_csr_build_normalize": (cint, [vp, vp, i64, i64, i64, i64, u32, cint, vp, i64, i64,
                                       vp, vp, vp, vp, vp, vp, vp, vp, P(i64), P(i64), vp, sz, vp]),
    "sag_csr_schedule_bytes": (sz, [i64, i64, i32]),
    "sag_csr_schedule_workspace_bytes": (sz, [i64]),
    "sag_csr_schedule": (cint, [PCSR, i32, vp, sz, vp, sz, vp]),
    "sag_csr_hub_split_workspace_bytes": (sz, [i64, i64]),
    "sag_csr_hub_split": (cint, [PCSR, i64, i64, vp, vp, vp, i64, vp, vp, vp, P(i64), vp, sz, vp]),
    "sag_halo_gather": (cint, [vp, i64, vp, i64, i64, i64, cint, vp, i64, vp]),
    "sag_halo_push": (cint, [vp, i64, vp, i64, i64, i64, cint, cint, vp, i64, i64, vp]),
    "sag_code_row_bytes": (sz, [i64, cint]),
    "sag_quantize_rows": (cint, [vp, i64, cint, vp, i64, vp, i64, i64, cint, ctypes.c_uint64, u32,
                                 vp, i64, vp, vp, vp]),
    "sag_dequantize_rows": (cint, [vp, i64, vp, vp, i64, i64, cint, vp, i64, cint, cint, vp, i64, i64, vp]),
    "sag_spmm_workspace_bytes": (sz, [PCSR, i64]),
    "sag_spmm_csr": (cint, [PCSR, vp, i64, cint, i64, vp, i64, cint, vp, i64, i64, vp, sz, vp]),
    "sag_spmm_csr_t": (cint, [PCSR, vp, i64, cint, i64, vp, i64, cint, vp, i64, i64, vp, sz, vp]),
    "sag_spmm_noalloc_scratch_bytes": (sz, []),
    "sag_spmm_csr_noalloc": (cint, [PCSR, vp, i64, cint, i64, vp, i64, cint, vp, i64, i64, vp]),
    "sag_gcn_save_bytes": (sz, [i64, i64, i64, cint]),
    "sag_gcn_forward_workspace_bytes": (sz, [PCSR, i64, i64, cint]),
    "sag_gcn_layer_forward": (cint, [PCSR, vp, i64, i64, vp, vp, i64, cint, u32, cint, vp, vp, i64,
                                     vp, sz, vp, sz, vp]),
    "sag_gcn_backward_workspace_bytes": (sz, [PCSR, i64, i64, i64, cint]),
    "sag_gcn_layer_backward": (cint, [PCSR, i64, vp, i64, i64, vp, i64, cint, vp, vp, i64,
                                      vp, vp, vp, i64, cint, vp, sz, vp, sz, vp]),
    "sag_sage_save_bytes": (sz, [i64, i64, i64, cint]),
    "sag_sage_forward_workspace_bytes": (sz, [PCSR, i64, i64, cint]),
    "sag_sage_layer_forward": (cint, [PCSR, vp, i64, i64, vp, vp, i64, cint, u32, cint, vp, vp, i64,
                                      vp, sz, vp, sz, vp]),
    "sag_sage_backward_workspace_bytes": (sz, [PCSR, i64, i64, i64, cint]),
    "sag_sage_layer_backward": (cint, [PCSR, i64, vp, i64, i64, vp, i64, cint, vp, vp, i64,
                                       vp, vp, vp, i64, cint, vp, sz, vp, sz, vp]),
    "sag_aggregate_transform_workspace_bytes": (sz, [PCSR, i64, i64, cint, cint]),
    "sag_aggregate_transform": (cint, [PCSR, vp, i64, i64, vp, vp, i64, cint, cint, cint, vp, vp, i64,
                                       vp, i64, vp, sz, vp]),
    "sag_gat_save_bytes": (sz, [i64, i64, i64, i64, cint]),
    "sag_gat_forward_workspace_bytes": (sz, [PCSR, i64, i64, i64, cint]),
    "sag_gat_layer_forward": (cint, [PCSR, vp, i64, i64, vp, vp, vp, vp, i64, i64, ctypes.c_float, cint,
                                     cint, vp, i64, vp, sz, vp, sz, vp]),
    "sag_gat_backward_workspace_bytes": (sz, [PCSR, PCSR, i64, i64, i64, cint]),
    "sag_gat_layer_backward": (cint, [PCSR, PCSR, vp, i64, i64, vp, vp, vp, i64, i64, ctypes.c_float,
                                      cint, vp, vp, i64, vp, vp, vp, vp, vp, i64, cint, vp, sz, vp, sz,
                                      vp]),
    "sag_gemm_workspace_bytes": (sz, [i64, i64, i64, cint]),
    "sag_gemm": (cint, [i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, vp, i64, cint, vp,
                        vp, i64, cint, vp, vp, i64, cint, vp, sz, vp]),
    "sag_gemm_tn_workspace_bytes": (sz, [i64, i64, i64, cint]),
    "sag_gemm_tn": (cint, [i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, vp, i64, vp, i64,
                           vp, cint, vp, sz, vp]),
    "sag_trace_enable": (cint, [cint]),
    "sag_trace_count": (i64, []),
    "sag_trace_get": (cint, [i64, ctypes.c_char_p, sz, P(ctypes.c_float), P(i64), P(i64)]),
    "sag_trace_clear": (cint, []),
    "sag_gather_probe_sink_bytes": (sz, []),
    "sag_gather_probe": (cint, [vp, i64, i64, cint, vp, i64, vp, sz, vp]),
    "sag_status_string": (ctypes.c_char_p, [cint]),
    "sag_last_error": (ctypes.c_char_p, []),
    "sag_version": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """The loaded libsag.so (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it first with "
                "`python -m sparse_aggregation_gemm_amd.build_lib` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class SagError(RuntimeError):
    def __init__(self, fn: str, status: int):
        L = lib()
        self.status = status
        super().__init__(f"{fn}: {L.sag_status_string(status).decode()} "
                         f"({L.sag_last_error().decode()})")


def check(fn: str, status: int) -> None:
    if status != SAG_OK:
        raise SagError(fn, status)
