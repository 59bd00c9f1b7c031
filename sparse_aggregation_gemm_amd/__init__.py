"""MI355X (gfx950) hot path of one GNN layer on one GPU's share of a graph.

The computation lives in libsag.so (hand-written HIP, C ABI in
include/sag.h); this package is its Python binding.  Build the library with
``python -m sparse_aggregation_gemm_amd.build_lib``.
"""
from .ops import (  # noqa: F401
    Built, Csr, LayerCtx, aggregate_transform, as_dense, code_row_bytes, csr_build_normalize,
    csr_build_normalize_query, csr_hub_split, csr_info, csr_schedule, hub_chain, hub_split_pays,
    csr_set_col_slices, csr_tune_col_slices, col_slices_apply, auto_seg_len,
    dequantize_rows, dtype_code, empty_dense, GatCtx, gat_layer_backward, gat_layer_forward,
    gather_probe, gcn_layer_backward, gcn_layer_forward, gemm, gemm_tn,
    halo_gather, halo_push, padded_ld, quantize_rows, sage_layer_backward, sage_layer_forward,
    spmm_csr, spmm_csr_noalloc, spmm_csr_t, spmm_noalloc_scratch_bytes, trace_enable, trace_records, version,
)
from . import _lib  # noqa: F401
