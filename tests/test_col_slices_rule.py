"""Host-side rules of column slices (no GPU): which products a matrix's
col_slices flag applies to, that the binding's setter keeps the C struct in
step, that the tuner leaves an ineligible matrix whole without timing
anything, and that the workspace a product needs does not depend on the
flag.  The CSRs hold CPU tensors whose addresses are never dereferenced."""
import ctypes

import pytest
import torch

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from sparse_aggregation_gemm_amd import _lib as L  # noqa: E402


def fake_csr(n_rows=10, n_cols=20, nnz=30):
    return sag.Csr(n_rows, n_cols, torch.zeros(n_rows + 1, dtype=torch.int64),
                   torch.zeros(nnz, dtype=torch.int32), torch.ones(nnz))


@pytest.mark.parametrize("dtype,d,want", [(torch.float32, 64, False), (torch.float32, 65, True),
                                          (torch.float32, 1000, True), (torch.bfloat16, 128, False),
                                          (torch.bfloat16, 129, True), (torch.bfloat16, 100, False),
                                          (torch.bfloat16, 47, False)])
def test_rows_over_256_bytes_are_eligible(dtype, d, want):
    assert sag.col_slices_apply(fake_csr(), d, dtype) == want


def test_split_matrices_are_not_eligible():
    A = fake_csr()
    A.hub_part, A.cold_part = fake_csr(), fake_csr()
    assert not sag.col_slices_apply(A, 256, torch.bfloat16)


def test_setter_keeps_the_struct_in_step():
    A = fake_csr()
    assert A.raw.col_slices == 0 and not A.col_slices
    sag.csr_set_col_slices(A, True)
    assert A.col_slices and A.raw.col_slices == 1
    sag.csr_set_col_slices(A, False)
    assert not A.col_slices and A.raw.col_slices == 0


def test_tuner_leaves_ineligible_matrices_whole():
    A = fake_csr()
    sag.csr_set_col_slices(A, True)
    r = sag.csr_tune_col_slices(A, 100, torch.bfloat16)
    assert r == {"on": False, "whole_ms": None, "sliced_ms": None}
    assert not A.col_slices and A.raw.col_slices == 0


def test_workspace_does_not_depend_on_the_flag():
    lib = L.lib()
    A = L.SagCsr()
    A.n_rows, A.n_cols, A.nnz = 1000, 1000, 5000
    for d in (47, 100, 256, 1000):
        A.col_slices = 0
        a = lib.sag_spmm_workspace_bytes(ctypes.byref(A), d)
        A.col_slices = 1
        assert lib.sag_spmm_workspace_bytes(ctypes.byref(A), d) == a
