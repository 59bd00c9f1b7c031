"""The binding's size checks (no GPU): the C ABI takes pointers and cannot
see tensor sizes, so the Python entry points refuse buffers with fewer rows
than the call would read or write, before anything reaches the library.
A stand-in CSR with only its row and column counts is enough, since the
checks run first."""
from types import SimpleNamespace

import pytest
import torch

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from sparse_aggregation_gemm_amd import ops  # noqa: E402

A = SimpleNamespace(n_rows=10, n_cols=15)      # 10 local rows, 5 halo columns
AT = SimpleNamespace(n_rows=15, n_cols=10)


def z(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def test_spmm_needs_every_column_row_of_x():
    with pytest.raises(ValueError, match="X has 12 rows; the call reads or writes 15"):
        sag.spmm_csr(A, z(12, 8))
    with pytest.raises(ValueError, match="Y has 9 rows"):
        sag.spmm_csr(A, z(15, 8), Y=z(9, 8))
    with pytest.raises(ValueError, match="X has 14 rows"):
        sag.spmm_csr_noalloc(A, z(14, 8), z(10, 8))


def test_layer_forward_needs_halo_rows():
    # a layer's input must hold its halo rows too (local rows only is the
    # mistake this guards against)
    for fwd in (sag.gcn_layer_forward, sag.sage_layer_forward):
        with pytest.raises(ValueError, match="H_ext .local . halo rows. has 10 rows"):
            fwd(A, z(10, 8), z(16, 4))
    with pytest.raises(ValueError, match="W has 8 rows; the call reads or writes 16"):
        sag.sage_layer_forward(A, z(15, 8), z(8, 4))
    with pytest.raises(ValueError, match="Out has 3 rows"):
        sag.gcn_layer_forward(A, z(15, 8), z(8, 4), Out=z(3, 4))
    with pytest.raises(ValueError, match="H_ext .local . halo rows. has 11 rows"):
        sag.aggregate_transform(A, z(11, 8), z(8, 4))
    with pytest.raises(ValueError, match="H_ext .local . halo rows. has 11 rows"):
        sag.gat_layer_forward(A, z(11, 8), z(8, 4), z(1, 4), z(1, 4))


def test_layer_backward_sizes():
    ctx = ops.LayerCtx("gcn", z(1), z(15, 8), z(8, 4), 8, 4, True)
    with pytest.raises(ValueError, match="G_out has 9 rows"):
        sag.gcn_layer_backward(ctx, AT, 10, z(10, 4), z(9, 4))
    with pytest.raises(ValueError, match="Y has 2 rows"):
        sag.gcn_layer_backward(ctx, AT, 10, z(2, 4), z(10, 4))
    with pytest.raises(ValueError, match="dH has 10 rows; the call reads or writes 15"):
        sag.gcn_layer_backward(ctx, AT, 10, z(10, 4), z(10, 4), dH=z(10, 8))
    short = ops.LayerCtx("sage", z(1), z(12, 8), z(16, 4), 8, 4, False)
    with pytest.raises(ValueError, match="H_ext has 12 rows"):
        sag.sage_layer_backward(short, AT, 10, None, z(10, 4))


def test_gather_push_and_gemm_sizes():
    with pytest.raises(ValueError, match="halo_gather out has 2 rows; the call reads or writes 3"):
        sag.halo_gather(z(6, 4), torch.tensor([0, 1, 2]), z(2, 4))
    with pytest.raises(ValueError, match="halo_push src has 1 rows"):
        sag.halo_push(z(1, 4), torch.tensor([0, 1]), z(6, 4))
    with pytest.raises(ValueError, match="gemm A2 has 5 rows; the call reads or writes 6"):
        sag.gemm(z(6, 4), z(8, 3), A2=z(5, 4))
    with pytest.raises(ValueError, match="gemm B .rows = K. has 7 rows"):
        sag.gemm(z(6, 4), z(7, 3), A2=z(6, 4))
    with pytest.raises(ValueError, match="gemm bias has 2 rows"):
        sag.gemm(z(6, 4), z(4, 3), bias=z(2))
    with pytest.raises(ValueError, match="gemm addend has 5 rows"):
        sag.gemm(z(6, 4), z(4, 3), addend=z(5, 3))
    with pytest.raises(ValueError, match="gemm_tn B has 5 rows"):
        sag.gemm_tn(z(6, 4), z(5, 3))


@pytest.mark.parametrize("nnz,want", [(0, 1024), (36_864, 1024), (7_918_846, 1024), (41_900_000, 1024),
                                      (50_000_000, 2048), (114_828_449, 4096), (126_150_500, 4096),
                                      (193_750_000, 4096), (3 * 10 ** 9, 4096)])
def test_auto_segment_length(nnz, want):
    """nnz / 32768 to the nearest power of two, within [1024, 4096]."""
    assert sag.auto_seg_len(SimpleNamespace(nnz=nnz)) == want
