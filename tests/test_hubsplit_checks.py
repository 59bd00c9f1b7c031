"""Host-side checks of hub splits (no GPU): a matrix whose hub_part and
cold_part do not form a valid split is refused before anything is launched,
as is a split of a matrix that already has one; and the binding's rule for
when a split pays.  The CSRs are stand-ins whose device pointers are never
dereferenced, since every check runs first."""
import ctypes
from types import SimpleNamespace

import pytest

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from sparse_aggregation_gemm_amd import _lib as L  # noqa: E402

FAKE = 1 << 20   # 16-B aligned stand-in addresses, never read


def csr(n_rows, n_cols, nnz, values=True, row_mean=0):
    c = L.SagCsr()
    c.n_rows, c.n_cols, c.nnz = n_rows, n_cols, nnz
    c.indptr, c.indices = FAKE, 2 * FAKE
    c.values = 3 * FAKE if values else None
    c.row_mean = row_mean
    return c


def attach(A, hub, cold):
    A.hub_part = ctypes.addressof(hub) if hub is not None else None
    A.cold_part = ctypes.addressof(cold) if cold is not None else None


def spmm(A):
    lib = L.lib()
    st = lib.sag_spmm_csr(ctypes.byref(A), 4 * FAKE, 16, L.SAG_F32, 16, 5 * FAKE, 16, L.SAG_F32, None, 0, 0,
                          None, 0, None)
    return st, lib.sag_last_error().decode()


def test_split_needs_both_parts():
    A, h = csr(10, 20, 30), csr(10, 20, 12)
    attach(A, h, None)
    st, msg = spmm(A)
    assert st == L.SAG_E_INVALID and "both parts" in msg


@pytest.mark.parametrize("bad", ["shape", "entries", "row_mean", "values", "nested"])
def test_inconsistent_parts_refused(bad):
    A = csr(10, 20, 30)
    h, c = csr(10, 20, 12), csr(10, 20, 18)
    inner_h, inner_c = csr(10, 20, 5), csr(10, 20, 7)
    if bad == "shape":
        c = csr(11, 20, 18)
    elif bad == "entries":
        c = csr(10, 20, 17)
    elif bad == "row_mean":
        h = csr(10, 20, 12, row_mean=1)
    elif bad == "values":
        c = csr(10, 20, 18, values=False)
    elif bad == "nested":
        attach(h, inner_h, inner_c)
    attach(A, h, c)
    st, msg = spmm(A)
    want = {"shape": "shape", "entries": "entries", "row_mean": "row_mean 0", "values": "carry them",
            "nested": "has a split"}[bad]
    assert st == L.SAG_E_INVALID and want in msg, msg


def test_row_mean_split_needs_stored_values():
    A = csr(10, 20, 30, values=False, row_mean=1)
    h, c = csr(10, 20, 12, values=False), csr(10, 20, 18, values=False)
    attach(A, h, c)
    st, msg = spmm(A)
    assert st == L.SAG_E_INVALID and "store its values" in msg


def test_split_of_a_split_matrix_and_bad_hub_count_refused():
    lib = L.lib()
    A = csr(10, 20, 30)
    h, c = csr(10, 20, 12), csr(10, 20, 18)
    attach(A, h, c)
    nh = ctypes.c_int64(-1)
    st = lib.sag_csr_hub_split(ctypes.byref(A), 4, 30, FAKE, FAKE, FAKE, 30, FAKE, FAKE, FAKE, ctypes.byref(nh),
                               FAKE, 1 << 30, None)
    assert st == L.SAG_E_INVALID and "already has a split" in lib.sag_last_error().decode()
    B = csr(10, 20, 30)
    st = lib.sag_csr_hub_split(ctypes.byref(B), 0, 30, FAKE, FAKE, FAKE, 30, FAKE, FAKE, FAKE, ctypes.byref(nh),
                               FAKE, 1 << 30, None)
    assert st == L.SAG_E_INVALID and "n_hub" in lib.sag_last_error().decode()


def test_split_pays_rule():
    rule = sag.hub_split_pays
    # the dense power-law graph (493 entries per row) splits; the large
    # sparse graph (51 per row) and small matrices do not
    assert rule(SimpleNamespace(n_rows=232_965, n_cols=232_965, nnz=114_828_449))
    assert not rule(SimpleNamespace(n_rows=2_450_000, n_cols=2_450_000, nnz=126_150_500))
    assert not rule(SimpleNamespace(n_rows=900, n_cols=900, nnz=400_000))
    assert not rule(SimpleNamespace(n_rows=0, n_cols=0, nnz=0))


def test_chain_arguments_and_counts():
    """The binding refuses a depth below one and a second split of a split
    matrix before calling the library; hub_chain lists the entry counts of
    the hub parts, then of the final cold part."""
    with pytest.raises(ValueError, match="levels"):
        sag.csr_hub_split(SimpleNamespace(hub_part=None), levels=0)
    with pytest.raises(ValueError, match="already has a hub split"):
        sag.csr_hub_split(SimpleNamespace(hub_part=object()))
    last = SimpleNamespace(hub_part=None, nnz=5)
    mid = SimpleNamespace(hub_part=SimpleNamespace(nnz=7), cold_part=last)
    top = SimpleNamespace(hub_part=SimpleNamespace(nnz=30), cold_part=mid)
    assert sag.hub_chain(top) == [30, 7, 5]
    assert sag.hub_chain(last) == []
