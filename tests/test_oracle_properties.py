"""Property tests of the oracle on random tiny graphs (hypothesis): any edge
list over at most 64 nodes -- empty rows, isolated nodes, repeated edges and
self-loops in the input included -- and any row range, with and without
symmetrisation and self connections, against dense brute force: the
structure and halo list, the full-graph GCN values D^-1/2 (A+I) D^-1/2 and
the mean values (symmetric graphs for GCN), and the SpMM against the dense
product.  CPU only."""
import numpy as np
from hypothesis import given, settings, strategies as st

from helpers import dense_adjacency, dense_structure
from oracle import csr, layers


@st.composite
def graphs(draw):
    n = draw(st.integers(1, 64))
    m = draw(st.integers(0, 3 * n))
    ids = st.integers(0, n - 1)
    src = np.array(draw(st.lists(ids, min_size=m, max_size=m)), dtype=np.int32)
    dst = np.array(draw(st.lists(ids, min_size=m, max_size=m)), dtype=np.int32)
    lo = draw(st.integers(0, n))
    hi = draw(st.integers(lo, n))
    return n, src, dst, lo, hi, draw(st.booleans()), draw(st.booleans())


@settings(max_examples=150, deadline=None)
@given(graphs())
def test_structure_and_halo(gr):
    n, src, dst, lo, hi, sym, loops = gr
    b = csr.build(src, dst, n, lo, hi, sym, loops, "gcn")
    rows, halo = dense_structure(src, dst, n, lo, hi, sym, loops)
    assert b.halo_gid.tolist() == halo
    assert b.A.indptr.tolist() == [0] + list(np.cumsum([len(r) for r in rows]))
    assert b.A.indices.tolist() == [c for r in rows for c in r]
    assert int(b.deg_row.sum()) == b.A.nnz


@settings(max_examples=150, deadline=None)
@given(graphs())
def test_full_graph_values_and_product(gr):
    n, src, dst, _, _, sym, loops = gr
    A = dense_adjacency(src, dst, n, symmetrize=sym) + (np.eye(n) if loops else 0)
    deg = A.sum(1)
    for norm in ("gcn", "mean"):
        b = csr.build(src, dst, n, 0, n, sym, loops, norm)
        if norm == "gcn":
            # symmetric graphs: row and column degrees coincide, so the closed
            # form is D^-1/2 (A+I) D^-1/2 with the row sums (directed graphs:
            # the structure only)
            d = np.where(deg > 0, 1 / np.sqrt(np.maximum(deg, 1)), 0.0)
            ref = d[:, None] * A * d[None, :] if sym else None
        else:
            ref = A / np.maximum(deg, 1)[:, None]
        dense = np.zeros((n, n))
        dense[b.A.row_ids(), b.A.indices] = b.A.values
        assert np.array_equal(dense != 0, A != 0)
        if ref is not None:
            assert np.allclose(dense, ref, rtol=6e-8, atol=0)
        x = np.random.default_rng(n).standard_normal((n, 3))
        y = layers.spmm(b.A, x)
        assert np.allclose(y, dense @ x, rtol=1e-12, atol=1e-12)
