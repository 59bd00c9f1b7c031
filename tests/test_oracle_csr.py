"""Pins of the oracle's CSR build: brute force, closed forms, invariants and
a hand-derived fixture.  CPU only."""
import json
import os

import numpy as np
import pytest

import gen
from helpers import closed_form, dense_structure, dense_adjacency
from oracle import csr, layers

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _random_edges(g, n, m, dup=True):
    src = g.integers(0, n, m).astype(np.int32)
    dst = g.integers(0, n, m).astype(np.int32)
    if dup:   # repeat some edges and add explicit self-loops
        k = m // 5
        src = np.concatenate([src, src[:k], np.arange(3, dtype=np.int32)])
        dst = np.concatenate([dst, dst[:k], np.arange(3, dtype=np.int32)])
    return src, dst


@pytest.mark.parametrize("seed", range(12))
def test_structure_matches_brute_force(seed):
    g = np.random.default_rng(seed)
    n = int(g.integers(5, 60))
    m = int(g.integers(0, 4 * n))
    src, dst = _random_edges(g, n, m)
    lo = int(g.integers(0, n))
    hi = int(g.integers(lo, n + 1))
    sym = bool(seed % 2)
    loops = bool((seed // 2) % 2)
    b = csr.build(src, dst, n, lo, hi, sym, loops, "gcn")
    rows, halo = dense_structure(src, dst, n, lo, hi, sym, loops)
    assert b.halo_gid.tolist() == halo
    assert b.A.indptr.tolist() == [0] + list(np.cumsum([len(r) for r in rows]))
    assert b.A.indices.tolist() == [c for r in rows for c in r]
    assert b.deg_row.tolist() == [len(r) for r in rows]
    # invariants: halo ids sorted, unique, outside the range
    assert np.all(np.diff(b.halo_gid) > 0)
    assert not np.any((b.halo_gid >= lo) & (b.halo_gid < hi))
    assert int(b.deg_row.sum()) == b.A.nnz


def test_golden_path3():
    fx = json.load(open(os.path.join(GOLD, "path3_gcn.json")))
    b = csr.build(fx["edges_src"], fx["edges_dst"], fx["n"], 0, fx["n"], True, True, "gcn")
    assert b.A.indptr.tolist() == fx["indptr"]
    assert b.A.indices.tolist() == fx["indices"]
    assert b.deg_row.tolist() == fx["degrees"]
    want = np.array([closed_form(e) for e in fx["values"]])
    assert np.allclose(b.A.values, want, rtol=6e-8, atol=0)
    H = np.array([[closed_form(e) for e in r] for r in fx["H"]])
    AH = np.array([[closed_form(e) for e in r] for r in fx["AH"]])
    assert np.allclose(layers.spmm(b.A, H), AH, rtol=2e-7, atol=0)
    bm = csr.build(fx["edges_src"], fx["edges_dst"], fx["n"], 0, fx["n"], True, True, "mean")
    assert np.allclose(bm.A.values, [closed_form(e) for e in fx["mean_values"]], rtol=6e-8)
    p = fx["partition"]
    bp = csr.build(fx["edges_src"], fx["edges_dst"], fx["n"], p["lo"], p["hi"], True, True, "gcn")
    assert bp.halo_gid.tolist() == p["halo_gid"]
    assert bp.A.indptr.tolist() == p["indptr"]
    assert bp.A.indices.tolist() == p["indices"]
    H_ext = np.concatenate([H[p["lo"]:p["hi"]], csr.gather(H, csr.halo_rows(bp, 0))])
    AHp = np.array([[closed_form(e) for e in r] for r in p["AH"]])
    assert np.allclose(layers.spmm(bp.A, H_ext), AHp, rtol=2e-7, atol=0)


@pytest.mark.parametrize("k", [1, 3, 7, 15, 31])
def test_regular_graph_row_sums_exactly_one(k):
    """k-regular: every degree of A+I is k+1, a power of two, so each entry
    is exactly 1/(k+1) and A 1 = 1 bit-exactly in any summation order."""
    n = 2 * (k + 1) + 10
    src, dst = gen.random_regular_pairs(n, k, np.random.default_rng(k))
    b = csr.build(src, dst, n, 0, n, True, True, "gcn")
    assert np.all(b.A.values == np.float32(1.0 / (k + 1)))
    ones = np.ones((n, 1))
    assert np.all(layers.spmm(b.A, ones) == 1.0)
    bm = csr.build(src, dst, n, 0, n, True, True, "mean")
    assert np.all(layers.spmm(bm.A, ones) == 1.0)


def test_sqrt_degree_is_eigenvector():
    """D^-1/2 (A+I) D^-1/2 maps D^1/2 1 to itself on any undirected graph
    (row r: sum_c (d_r d_c)^-1/2 d_c^1/2 = d_r / d_r^1/2).  Fails if the self
    connection is counted wrongly or the row degree is used twice."""
    g = np.random.default_rng(5)
    n = 300
    w = gen.power_law_weights(n, 12.0, 2.1, 40.0, g)
    src, dst = gen.chung_lu_pairs(n, 1500, w, g)
    b = csr.build(src, dst, n, 0, n, True, True, "gcn")
    s = np.sqrt(b.deg_row.astype(np.float64))[:, None]
    y = layers.spmm(b.A, s)
    assert np.max(np.abs(y - s) / s) < 1e-6


def test_mean_rows_sum_to_one():
    g = np.random.default_rng(6)
    src, dst = _random_edges(g, 200, 900)
    b = csr.build(src, dst, 200, 0, 200, False, False, "mean")
    y = layers.spmm(b.A, np.ones((200, 1)))[:, 0]
    nonempty = b.deg_row > 0
    assert np.all(np.abs(y[nonempty] - 1) < 1e-6 * b.deg_row[nonempty])
    assert np.all(y[~nonempty] == 0)


def test_values_match_dense_normalisation():
    """Full-graph values against the dense matrix form D^-1/2 (A+I) D^-1/2."""
    g = np.random.default_rng(7)
    n = 50
    src, dst = _random_edges(g, n, 150)
    b = csr.build(src, dst, n, 0, n, True, True, "gcn")
    A = dense_adjacency(src, dst, n) + np.eye(n)
    D = np.diag(1 / np.sqrt(A.sum(1)))
    An = D @ A @ D
    dense = np.zeros((n, n))
    dense[b.A.row_ids(), b.A.indices] = b.A.values
    assert np.allclose(dense, An, rtol=6e-8, atol=0)
    assert np.array_equal(dense != 0, A != 0)


@pytest.mark.parametrize("seed", range(4))
def test_transpose_invariants(seed):
    g = np.random.default_rng(100 + seed)
    n = 80
    src, dst = _random_edges(g, n, 300)
    b = csr.build(src, dst, n, 10, 50, False, True, "gcn", )
    # transpose twice gives the original
    tt = csr.transpose(b.AT)
    assert np.array_equal(tt.indptr, b.A.indptr)
    assert np.array_equal(tt.indices, b.A.indices)
    assert np.array_equal(tt.values, b.A.values)
    assert b.AT.n_rows == b.n_local + b.n_halo
    # rows of the transpose are ascending
    for r in range(b.AT.n_rows):
        seg = b.AT.indices[b.AT.indptr[r]:b.AT.indptr[r + 1]]
        assert np.all(np.diff(seg) > 0)
    # symmetric full graph: the transpose equals the matrix
    bs = csr.build(src, dst, n, 0, n, True, True, "gcn")
    assert np.array_equal(bs.AT.indices, bs.A.indices)
    assert np.array_equal(bs.AT.values, bs.A.values)


def test_halo_degrees_default_and_given():
    src, dst = gen.ring_pairs(12)
    b = csr.build(src, dst, 12, 0, 4, True, True, "gcn")
    # local rows 0..3 of the ring see halo nodes 11 (by 0) and 4 (by 3)
    assert b.halo_gid.tolist() == [4, 11]
    assert b.deg_col.tolist() == [3, 3, 3, 3, 2, 2]
    deg = np.full(12, 3, np.int32)
    bg = csr.build(src, dst, 12, 0, 4, True, True, "gcn", deg_global=deg)
    assert bg.deg_col.tolist() == [3] * 6
    assert np.all(bg.A.values == np.float32(1 / 3))


def test_first_config_edge_count():
    w = gen.make_config(1)
    src, dst = w.edges
    b = csr.build(src, dst, w.n_global, w.lo, w.hi, w.symmetrize, w.self_loops, w.norm)
    assert b.A.nnz == 36864 and b.n_halo == 0


def test_bad_inputs_raise():
    with pytest.raises(ValueError):
        csr.build([0], [5], 4, 0, 4, True, True, "gcn")
    with pytest.raises(ValueError):
        csr.build([0], [1], 4, 3, 2, True, True, "gcn")
    with pytest.raises(ValueError):
        csr.build([0], [1], 4, 0, 4, True, True, "sum")


def test_empty_graph():
    b = csr.build(np.zeros(0, np.int32), np.zeros(0, np.int32), 10, 2, 2, True, True, "gcn")
    assert b.A.n_rows == 0 and b.A.nnz == 0 and b.AT.n_rows == 0
    b = csr.build(np.zeros(0, np.int32), np.zeros(0, np.int32), 10, 0, 5, True, False, "mean")
    assert b.A.nnz == 0 and b.A.indptr.tolist() == [0] * 6


@pytest.mark.parametrize("seed", range(10))
def test_build_rows_matches_whole_build(seed):
    """The row-by-row build (used for checks at full size) gives the same
    entries and bit-identical values as the whole-partition build."""
    g = np.random.default_rng(500 + seed)
    n = int(g.integers(5, 90))
    src, dst = _random_edges(g, n, int(g.integers(0, 5 * n)))
    lo = int(g.integers(0, n))
    hi = int(g.integers(lo + 1, n + 1))
    sym, loops = bool(seed % 2), bool((seed // 2) % 2)
    norm = ("gcn", "mean", "none")[seed % 3]
    b = csr.build(src, dst, n, lo, hi, sym, loops, norm)
    rows = np.arange(lo, hi)
    got = csr.build_rows(src, dst, n, lo, hi, sym, loops, norm, rows)
    n_l = hi - lo
    halo = np.concatenate([b.halo_gid.astype(np.int64), [0]])
    for i, (cols, vals) in enumerate(got):
        s, e = b.A.indptr[i], b.A.indptr[i + 1]
        c = b.A.indices[s:e].astype(np.int64)
        glob = np.where(c < n_l, c + lo, halo[np.clip(c - n_l, 0, halo.size - 1)])
        order = np.argsort(glob)
        assert np.array_equal(glob[order], cols)
        assert np.array_equal(b.A.values[s:e][order].view(np.uint32), vals.view(np.uint32))
