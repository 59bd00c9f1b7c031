"""Pins of the oracle's SpMM: closed-form spectra, integer exactness against
dense brute force, the adjoint identity and the DIGEST partition split.
CPU only."""
import numpy as np
import pytest

import gen
from helpers import dense_adjacency
from oracle import csr, layers


def test_ring_stencil():
    """Cycle C_n + I: every degree is 3, so (A H)_i = (H_{i-1}+H_i+H_{i+1})/3."""
    n = 97
    src, dst = gen.ring_pairs(n)
    b = csr.build(src, dst, n, 0, n, True, True, "gcn")
    H = np.random.default_rng(0).standard_normal((n, 5))
    want = (np.roll(H, 1, 0) + H + np.roll(H, -1, 0)) / 3
    den = (np.roll(np.abs(H), 1, 0) + np.abs(H) + np.roll(np.abs(H), -1, 0)) / 3
    assert np.max(np.abs(layers.spmm(b.A, H) - want) / den) < 1e-7


@pytest.mark.parametrize("f", [0, 1, 5, 13])
def test_circulant_fourier_modes(f):
    """Circulant k=7 graph (offsets 1,2,3 and the antipode n/2) plus I: all
    degrees 8, entries 1/8 exactly; cos(2 pi f i / n) is an eigenvector with
    eigenvalue (1 + 2cos t + 2cos 2t + 2cos 3t + cos(pi f)) / 8, t = 2 pi f/n.
    The mean (no self-loops) of the ring has eigenvalue cos t."""
    n = 64
    src, dst = gen.circulant_pairs(n, [1, 2, 3, n // 2])
    b = csr.build(src, dst, n, 0, n, True, True, "gcn")
    assert np.all(b.A.values == np.float32(0.125))
    t = 2 * np.pi * f / n
    x = np.cos(t * np.arange(n))[:, None]
    lam = (1 + 2 * np.cos(t) + 2 * np.cos(2 * t) + 2 * np.cos(3 * t) + np.cos(np.pi * f)) / 8
    assert np.max(np.abs(layers.spmm(b.A, x) - lam * x)) < 1e-12
    rs, rd = gen.ring_pairs(n)
    bm = csr.build(rs, rd, n, 0, n, True, False, "mean")
    assert np.max(np.abs(layers.spmm(bm.A, x) - np.cos(t) * x)) < 1e-7


def test_integer_inputs_exact_vs_dense():
    """Entries 1/8 and small-integer H: every partial sum is exact, so the
    product equals dense brute force bit for bit."""
    n = 48
    src, dst = gen.random_regular_pairs(n, 7, np.random.default_rng(1))
    b = csr.build(src, dst, n, 0, n, True, True, "gcn")
    H = np.random.default_rng(2).integers(-8, 9, (n, 6)).astype(np.float64)
    A = (dense_adjacency(src, dst, n) + np.eye(n)) / 8
    assert np.array_equal(layers.spmm(b.A, H), A @ H)


def test_adjoint_identity():
    """<Y, A X> = <A^T Y, X> with A^T the oracle's transposed CSR."""
    g = np.random.default_rng(3)
    n = 400
    src = g.integers(0, n, 3000).astype(np.int32)
    dst = g.integers(0, n, 3000).astype(np.int32)
    b = csr.build(src, dst, n, 100, 250, False, True, "gcn")
    X = g.standard_normal((b.A.n_cols, 4))
    Y = g.standard_normal((b.A.n_rows, 4))
    lhs = np.sum(Y * layers.spmm(b.A, X))
    rhs = np.sum(layers.spmm(b.AT, Y) * X)
    assert abs(lhs - rhs) < 1e-11 * (1 + abs(lhs))


def test_partition_split_equals_full_graph():
    """DIGEST: P_m = P_in + P_out.  With the stale buffer equal to the fresh
    features, the 8 partitions' products reassemble the full-graph product
    exactly (integer inputs, 1/8 entries)."""
    w = gen.make_config(3, scale=1 / 256)
    src, dst = w.edges
    n = w.n_global
    full = csr.build(src, dst, n, 0, n, True, False, "mean")
    H = np.random.default_rng(4).integers(-4, 5, (n, 3)).astype(np.float64)
    ref = layers.spmm(full.A, H)
    parts = []
    for p in range(8):
        lo, hi = p * n // 8, (p + 1) * n // 8
        b = csr.build(src, dst, n, lo, hi, True, False, "mean")
        H_ext = np.concatenate([H[lo:hi], csr.gather(H, csr.halo_rows(b, 0))])
        parts.append(layers.spmm(b.A, H_ext))
    got = np.concatenate(parts)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)
    # the halo share of the first partition is near (n - n_l) / (n - 1)
    b0 = csr.build(src, dst, n, 0, n // 8, True, False, "mean")
    share = np.mean(b0.A.indices >= b0.n_local)
    assert abs(share - 7 / 8) < 0.05


def test_rows_subset_matches_full():
    g = np.random.default_rng(8)
    src, dst = g.integers(0, 300, 2000), g.integers(0, 300, 2000)
    b = csr.build(src, dst, 300, 0, 300, True, True, "gcn")
    X = g.standard_normal((300, 7))
    rows = np.array([5, 0, 299, 17])
    assert np.array_equal(layers.spmm(b.A, X, rows=rows), layers.spmm(b.A, X)[rows])


def test_fp32_instantiation_follows_the_fp64_loops():
    """The timing instantiation (float32 X) runs the same loops in fp32: it
    agrees with the fp64 product to fp32 rounding (at most len(row) ulps of
    the absolute-value sum), and exactly on small integers."""
    import numpy as np
    from oracle import csr, native
    g = np.random.default_rng(4)
    n = 700
    src, dst = g.integers(0, n, 9000), g.integers(0, n, 9000)
    b = csr.build(src, dst, n, 0, n, True, True, "gcn")
    X = g.standard_normal((n, 24))
    y64 = native.spmm(b.A.indptr, b.A.indices, b.A.values, X.astype(np.float32).astype(np.float64))
    y32 = native.spmm(b.A.indptr, b.A.indices, b.A.values, X.astype(np.float32))
    den = native.spmm(b.A.indptr, b.A.indices, b.A.values, np.abs(X.astype(np.float32).astype(np.float64)),
                      abs_mode=True)
    lens = np.diff(b.A.indptr)[:, None]
    assert y32.dtype == np.float32
    assert np.all(np.abs(y32 - y64) <= (lens + 1) * 2.0 ** -24 * den + 1e-30)
    Xi = g.integers(-8, 9, (n, 24)).astype(np.float32)
    ones = np.ones(b.A.nnz, np.float32)
    assert np.array_equal(native.spmm(b.A.indptr, b.A.indices, ones, Xi),
                          native.spmm(b.A.indptr, b.A.indices, ones, Xi.astype(np.float64)))
