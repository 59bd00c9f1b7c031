"""Pins of the oracle's GAT layer against facts outside it: a dense
brute-force evaluation of the attention on tiny graphs, the special cases
that reduce to other layers (zero attention vectors give the neighbourhood
mean; a slope of one makes the softmax blind to the target's score), the
concatenation of heads, exact bf16 storage of integer-valued products, and
central finite differences for every gradient.  CPU only."""
import numpy as np
import pytest

from helpers import dense_adjacency
from oracle import csr, gat, layers


def _graph(seed, n=36, lo=0, hi=None, sym=True, loops=True, m=3):
    g = np.random.default_rng(seed)
    src = g.integers(0, n, m * n)
    dst = g.integers(0, n, m * n)
    hi = n if hi is None else hi
    return g, src, dst, csr.build(src, dst, n, lo, hi, sym, loops, "none")


def _params(g, d_in, heads, dh, scale=1.0):
    W = g.standard_normal((d_in, heads * dh)) * scale
    a_src = g.standard_normal((heads, dh)) * 0.5
    a_dst = g.standard_normal((heads, dh)) * 0.5
    b = g.standard_normal(heads * dh) * 0.1
    return W, a_src, a_dst, b


@pytest.mark.parametrize("seed,heads,dh,slope", [(0, 1, 4, 0.2), (1, 3, 2, 0.2), (2, 2, 5, 0.01)])
def test_forward_dense_brute_force(seed, heads, dh, slope):
    """Full graph: per head a dense n x n score matrix masked to the edges
    (-inf elsewhere), softmax along each row, times the transformed rows."""
    g, src, dst, b = _graph(seed)
    n = b.A.n_rows
    H = g.standard_normal((n, 6))
    W, a_src, a_dst, bias = _params(g, 6, heads, dh)
    f = gat.gat_forward(b.A, H, W, a_src, a_dst, bias, heads, slope, True)
    adj = dense_adjacency(src, dst, n, symmetrize=True) + np.eye(n)
    want = []
    for k in range(heads):
        Wk = H @ W[:, k * dh:(k + 1) * dh]
        S = (Wk @ a_dst[k])[:, None] + (Wk @ a_src[k])[None, :]
        S = np.where(S > 0, S, slope * S)
        S = np.where(adj > 0, S, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        want.append(P @ Wk)
    Y = np.concatenate(want, axis=1) + bias
    assert np.allclose(f["Y"], Y, rtol=1e-12, atol=1e-12)
    assert np.array_equal(f["Out"], np.maximum(f["Y"], 0))
    # each row's weights sum to one and lse is the log normaliser
    sums = np.zeros((n, heads))
    np.add.at(sums, b.A.row_ids(), f["alpha"])
    assert np.allclose(sums, 1.0, rtol=0, atol=1e-13)


def test_zero_attention_is_the_neighbourhood_mean():
    """a_src = a_dst = 0: every score is 0, the weights are 1 / deg, and the
    layer is the GraphSAGE-mean aggregation of H W, i.e. mean-CSR H W + b."""
    g, src, dst, b = _graph(5, lo=4, hi=30, sym=False)
    bm = csr.build(src, dst, 36, 4, 30, False, True, "mean")
    H = g.standard_normal((b.A.n_cols, 7))
    W, _, _, bias = _params(g, 7, 2, 3)
    z = np.zeros((2, 3))
    f = gat.gat_forward(b.A, H, W, z, z, bias, 2, 0.2, True)
    _, Y, Out = layers.gcn_forward(bm.A, H, W, bias, True)
    assert np.allclose(f["Y"], Y, rtol=1e-6, atol=1e-6)   # mean values are fp32 in the CSR
    assert np.allclose(f["Out"], Out, rtol=1e-6, atol=1e-6)


def test_unit_slope_ignores_the_target_score():
    """slope = 1: e_vu = a_dst.Wh_v + a_src.Wh_u, and the row's shared first
    term cancels in the softmax, so a_dst does not change the output."""
    g, _, _, b = _graph(7, lo=3, hi=33, sym=False)
    H = g.standard_normal((b.A.n_cols, 5))
    W, a_src, a_dst, bias = _params(g, 5, 2, 4)
    f1 = gat.gat_forward(b.A, H, W, a_src, a_dst, bias, 2, 1.0, False)
    f2 = gat.gat_forward(b.A, H, W, a_src, 3.0 * g.standard_normal(a_dst.shape), bias, 2, 1.0, False)
    assert np.allclose(f1["Y"], f2["Y"], rtol=1e-12, atol=1e-12)
    # ... while with slope 0.2 it does
    f3 = gat.gat_forward(b.A, H, W, a_src, a_dst, bias, 2, 0.2, False)
    f4 = gat.gat_forward(b.A, H, W, a_src, -a_dst, bias, 2, 0.2, False)
    assert not np.allclose(f3["Y"], f4["Y"])


def test_heads_are_concatenated_single_head_layers():
    g, _, _, b = _graph(9, lo=0, hi=30)
    H = g.standard_normal((b.A.n_cols, 6))
    heads, dh = 3, 4
    W, a_src, a_dst, bias = _params(g, 6, heads, dh)
    f = gat.gat_forward(b.A, H, W, a_src, a_dst, bias, heads, 0.2, False)
    for k in range(heads):
        cols = slice(k * dh, (k + 1) * dh)
        fk = gat.gat_forward(b.A, H, W[:, cols], a_src[k:k + 1], a_dst[k:k + 1], bias[cols], 1, 0.2, False)
        assert np.allclose(f["Y"][:, cols], fk["Y"], rtol=1e-13, atol=1e-13)


def test_bf16_store_is_exact_for_small_integers():
    """Integer H and W with small products: Wh is a bf16 value already, so
    the bf16 storage model changes nothing."""
    g, _, _, b = _graph(11)
    H = g.integers(-3, 4, (b.A.n_cols, 5)).astype(np.float64)
    W = g.integers(-3, 4, (5, 8)).astype(np.float64)
    a = g.standard_normal((2, 4)) * 0.1
    f1 = gat.gat_forward(b.A, H, W, a, -a, None, 2, 0.2, False, store="f32")
    f2 = gat.gat_forward(b.A, H, W, a, -a, None, 2, 0.2, False, store="bf16")
    assert np.array_equal(f1["Y"], f2["Y"])
    # and a non-representable product is rounded to 8 significant bits
    f3 = gat.gat_forward(b.A, H, W / 3.0, a, -a, None, 2, 0.2, False, store="bf16")
    m, _ = np.frexp(f3["Wh"])
    assert np.array_equal(m * 256, np.rint(m * 256))


def _fd(f, P, dP, h=1e-6, tol=1e-6, k=20):
    flat = P.reshape(-1)
    idx = np.random.default_rng(1).choice(flat.size, min(k, flat.size), replace=False)
    for i in idx:
        old = flat[i]
        flat[i] = old + h
        fp = f()
        flat[i] = old - h
        fm = f()
        flat[i] = old
        num = (fp - fm) / (2 * h)
        ana = dP.reshape(-1)[i]
        assert abs(num - ana) <= tol * (1 + abs(ana)), (num, ana)


@pytest.mark.parametrize("relu,slope", [(False, 0.2), (True, 0.2), (False, 1.0)])
def test_backward_finite_differences(relu, slope):
    """Loss <G, Out> on a partition with halo rows: dH_ext (including the
    halo rows sent back to their owners), dW, da_src, da_dst and db by
    central differences."""
    g, _, _, b = _graph(13, n=40, lo=6, hi=30, sym=False, m=4)
    A = b.A
    heads, dh, d_in = 2, 3, 4
    H = g.standard_normal((A.n_cols, d_in))
    W, a_src, a_dst, bias = _params(g, d_in, heads, dh)
    G = g.standard_normal((A.n_rows, heads * dh))

    def loss():
        return float(np.sum(G * gat.gat_forward(A, H, W, a_src, a_dst, bias, heads, slope, relu)["Out"]))

    f = gat.gat_forward(A, H, W, a_src, a_dst, bias, heads, slope, relu)
    r = gat.gat_backward(A, H, W, a_src, a_dst, heads, slope, relu, f, f["Y"], G)
    for P, dP in [(H, r["dH_ext"]), (W, r["dW"]), (a_src, r["da_src"]), (a_dst, r["da_dst"]), (bias, r["db"])]:
        _fd(loss, P, dP)
    if slope == 1.0:
        # the target's score cancels: no gradient reaches a_dst
        assert np.allclose(r["da_dst"], 0, atol=1e-12)


def test_backward_den_bounds_terms():
    g, _, _, b = _graph(17, lo=2, hi=30, sym=False)
    A = b.A
    H = g.standard_normal((A.n_cols, 5))
    W, a_src, a_dst, bias = _params(g, 5, 2, 3)
    G = g.standard_normal((A.n_rows, 6))
    f = gat.gat_forward(A, H, W, a_src, a_dst, bias, 2, 0.2, True)
    r = gat.gat_backward(A, H, W, a_src, a_dst, 2, 0.2, True, f, f["Y"], G)
    d = gat.gat_backward_den(A, H, W, a_src, a_dst, 2, 0.2, True, f, f["Y"], G)
    for k in ("dWh", "da_src", "da_dst", "db", "dW", "dH_ext", "der", "dl"):
        assert np.all(np.abs(r[k]) <= d[k] * (1 + 1e-12) + 1e-300), k
    yd = gat.gat_forward_den(A, f, bias, 2, H, W, a_src, a_dst)
    assert np.all(np.abs(f["Y"]) <= yd * (1 + 1e-12))
