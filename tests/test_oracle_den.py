"""Pins of the oracle's error denominators (``layers.*_den`` and the GAT
bound).  Every GPU parity verdict divides by these, so an inflated one would
loosen every test; each is tied here to something other than itself:

* a dense brute force on graphs of at most 64 nodes: the normalised
  adjacency written out from its definition on a dense 0/1 matrix (degrees of
  A + I, D^-1/2 (A + I) D^-1/2 or the row mean), with the layer's expressions
  evaluated on absolute values by dense matrix products;
* the defining property of a magnitude bound: on non-negative inputs there is
  no cancellation, so the bound equals the value itself, and flipping the
  signs of the inputs leaves it unchanged.  Together these say den(x) equals
  the value function at |x|, whatever the oracle's own code for den is.

A planted factor of two on any denominator (or on the GAT score weight) fails
these checks; the last tests plant one and check that it is caught.  CPU
only."""
import numpy as np
import pytest

from helpers import dense_adjacency
from oracle import csr, gat, layers

RTOL = 1e-12


# ---- dense brute force of the normalised adjacency of a partition -----------------------

def _graph(seed, n=48, m=3, lo=6, hi=40):
    g = np.random.default_rng(seed)
    return g, g.integers(0, n, m * n), g.integers(0, n, m * n), n, lo, hi


def _dense_partition(src, dst, n, lo, hi, sym, loops, norm):
    """(dense normalised A of rows [lo, hi) over the columns [local | halo],
    halo ids): rows of the whole graph's dense matrix, columns picked in the
    remapped order.  The GCN column degree of a halo column is its degree in
    the whole graph (the oracle is called with deg_global = those)."""
    A = dense_adjacency(src, dst, n, symmetrize=sym)
    if loops:
        A = A + np.eye(n)
    deg = np.maximum(A.sum(axis=1), 1)
    if norm == "gcn":
        An = A / np.sqrt(np.outer(deg, deg))
    elif norm == "mean":
        An = A / deg[:, None]
    else:
        An = A
    rows = An[lo:hi]
    outside = [c for c in range(n) if not (lo <= c < hi) and np.any(A[lo:hi, c] != 0)]
    cols = list(range(lo, hi)) + outside
    deg_global = deg.astype(np.int32)
    return rows[:, cols], np.asarray(outside, np.int64), deg_global


def _build(seed, norm, sym=False, loops=True):
    g, src, dst, n, lo, hi = _graph(seed)
    Ad, halo, deg_global = _dense_partition(src, dst, n, lo, hi, sym, loops, norm)
    b = csr.build(src, dst, n, lo, hi, sym, loops, norm, deg_global=deg_global if norm == "gcn" else None)
    assert np.array_equal(b.halo_gid, halo)
    # the stored values are fp32: compare the dense matrix after the same rounding
    Ad = Ad.astype(np.float32).astype(np.float64)
    return g, b, Ad


def check_gcn_forward_den(seed):
    g, b, Ad = _build(seed, "gcn")
    H = g.standard_normal((b.A.n_cols, 5))
    W = g.standard_normal((5, 3))
    bias = g.standard_normal(3)
    Zd, Yd = layers.gcn_forward_den(b.A, H, W, bias)
    assert np.allclose(Zd, np.abs(Ad) @ np.abs(H), rtol=RTOL, atol=0)
    assert np.allclose(Yd, np.abs(Ad) @ np.abs(H) @ np.abs(W) + np.abs(bias), rtol=RTOL, atol=0)


def check_gcn_backward_den(seed):
    g, b, Ad = _build(seed, "gcn")
    n_l = b.n_local
    Z = g.standard_normal((n_l, 4))
    W = g.standard_normal((4, 3))
    Y = g.standard_normal((n_l, 3))
    G = g.standard_normal((n_l, 3))
    dWd, dbd, dZd, dHd = layers.gcn_backward_den(b.AT, Z, W, Y, True, G)
    GY = np.abs(G) * (Y > 0)
    assert np.allclose(dWd, np.abs(Z).T @ GY, rtol=RTOL, atol=0)
    assert np.allclose(dbd, GY.sum(axis=0), rtol=RTOL, atol=0)
    assert np.allclose(dZd, GY @ np.abs(W).T, rtol=RTOL, atol=0)
    assert np.allclose(dHd, np.abs(Ad).T @ (GY @ np.abs(W).T), rtol=RTOL, atol=0)


def check_sage_forward_den(seed):
    g, b, Ad = _build(seed, "mean", sym=True, loops=False)
    n_l = b.n_local
    H = g.standard_normal((b.A.n_cols, 4))
    W = g.standard_normal((8, 3))
    bias = g.standard_normal(3)
    Md, Yd = layers.sage_forward_den(b.A, H, n_l, W, bias)
    M_ref = np.abs(Ad) @ np.abs(H)
    assert np.allclose(Md, M_ref, rtol=RTOL, atol=0)
    want = np.abs(H[:n_l]) @ np.abs(W[:4]) + M_ref @ np.abs(W[4:]) + np.abs(bias)
    assert np.allclose(Yd, want, rtol=RTOL, atol=0)


def check_sage_backward_den(seed):
    g, b, Ad = _build(seed, "mean", sym=True, loops=True)
    n_l = b.n_local
    Hl = g.standard_normal((n_l, 4))
    M = g.standard_normal((n_l, 4))
    W = g.standard_normal((8, 3))
    Y = g.standard_normal((n_l, 3))
    G = g.standard_normal((n_l, 3))
    dWd, dbd, dHd = layers.sage_backward_den(b.AT, Hl, M, W, Y, True, G)
    GY = np.abs(G) * (Y > 0)
    X = np.abs(np.concatenate([Hl, M], axis=1))
    assert np.allclose(dWd, X.T @ GY, rtol=RTOL, atol=0)
    assert np.allclose(dbd, GY.sum(axis=0), rtol=RTOL, atol=0)
    dX = GY @ np.abs(W).T
    want = np.abs(Ad).T @ dX[:, 4:]
    want[:n_l] += dX[:, :4]
    assert np.allclose(dHd, want, rtol=RTOL, atol=0)


CHECKS = {"gcn_forward_den": check_gcn_forward_den, "gcn_backward_den": check_gcn_backward_den,
          "sage_forward_den": check_sage_forward_den, "sage_backward_den": check_sage_backward_den}


@pytest.mark.parametrize("name", sorted(CHECKS))
@pytest.mark.parametrize("seed", range(3))
def test_den_matches_dense_brute_force(name, seed):
    CHECKS[name](seed)


# ---- the magnitude-bound property: den(x) = value(|x|) ------------------------------------

def _random_signs(g, *xs):
    return [x * g.choice([-1.0, 1.0], size=np.shape(x)) for x in xs]


@pytest.mark.parametrize("seed", range(4))
def test_gcn_den_is_the_value_at_absolute_inputs(seed):
    g, src, dst, n, lo, hi = _graph(10 + seed)
    b = csr.build(src, dst, n, lo, hi, True, True, "gcn")
    Hp = np.abs(g.standard_normal((b.A.n_cols, 5)))
    Wp = np.abs(g.standard_normal((5, 3)))
    bp = np.abs(g.standard_normal(3))
    Gp = np.abs(g.standard_normal((b.n_local, 3)))
    Z, Y, _ = layers.gcn_forward(b.A, Hp, Wp, bp, False)
    dW, db, dZ, dH = layers.gcn_backward(b.AT, Z, Wp, Y, False, Gp)
    H, W, bias, G = _random_signs(g, Hp, Wp, bp, Gp)
    Zd, Yd = layers.gcn_forward_den(b.A, H, W, bias)
    assert np.allclose(Zd, Z, rtol=RTOL, atol=0) and np.allclose(Yd, Y, rtol=RTOL, atol=0)
    Zs = _random_signs(g, Z)[0]
    # no ReLU mask: every Y entry passes (a positive Y marks every entry live)
    dWd, dbd, dZd, dHd = layers.gcn_backward_den(b.AT, Zs, W, np.ones_like(Y), True, G)
    for got, want in ((dWd, dW), (dbd, db), (dZd, dZ), (dHd, dH)):
        assert np.allclose(got, want, rtol=RTOL, atol=0)


@pytest.mark.parametrize("seed", range(4))
def test_sage_den_is_the_value_at_absolute_inputs(seed):
    g, src, dst, n, lo, hi = _graph(20 + seed)
    b = csr.build(src, dst, n, lo, hi, True, False, "mean")
    n_l = b.n_local
    Hp = np.abs(g.standard_normal((b.A.n_cols, 4)))
    Wp = np.abs(g.standard_normal((8, 3)))
    bp = np.abs(g.standard_normal(3))
    Gp = np.abs(g.standard_normal((n_l, 3)))
    M, Y, _ = layers.sage_forward(b.A, Hp, n_l, Wp, bp, False)
    dW, db, dH = layers.sage_backward(b.AT, Hp[:n_l], M, Wp, Y, False, Gp)
    H, W, bias, G = _random_signs(g, Hp, Wp, bp, Gp)
    Md, Yd = layers.sage_forward_den(b.A, H, n_l, W, bias)
    assert np.allclose(Md, M, rtol=RTOL, atol=0) and np.allclose(Yd, Y, rtol=RTOL, atol=0)
    Ms = _random_signs(g, M)[0]
    dWd, dbd, dHd = layers.sage_backward_den(b.AT, H[:n_l], Ms, W, np.ones_like(Y), True, G)
    for got, want in ((dWd, dW), (dbd, db), (dHd, dH)):
        assert np.allclose(got, want, rtol=RTOL, atol=0)


@pytest.mark.parametrize("relu", [True, False])
def test_relu_mask_in_backward_den(relu):
    """Entries masked by the ReLU contribute nothing to the bound: a mask
    that kills a column of G_Y zeroes that column of dW's and db's bounds."""
    g, src, dst, n, lo, hi = _graph(31)
    b = csr.build(src, dst, n, lo, hi, True, True, "gcn")
    n_l = b.n_local
    Z = g.standard_normal((n_l, 4))
    W = g.standard_normal((4, 3))
    G = g.standard_normal((n_l, 3))
    Y = np.abs(g.standard_normal((n_l, 3))) + 0.1
    Y[:, 1] = -1.0
    dWd, dbd, _, _ = layers.gcn_backward_den(b.AT, Z, W, Y, relu, G)
    if relu:
        assert np.all(dWd[:, 1] == 0) and dbd[1] == 0
    else:
        assert np.all(dWd[:, 1] > 0) and dbd[1] > 0


# ---- GAT: the bound of the forward and backward, and the score weight -----------------------

def _gat_case(seed, heads=2, dh=3, d_in=5, lo=4, hi=30):
    g = np.random.default_rng(seed)
    n = 36
    src, dst = g.integers(0, n, 3 * n), g.integers(0, n, 3 * n)
    b = csr.build(src, dst, n, lo, hi, False, True, "none")
    A = b.A
    H = g.standard_normal((A.n_cols, d_in))
    W = g.standard_normal((d_in, heads * dh))
    a_src = g.standard_normal((heads, dh)) * 0.5
    a_dst = g.standard_normal((heads, dh)) * 0.5
    bias = g.standard_normal(heads * dh) * 0.1
    G = g.standard_normal((A.n_rows, heads * dh))
    return A, H, W, a_src, a_dst, bias, G


def _dense_alpha(A, alpha_h):
    P = np.zeros((A.n_rows, A.n_cols))
    P[A.row_ids(), A.indices] = alpha_h
    return P


def check_gat_den(seed, w, slope=0.2, relu=True):
    heads, dh = 2, 3
    A, H, W, a_src, a_dst, bias, G = _gat_case(seed, heads, dh)
    f = gat.gat_forward(A, H, W, a_src, a_dst, bias, heads, slope, relu)
    mask = A.row_ids(), A.indices
    HW = np.abs(H) @ np.abs(W)
    Wh = np.abs(f["Wh"])
    yd = np.zeros((A.n_rows, heads * dh))
    ad_dense = []
    for k in range(heads):
        cols = slice(k * dh, (k + 1) * dh)
        sr = HW[:A.n_rows, cols] @ np.abs(a_dst[k])      # target ends (local rows)
        sl = HW[:, cols] @ np.abs(a_src[k])               # source ends (all columns)
        S = sr[:, None] + sl[None, :] + np.abs(f["lse"][:, k])[:, None]
        P = _dense_alpha(A, f["alpha"][:, k])
        ad = np.where(P > 0, P * (1 + w * S), 0.0)
        ad_dense.append(ad)
        yd[:, cols] = ad @ Wh[:, cols]
    yd += np.abs(bias)
    got = gat.gat_forward_den(A, f, bias, heads, H, W, a_src, a_dst, w)
    assert np.allclose(got, yd, rtol=RTOL, atol=0)

    # backward bound, dense: the softmax derivative's difference becomes a sum
    GY = np.abs(G) * (f["Y"] > 0) if relu else np.abs(G)
    x = np.zeros((A.n_rows, A.n_cols, heads))
    x[mask[0], mask[1]] = f["x"]
    dlr = np.where(x > 0, 1.0, slope)
    der = np.zeros((A.n_rows, heads))
    dl = np.zeros((A.n_cols, heads))
    dWh = np.zeros((A.n_cols, heads * dh))
    for k in range(heads):
        cols = slice(k * dh, (k + 1) * dh)
        ad = ad_dense[k]
        dal = GY[:, cols] @ Wh[:, cols].T                  # |G_v| . |Wh_u| for every (v, u)
        t = (ad * dal).sum(axis=1)
        dx = ad * (dal + t[:, None]) * dlr[:, :, k]
        der[:, k] = dx.sum(axis=1)
        dl[:, k] = dx.sum(axis=0)
        dWh[:, cols] = ad.T @ GY[:, cols] + dl[:, k:k + 1] * np.abs(a_src[k])[None, :]
        dWh[:A.n_rows, cols] += der[:, k:k + 1] * np.abs(a_dst[k])[None, :]
    d = gat.gat_backward_den(A, H, W, a_src, a_dst, heads, slope, relu, f, f["Y"], G, w)
    W3 = Wh.reshape(A.n_cols, heads, dh)
    want = {"der": der, "dl": dl, "dWh": dWh, "db": GY.sum(axis=0),
            "da_src": np.einsum("uk,ukd->kd", dl, W3), "da_dst": np.einsum("vk,vkd->kd", der, W3[:A.n_rows]),
            "dW": np.abs(H).T @ dWh, "dH_ext": dWh @ np.abs(W).T}
    for k, v in want.items():
        assert np.allclose(d[k], v, rtol=RTOL, atol=0), k


@pytest.mark.parametrize("w", [0.0, 0.37])
@pytest.mark.parametrize("seed", range(3))
def test_gat_den_matches_dense_brute_force(seed, w):
    check_gat_den(seed, w)


def test_gat_score_magnitude_dense():
    """The score magnitude S_vu = |a_dst| . (|H||W|)_v + |a_src| . (|H||W|)_u
    + |lse_v| per entry and head, from dense per-entry loops."""
    heads, dh = 2, 3
    A, H, W, a_src, a_dst, bias, _ = _gat_case(5, heads, dh)
    f = gat.gat_forward(A, H, W, a_src, a_dst, bias, heads, 0.2, False)
    S = gat.score_magnitude(A, H, W, a_src, a_dst, heads, f["lse"])
    rows = A.row_ids()
    for e in range(0, A.nnz, 7):
        v, u = rows[e], A.indices[e]
        for k in range(heads):
            hv = sum(abs(H[v, i]) * abs(W[i, k * dh + j]) * abs(a_dst[k, j]) for i in range(H.shape[1])
                     for j in range(dh))
            hu = sum(abs(H[u, i]) * abs(W[i, k * dh + j]) * abs(a_src[k, j]) for i in range(H.shape[1])
                     for j in range(dh))
            assert abs(S[e, k] - (hv + hu + abs(f["lse"][v, k]))) <= 1e-12 * S[e, k]


# ---- planted inflations are caught -------------------------------------------------------

def _inflate(fn, which):
    """fn with output `which` (index, or dict key) multiplied by 2."""
    def wrapped(*a, **k):
        out = fn(*a, **k)
        if isinstance(out, dict):
            out = dict(out)
            out[which] = out[which] * 2
            return out
        if isinstance(out, tuple):
            out = list(out)
            out[which] = out[which] * 2
            return tuple(out)
        return out * 2
    return wrapped


@pytest.mark.parametrize("name,which", [
    ("gcn_forward_den", 0), ("gcn_forward_den", 1), ("gcn_backward_den", 0), ("gcn_backward_den", 1),
    ("gcn_backward_den", 3), ("sage_forward_den", 0), ("sage_forward_den", 1), ("sage_backward_den", 0),
    ("sage_backward_den", 1), ("sage_backward_den", 2)])
def test_planted_layer_inflation_fails(monkeypatch, name, which):
    monkeypatch.setattr(layers, name, _inflate(getattr(layers, name), which))
    with pytest.raises(AssertionError):
        CHECKS[name](0)


@pytest.mark.parametrize("which", ["dWh", "dH_ext", "dW", "da_src", "da_dst", "db"])
def test_planted_gat_backward_inflation_fails(monkeypatch, which):
    monkeypatch.setattr(gat, "gat_backward_den", _inflate(gat.gat_backward_den, which))
    with pytest.raises(AssertionError):
        check_gat_den(0, 0.37)


def test_planted_gat_forward_and_score_weight_inflation_fail(monkeypatch):
    orig = gat.gat_forward_den
    monkeypatch.setattr(gat, "gat_forward_den", _inflate(orig, None))
    with pytest.raises(AssertionError):
        check_gat_den(0, 0.0)
    monkeypatch.setattr(gat, "gat_forward_den", orig)
    # the score weight applied twice over: alpha (1 + 2 w S)
    monkeypatch.setattr(gat, "gat_forward_den",
                        lambda A, f, b, h, H, W, s, d, w=0.0: orig(A, f, b, h, H, W, s, d, 2 * w))
    with pytest.raises(AssertionError):
        check_gat_den(0, 0.37)
    monkeypatch.setattr(gat, "gat_forward_den", orig)
    sm = gat.score_magnitude
    monkeypatch.setattr(gat, "score_magnitude", lambda *a: 2 * sm(*a))
    with pytest.raises(AssertionError):
        check_gat_den(0, 0.37)
