"""Pins of the oracle's layers: dense brute force forward, central finite
differences for the backward, GEMM special cases and bf16 rounding.
CPU only."""
import numpy as np
import pytest

from helpers import dense_adjacency
from oracle import csr, layers


def _tiny(seed, n=40, lo=8, hi=30, sym=True):
    g = np.random.default_rng(seed)
    src = g.integers(0, n, 3 * n)
    dst = g.integers(0, n, 3 * n)
    return g, src, dst, n, lo, hi, sym


def _dense_norm(src, dst, n, sym, kind):
    A = dense_adjacency(src, dst, n, symmetrize=sym) + np.eye(n)
    if kind == "gcn":
        d = A.sum(1)
        return A / np.sqrt(np.outer(d, d))
    return A / A.sum(1, keepdims=True)


@pytest.mark.parametrize("seed", range(3))
def test_gcn_forward_dense_brute_force(seed):
    """Full graph, all rows local: relu(A_norm H W + b) with a dense A_norm."""
    g, src, dst, n, _, _, sym = _tiny(seed)
    b = csr.build(src, dst, n, 0, n, sym, True, "gcn")
    H = g.standard_normal((n, 5))
    W = g.standard_normal((5, 3))
    bias = g.standard_normal(3)
    _, Y, Out = layers.gcn_forward(b.A, H, W, bias, True)
    An = _dense_norm(src, dst, n, sym, "gcn")
    Yd = An @ H @ W + bias
    assert np.allclose(Y, Yd, rtol=1e-6, atol=1e-6)
    assert np.array_equal(Out, np.maximum(Y, 0))


@pytest.mark.parametrize("seed", range(3))
def test_sage_forward_dense_brute_force(seed):
    g, src, dst, n, _, _, sym = _tiny(seed)
    b = csr.build(src, dst, n, 0, n, sym, True, "mean")
    H = g.standard_normal((n, 4))
    W = g.standard_normal((8, 3))
    bias = g.standard_normal(3)
    M, Y, _ = layers.sage_forward(b.A, H, n, W, bias, False)
    Am = _dense_norm(src, dst, n, sym, "mean")
    Yd = H @ W[:4] + (Am @ H) @ W[4:] + bias
    assert np.allclose(Y, Yd, rtol=1e-6, atol=1e-6)


def _fd_check(f, params, grads, h=1e-6, tol=1e-6):
    """Central differences of the scalar f() against analytic grads."""
    for P, dP in zip(params, grads):
        flat = P.reshape(-1)
        idx = np.random.default_rng(0).choice(flat.size, min(25, flat.size), replace=False)
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


@pytest.mark.parametrize("relu", [True, False])
def test_gcn_backward_finite_differences(relu):
    """Loss <G, Out> on a partition with halo rows: dW, db and dH_ext
    (including the halo rows that would be sent back) by central
    differences."""
    g, src, dst, n, lo, hi, _ = _tiny(11, sym=False)
    b = csr.build(src, dst, n, lo, hi, False, True, "gcn")
    H = g.standard_normal((b.A.n_cols, 4))
    W = g.standard_normal((4, 3))
    bias = g.standard_normal(3)
    G = g.standard_normal((b.n_local, 3))

    def loss():
        return np.sum(G * layers.gcn_forward(b.A, H, W, bias, relu)[2])

    Z, Y, _ = layers.gcn_forward(b.A, H, W, bias, relu)
    dW, db, _, dH = layers.gcn_backward(b.AT, Z, W, Y, relu, G)
    _fd_check(loss, [W, bias, H], [dW, db, dH])


@pytest.mark.parametrize("relu", [True, False])
def test_sage_backward_finite_differences(relu):
    g, src, dst, n, lo, hi, _ = _tiny(12, sym=True)
    b = csr.build(src, dst, n, lo, hi, True, False, "mean")
    H = g.standard_normal((b.A.n_cols, 3))
    W = g.standard_normal((6, 4))
    bias = g.standard_normal(4)
    G = g.standard_normal((b.n_local, 4))
    nl = b.n_local

    def loss():
        return np.sum(G * layers.sage_forward(b.A, H, nl, W, bias, relu)[2])

    M, Y, _ = layers.sage_forward(b.A, H, nl, W, bias, relu)
    dW, db, dH = layers.sage_backward(b.AT, H[:nl], M, W, Y, relu, G)
    _fd_check(loss, [W, bias, H], [dW, db, dH])


def test_identity_and_permutation_weights():
    g, src, dst, n, _, _, sym = _tiny(3)
    b = csr.build(src, dst, n, 0, n, sym, True, "gcn")
    H = g.standard_normal((n, 5))
    bias = g.standard_normal(5)
    Z, Y, _ = layers.gcn_forward(b.A, H, np.eye(5), bias, False)
    assert np.array_equal(Y, Z + bias)
    P = np.eye(5)[[3, 0, 4, 1, 2]]
    _, Yp, _ = layers.gcn_forward(b.A, H, P, None, False)
    assert np.array_equal(Yp, Z[:, [1, 3, 4, 0, 2]])


def test_small_integer_layer_exact():
    """Integer H and W with 1/8 entries: the oracle's layer equals a Python
    triple loop exactly."""
    import gen
    n = 32
    src, dst = gen.random_regular_pairs(n, 7, np.random.default_rng(9))
    b = csr.build(src, dst, n, 0, n, True, True, "gcn")
    g = np.random.default_rng(10)
    H = g.integers(-3, 4, (n, 4)).astype(np.float64)
    W = g.integers(-3, 4, (4, 3)).astype(np.float64)
    _, Y, _ = layers.gcn_forward(b.A, H, W, None, False)
    A = (dense_adjacency(src, dst, n) + np.eye(n)) / 8
    Z = [[sum(A[i, k] * H[k, j] for k in range(n)) for j in range(4)] for i in range(n)]
    Yl = [[sum(Z[i][k] * W[k, j] for k in range(4)) for j in range(3)] for i in range(n)]
    assert np.array_equal(Y, np.array(Yl))


def test_round_bf16_known_values():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties to even gives 1
    assert layers.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6; even mantissa is 1+2^-6
    assert layers.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    assert layers.round_bf16(np.array([1 + 2 ** -8 + 2 ** -20]))[0] == 1 + 2 ** -7
    assert layers.round_bf16(np.array([-3.0, 0.0, 255.0, 257.0]))[0:3].tolist() == [-3.0, 0.0, 255.0]
    assert layers.round_bf16(np.array([257.0]))[0] == 256.0
    x = np.random.default_rng(0).standard_normal(1000)
    r = layers.round_bf16(x)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8)
    # idempotent, and bf16 values survive the fp32 bit view
    assert np.array_equal(layers.round_bf16(r), r)
    bits = (r.astype(np.float32).view(np.uint32) & 0xFFFF)
    assert np.all(bits == 0)
