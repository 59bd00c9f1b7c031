"""Oracle graph-attention (GAT) layer, forward and backward, in float64 (test
infrastructure only).

Definitions followed
--------------------
The pages name GAT (Velickovic et al., 2018) as one of the models the
partitioned training serves (Sylvie, first section; its results table; the
DIGEST evaluation section) but print none of its formulas, so the layer is
the textbook one from that paper, on one partition:

* Wh = H_ext W, viewed per head k as Wh_k (width d_head); heads are laid out
  side by side, head k in columns [k d_head, (k + 1) d_head).
* Score of the entry (v, u) of A (v a local row, u a column of [local | halo]):
  x_vu = a_dst_k . Wh_k[v] + a_src_k . Wh_k[u], e_vu = LeakyReLU(x_vu) with
  negative slope `slope` (0.2 in the paper).  The paper's attention vector
  a = [a_1 | a_2] acts on [W h_v | W h_u]; a_dst is a_1, a_src is a_2.
* alpha_vu = softmax of e_v. over the entries of row v (the neighbourhood
  includes v itself when A has self connections).
* Agg_k[v] = sum_u alpha_vu Wh_k[u]; heads concatenated; Y = Agg + b;
  Out = ReLU(Y) when asked.
* Backward: the chain rule through the same steps (softmax derivative
  alpha (g - sum_u alpha g), LeakyReLU' = 1 where x > 0, else `slope`).

Readings
--------
* Bias and ReLU are the same affine-update epilogue as the other layers
  (the GAT paper uses ELU between layers; the pages fix no activation).
* The halo rows enter exactly as in the GCN layer: H_ext holds the recovered
  stale rows, and the transform is applied after the pull.
* ``store="bf16"`` models the storage of Wh (and of the gradient dWh that the
  two backward products read) in bfloat16 (nearest, ties to even); all other
  arithmetic is float64.

``*_den`` functions evaluate the same expressions on absolute values (alpha
is already positive); they bound the magnitude of every term summed into an
output and serve as the denominator of a relative error.
"""
from __future__ import annotations

import numpy as np
import scipy.sparse as sp

from .csr import CSR
from .layers import round_bf16


def _heads(x, heads):
    n, f = x.shape
    return x.reshape(n, heads, f // heads)


def _lrelu(x, slope):
    return np.where(x > 0, x, slope * x)


def _dlrelu(x, slope):
    return np.where(x > 0, 1.0, slope)


def _alpha_matrix(A: CSR, alpha_h):
    """Sparse matrix of one head's attention weights on A's pattern."""
    return sp.csr_matrix((alpha_h, A.indices.astype(np.int64), A.indptr), shape=(A.n_rows, A.n_cols))


def scores(A: CSR, Wh, a_src, a_dst, heads: int, slope: float):
    """el [n_ext, heads], er [n_ext, heads], x and e per entry [nnz, heads]."""
    W3 = _heads(Wh, heads)
    el = np.einsum("nkd,kd->nk", W3, np.asarray(a_src, np.float64).reshape(heads, -1))
    er = np.einsum("nkd,kd->nk", W3, np.asarray(a_dst, np.float64).reshape(heads, -1))
    rows = A.row_ids()
    x = er[rows] + el[A.indices]
    return el, er, x, _lrelu(x, slope)


def softmax_rows(A: CSR, e):
    """alpha [nnz, heads] and the log of each row's normaliser lse [n_rows,
    heads] (max + log sum exp(e - max)); rows without entries get -inf."""
    rows = A.row_ids()
    n, heads = A.n_rows, e.shape[1]
    m = np.full((n, heads), -np.inf)
    np.maximum.at(m, rows, e)
    p = np.exp(e - m[rows])
    s = np.zeros((n, heads))
    np.add.at(s, rows, p)
    with np.errstate(divide="ignore"):
        lse = m + np.log(s)
    return p / s[rows], lse


def gat_forward(A: CSR, H_ext, W, a_src, a_dst, b, heads: int, slope: float, relu: bool,
                store: str = "f32"):
    """Returns a dict with Wh, el, er, alpha, lse, Agg, Y and Out."""
    Wh = np.asarray(H_ext, np.float64) @ np.asarray(W, np.float64)
    if store == "bf16":
        Wh = round_bf16(Wh)
    el, er, x, e = scores(A, Wh, a_src, a_dst, heads, slope)
    alpha, lse = softmax_rows(A, e)
    W3 = _heads(Wh, heads)
    Agg = np.concatenate([_alpha_matrix(A, alpha[:, k]) @ W3[:, k, :] for k in range(heads)], axis=1)
    Y = Agg + (0.0 if b is None else np.asarray(b, np.float64))
    Out = np.maximum(Y, 0.0) if relu else Y
    return dict(Wh=Wh, el=el, er=er, x=x, alpha=alpha, lse=lse, Agg=Agg, Y=Y, Out=Out)


def score_magnitude(A: CSR, H_ext, W, a_src, a_dst, heads: int, lse):
    """Per entry and head, the magnitude of the terms summed into the
    exponent of alpha_vu: the score on absolute values (|a| . (|H| |W|) for
    both ends, which also bounds the transform's own terms) plus |lse_v|.
    A relative perturbation eps of those terms moves alpha_vu by a factor
    of about 1 + eps * (this magnitude)."""
    HW = np.abs(np.asarray(H_ext, np.float64)) @ np.abs(np.asarray(W, np.float64))
    H3 = _heads(HW, heads)
    sl = np.einsum("nkd,kd->nk", H3, np.abs(np.asarray(a_src, np.float64)).reshape(heads, -1))
    sr = np.einsum("nkd,kd->nk", H3, np.abs(np.asarray(a_dst, np.float64)).reshape(heads, -1))
    rows = A.row_ids()
    return sr[rows] + sl[A.indices] + np.abs(lse[rows])


def gat_forward_den(A: CSR, fwd: dict, b, heads: int, H_ext, W, a_src, a_dst, score_weight: float = 0.0):
    """Magnitude bound of Y: sum_u alpha_vu (1 + w S_vu) |Wh_u| + |b|, S the
    score magnitude and w = score_weight.  With w = 0 it is the plain
    magnitude of the summed terms; a caller that allows a relative error
    tol adds the rounding of the weights' exponent (absolute error about
    n eps S for n-term fp32 sums) with w = n eps / tol."""
    W3 = np.abs(_heads(fwd["Wh"], heads))
    ad = fwd["alpha"] * (1.0 + score_weight * score_magnitude(A, H_ext, W, a_src, a_dst, heads, fwd["lse"]))
    Aggd = np.concatenate([_alpha_matrix(A, ad[:, k]) @ W3[:, k, :] for k in range(heads)], axis=1)
    return Aggd + (0.0 if b is None else np.abs(np.asarray(b, np.float64)))


def _edge_dot(A: CSR, Gv, Wu, heads, chunk=1 << 16):
    """[nnz, heads]: per entry (v, u) and head, Gv_k[v] . Wu_k[u]."""
    rows = A.row_ids()
    G3, W3 = _heads(Gv, heads), _heads(Wu, heads)
    out = np.empty((A.nnz, heads))
    for s in range(0, A.nnz, chunk):
        r, c = rows[s:s + chunk], A.indices[s:s + chunk]
        out[s:s + chunk] = np.einsum("ekd,ekd->ek", G3[r], W3[c])
    return out


def gat_backward(A: CSR, H_ext, W, a_src, a_dst, heads: int, slope: float, relu: bool, fwd: dict,
                 Ymask, G, store: str = "f32"):
    """Gradients of <G, Out>: dict with GY, dalpha, de, der, del, dWh (before
    storage rounding), da_src, da_dst, db, dW and dH_ext.  Ymask is the Y
    whose sign gives the ReLU mask."""
    n_l, n_ext = A.n_rows, A.n_cols
    rows = A.row_ids()
    alpha, x, Wh = fwd["alpha"], fwd["x"], fwd["Wh"]
    G = np.asarray(G, np.float64)
    GY = G * (np.asarray(Ymask) > 0) if relu else G
    dalpha = _edge_dot(A, GY, Wh, heads)
    t = np.zeros((n_l, heads))
    np.add.at(t, rows, alpha * dalpha)
    de = alpha * (dalpha - t[rows])
    dx = de * _dlrelu(x, slope)
    der = np.zeros((n_l, heads))
    np.add.at(der, rows, dx)
    dl = np.zeros((n_ext, heads))
    np.add.at(dl, A.indices, dx)
    G3 = _heads(GY, heads)
    dWh3 = np.stack([_alpha_matrix(A, alpha[:, k]).T @ G3[:, k, :] for k in range(heads)], axis=1)
    asrc = np.asarray(a_src, np.float64).reshape(heads, -1)
    adst = np.asarray(a_dst, np.float64).reshape(heads, -1)
    dWh3 = dWh3 + dl[:, :, None] * asrc[None]
    dWh3[:n_l] += der[:, :, None] * adst[None]
    W3 = _heads(Wh, heads)
    da_src = np.einsum("uk,ukd->kd", dl, W3)
    da_dst = np.einsum("vk,vkd->kd", der, W3[:n_l])
    dWh = dWh3.reshape(n_ext, -1)
    dWh_st = round_bf16(dWh) if store == "bf16" else dWh
    W = np.asarray(W, np.float64)
    return dict(GY=GY, dalpha=dalpha, de=de, der=der, dl=dl, dWh=dWh, da_src=da_src, da_dst=da_dst,
                db=GY.sum(axis=0), dW=np.asarray(H_ext, np.float64).T @ dWh_st, dH_ext=dWh_st @ W.T)


def gat_backward_den(A: CSR, H_ext, W, a_src, a_dst, heads: int, slope: float, relu: bool, fwd: dict,
                     Ymask, G, score_weight: float = 0.0):
    """The backward expressions on absolute values (the softmax derivative's
    difference becomes a sum), with alpha scaled by 1 + w S as in the
    forward bound."""
    n_l, n_ext = A.n_rows, A.n_cols
    rows = A.row_ids()
    x, Wh = fwd["x"], np.abs(fwd["Wh"])
    alpha = fwd["alpha"] * (1.0 + score_weight * score_magnitude(A, H_ext, W, a_src, a_dst, heads, fwd["lse"]))
    G = np.abs(np.asarray(G, np.float64))
    GY = G * (np.asarray(Ymask) > 0) if relu else G
    dalpha = _edge_dot(A, GY, Wh, heads)
    t = np.zeros((n_l, heads))
    np.add.at(t, rows, alpha * dalpha)
    dx = alpha * (dalpha + t[rows]) * _dlrelu(x, slope)
    der = np.zeros((n_l, heads))
    np.add.at(der, rows, dx)
    dl = np.zeros((n_ext, heads))
    np.add.at(dl, A.indices, dx)
    G3 = _heads(GY, heads)
    dWh3 = np.stack([_alpha_matrix(A, alpha[:, k]).T @ G3[:, k, :] for k in range(heads)], axis=1)
    asrc = np.abs(np.asarray(a_src, np.float64)).reshape(heads, -1)
    adst = np.abs(np.asarray(a_dst, np.float64)).reshape(heads, -1)
    dWh3 = dWh3 + dl[:, :, None] * asrc[None]
    dWh3[:n_l] += der[:, :, None] * adst[None]
    W3 = _heads(Wh, heads)
    dWh = dWh3.reshape(n_ext, -1)
    Wa = np.abs(np.asarray(W, np.float64))
    return dict(der=der, dl=dl, dWh=dWh, da_src=np.einsum("uk,ukd->kd", dl, W3),
                da_dst=np.einsum("vk,vkd->kd", der, W3[:n_l]), db=GY.sum(axis=0),
                dW=np.abs(np.asarray(H_ext, np.float64)).T @ dWh, dH_ext=dWh @ Wa.T)
