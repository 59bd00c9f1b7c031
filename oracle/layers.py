"""Oracle GNN layers, forward and backward, in float64 (test infrastructure).

Definitions followed
--------------------
* GCN layer: H' = sigma(A^T H W) with the normalised adjacency (CAGNET page,
  forward-propagation equation; Sylvie, "Forward Propagation": the matrix form
  of the aggregate and update steps on the concatenation of local rows and
  recovered halo rows).  On a partition the input is H_ext = [H_in ; H~_out]
  and the product is P_in H_in + P_out H~_out (DIGEST, matrix form of the
  modified forward pass), i.e. one SpMM over the remapped columns.
* GraphSAGE-mean layer: the aggregate z_v is the mean of the neighbours'
  rows, and the update takes it together with the node's own row (Sylvie,
  first paragraph).  Reading: Y = [h_v | z_v] W + b, self first, then sigma.
* Backward (CAGNET page: backpropagation uses the same primitives;
  Sylvie, "Backward Propagation": halo rows of the input gradient are what a
  partition sends back; DIGEST: the weight gradient depends on the stale
  rows): G_Y = G_out * 1[Y > 0] (ReLU'(0) = 0); dW = X^T G_Y; db = sum of
  G_Y's rows; dX = G_Y W^T; dH_ext = A_norm^T dZ over the transposed CSR.

Readings
--------
* The bias b and the ReLU flag are per layer; the pages show sigma but no
  bias.  The bias comes from the layer's affine update.
* Aggregation comes first ((A H) W); the GPU may associate differently.
* ``round_bf16`` models storage of an activation in bfloat16 (round to the
  nearest value with 8 significant bits, ties to even) where a bf16 path
  stores one between layers.  Subnormal bf16 values are not modelled.

The layers compute in the floating type of their input H (float64 for every
parity check; float32 only when the oracle is timed as a CPU baseline).

``*_den`` functions evaluate the same expressions on absolute values; the
result bounds the magnitude of every term summed into an output and serves as
the denominator of the relative error of a floating-point result.
"""
from __future__ import annotations

import numpy as np

from . import native
from .csr import CSR


def as_f64(x, dtype: str) -> np.ndarray:
    """Stored values (fp32 array or bf16 bit patterns) as exact float64."""
    x = np.asarray(x)
    if dtype == "bf16":
        return (x.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (8 significant
    bits, ties to even), returned as float64."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                 # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def spmm(A: CSR, X: np.ndarray, abs_mode: bool = False, rows=None) -> np.ndarray:
    return native.spmm(A.indptr, A.indices, A.values, X, abs_mode=abs_mode, rows=rows)


def _bias(b, n, dt=np.float64):
    return np.zeros(n, dt) if b is None else np.asarray(b, dt)


def _ft(x):
    """The floating type the layer computes in: float32 for a float32 input,
    else float64."""
    return np.float32 if np.asarray(x).dtype == np.float32 else np.float64


# ---- GCN -------------------------------------------------------------------

def gcn_forward(A: CSR, H_ext, W, b, relu: bool):
    """Z = A H_ext; Y = Z W + b; Out = relu(Y) or Y."""
    dt = _ft(H_ext)
    Z = spmm(A, H_ext)
    Y = Z @ np.asarray(W, dt) + _bias(b, W.shape[1], dt)
    Out = np.maximum(Y, 0.0) if relu else Y
    return Z, Y, Out


def gcn_forward_den(A: CSR, H_ext, W, b):
    Zd = spmm(A, np.abs(H_ext), abs_mode=True)
    Yd = Zd @ np.abs(np.asarray(W, np.float64)) + np.abs(_bias(b, W.shape[1]))
    return Zd, Yd


def gcn_backward(AT: CSR, Z, W, Y, relu: bool, G, want_dH: bool = True):
    """G_Y = G * 1[Y>0]; dW = Z^T G_Y; db = colsum G_Y; dZ = G_Y W^T;
    dH_ext = A^T dZ (over the transposed CSR)."""
    W = np.asarray(W, _ft(Z))
    GY = G * (Y > 0) if relu else G
    dW = Z.T @ GY
    db = GY.sum(axis=0)
    dZ = GY @ W.T
    dH = spmm(AT, dZ) if want_dH else None
    return dW, db, dZ, dH


def gcn_backward_den(AT: CSR, Z, W, Y, relu: bool, G, want_dH: bool = True):
    W = np.abs(np.asarray(W, np.float64))
    GY = np.abs(G * (Y > 0) if relu else G)
    dWd = np.abs(Z).T @ GY
    dbd = GY.sum(axis=0)
    dZd = GY @ W.T
    dHd = spmm(AT, dZd, abs_mode=True) if want_dH else None
    return dWd, dbd, dZd, dHd


# ---- GraphSAGE-mean ----------------------------------------------------------

def sage_forward(Am: CSR, H_ext, n_local: int, W, b, relu: bool):
    """M = mean-CSR H_ext; X = [H_local | M]; Y = X W + b; Out = relu(Y)."""
    dt = _ft(H_ext)
    M = spmm(Am, H_ext)
    X = np.concatenate([H_ext[:n_local], M], axis=1)
    Y = X @ np.asarray(W, dt) + _bias(b, W.shape[1], dt)
    Out = np.maximum(Y, 0.0) if relu else Y
    return M, Y, Out


def sage_forward_den(Am: CSR, H_ext, n_local: int, W, b):
    Md = spmm(Am, np.abs(H_ext), abs_mode=True)
    Xd = np.concatenate([np.abs(H_ext[:n_local]), Md], axis=1)
    Yd = Xd @ np.abs(np.asarray(W, np.float64)) + np.abs(_bias(b, W.shape[1]))
    return Md, Yd


def sage_backward(AmT: CSR, H_local, M, W, Y, relu: bool, G, want_dH: bool = True):
    """dW = [H|M]^T G_Y; db; [dH_self | dM] = G_Y W^T;
    dH_ext = mean-CSR^T dM, plus dH_self on the local rows."""
    W = np.asarray(W, _ft(H_local))
    d = H_local.shape[1]
    GY = G * (Y > 0) if relu else G
    X = np.concatenate([H_local, M], axis=1)
    dW = X.T @ GY
    db = GY.sum(axis=0)
    dX = GY @ W.T
    dH = None
    if want_dH:
        dH = spmm(AmT, dX[:, d:])
        dH[:H_local.shape[0]] += dX[:, :d]
    return dW, db, dH


def sage_backward_den(AmT: CSR, H_local, M, W, Y, relu: bool, G, want_dH: bool = True):
    W = np.abs(np.asarray(W, np.float64))
    d = H_local.shape[1]
    GY = np.abs(G * (Y > 0) if relu else G)
    X = np.abs(np.concatenate([H_local, M], axis=1))
    dWd = X.T @ GY
    dbd = GY.sum(axis=0)
    dXd = GY @ W.T
    dHd = None
    if want_dH:
        dHd = spmm(AmT, dXd[:, d:], abs_mode=True)
        dHd[:H_local.shape[0]] += dXd[:, :d]
    return dWd, dbd, dHd
