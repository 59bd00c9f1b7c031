"""Shared test helpers: closed-form evaluation, brute-force graph builds and
the error metric.  Nothing here is used by the product path."""
from __future__ import annotations

import ast
import math
import operator

import numpy as np

_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv, ast.USub: operator.neg}


def closed_form(expr: str) -> float:
    """Evaluate a closed-form expression made of numbers, + - * / and sqrt()."""
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant):
            return float(node.value)
        if isinstance(node, ast.BinOp):
            return _OPS[type(node.op)](ev(node.left), ev(node.right))
        if isinstance(node, ast.UnaryOp):
            return _OPS[type(node.op)](ev(node.operand))
        if isinstance(node, ast.Call) and node.func.id == "sqrt":
            return math.sqrt(ev(node.args[0]))
        raise ValueError(expr)
    return ev(ast.parse(expr, mode="eval"))


def dense_structure(src, dst, n_global, lo, hi, symmetrize, self_loops):
    """Brute force with Python sets: for each local row the sorted remapped
    columns, and the halo id list.  Independent of the oracle's numpy build."""
    nbrs = {v: set() for v in range(lo, hi)}
    for u, v in zip(list(map(int, src)), list(map(int, dst))):
        pairs = [(u, v), (v, u)] if symmetrize else [(u, v)]
        for a, b in pairs:             # a -> b : b aggregates a
            if a != b and lo <= b < hi:
                nbrs[b].add(a)
    if self_loops:
        for v in range(lo, hi):
            nbrs[v].add(v)
    halo = sorted({c for v in nbrs for c in nbrs[v] if not (lo <= c < hi)})
    n_l = hi - lo
    pos = {c: n_l + k for k, c in enumerate(halo)}
    rows = []
    for v in range(lo, hi):
        rows.append(sorted((c - lo) if lo <= c < hi else pos[c] for c in nbrs[v]))
    return rows, halo


def dense_adjacency(src, dst, n, symmetrize=True):
    A = np.zeros((n, n))
    for u, v in zip(src, dst):
        if u != v:
            A[v, u] = 1.0
            if symmetrize:
                A[u, v] = 1.0
    return A


def rel_err(got, ref, den):
    """max |got - ref| / (den + 1e-30): error relative to the magnitude of the
    summed terms (den = the same expression on absolute values)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.asarray(den, np.float64)
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (den + 1e-30)))
