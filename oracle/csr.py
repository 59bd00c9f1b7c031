"""Oracle CSR build: normalised adjacency, HALO set and transposed matrix.

Test infrastructure only.  Plain numpy; library sorts/uniques serve as steps.

Definitions followed
--------------------
* Modified adjacency (CAGNET page, background on GNN forward propagation;
  Sylvie, "Forward Propagation"): A gets self-connections, then rows and
  columns are scaled by D^-1/2 where D holds the degrees of A + I.
* An edge u -> v means node v aggregates u, so CSR row v lists the sources u
  (the CAGNET page writes the aggregation as A^T H and keeps A and A^T apart
  so that directed graphs work).
* HALO nodes of a partition (Sylvie, "Graph Engine" and the partition
  figure's description; DIGEST, the set H~_out of out-of-subgraph neighbours
  in the "pull" operation): neighbours of local nodes that lie outside the
  local range.

Readings where the pages are silent
-----------------------------------
* A is a 0/1 graph: duplicate edges collapse and input self-loops are dropped
  before I is added, so a self-loop counts once in its row's degree.
* The column degree of a local column j is the degree of row j; of a halo
  column it is ``deg_global[c]`` when given, else 1 + the number of entries
  in that column (the owner's self-loop plus the edges seen locally).
* Degrees are clamped to >= 1 before use (an empty row of the mean is 0).
* Values are stored in fp32: GCN (float)(1 / sqrt((double)d_r * (double)d_c)),
  mean (float)(1 / (double)d_r), none 1.
* Column ids are remapped: local c -> c - lo; halo c -> n_local + its rank in
  the ascending list of halo ids.  Each row is sorted by remapped id.
* The transposed CSR has n_local + n_halo rows; row c' lists the rows r that
  hold column c', ascending in r, with the same values.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

NORMS = ("gcn", "mean", "none")


@dataclass
class CSR:
    n_rows: int
    n_cols: int
    indptr: np.ndarray    # int64 [n_rows + 1]
    indices: np.ndarray   # int32 [nnz]
    values: np.ndarray    # float32 [nnz]

    @property
    def nnz(self) -> int:
        return int(self.indices.size)

    def row_ids(self) -> np.ndarray:
        return np.repeat(np.arange(self.n_rows, dtype=np.int64), np.diff(self.indptr))


@dataclass
class Built:
    A: CSR                # n_local x (n_local + n_halo)
    AT: CSR               # (n_local + n_halo) x n_local
    deg_row: np.ndarray   # int32 [n_local]
    deg_col: np.ndarray   # int32 [n_local + n_halo] (degree used per column)
    halo_gid: np.ndarray  # int32 [n_halo], ascending global ids

    @property
    def n_local(self) -> int:
        return self.A.n_rows

    @property
    def n_halo(self) -> int:
        return int(self.halo_gid.size)


def build(src, dst, n_global: int, lo: int, hi: int, symmetrize: bool,
          self_loops: bool, norm: str, deg_global=None) -> Built:
    """Build the normalised CSR of rows [lo, hi) from an edge list.

    src, dst: node ids of edges src -> dst (dst aggregates src).
    Raises ValueError for ids outside [0, n_global) or a bad range."""
    if norm not in NORMS:
        raise ValueError(f"norm must be one of {NORMS}")
    if not (0 <= lo <= hi <= n_global):
        raise ValueError("need 0 <= lo <= hi <= n_global")
    u = np.asarray(src, dtype=np.int64)
    v = np.asarray(dst, dtype=np.int64)
    if u.shape != v.shape:
        raise ValueError("src and dst differ in length")
    if u.size and (u.min() < 0 or v.min() < 0 or u.max() >= n_global or v.max() >= n_global):
        raise ValueError("edge id out of range")
    n_l = hi - lo

    # 1. optional symmetrisation: add the reverse of every edge
    if symmetrize:
        u, v = np.concatenate([u, v]), np.concatenate([v, u])
    # 2. drop input self-loops and rows outside the local range
    keep = (u != v) & (v >= lo) & (v < hi)
    u, v = u[keep], v[keep]
    # 3. 0/1 graph: each (row, column) pair once
    key = np.unique((v - lo) * n_global + u)
    rows = key // n_global
    gcol = key % n_global
    # 4. self-connections, one per local row
    if self_loops:
        r_self = np.arange(n_l, dtype=np.int64)
        rows = np.concatenate([rows, r_self])
        gcol = np.concatenate([gcol, r_self + lo])
    # 5. HALO set and remapped column ids
    is_local = (gcol >= lo) & (gcol < hi)
    halo_gid = np.unique(gcol[~is_local])
    col = np.where(is_local, gcol - lo, n_l + np.searchsorted(halo_gid, gcol))
    n_h = halo_gid.size
    # 6. rows sorted by remapped column
    order = np.lexsort((col, rows))
    rows, col = rows[order], col[order]
    counts = np.bincount(rows, minlength=n_l).astype(np.int64)
    indptr = np.zeros(n_l + 1, np.int64)
    np.cumsum(counts, out=indptr[1:])
    deg_row = counts.astype(np.int32)

    # 7. column degrees
    deg_col = np.zeros(n_l + n_h, np.int64)
    deg_col[:n_l] = counts
    if n_h:
        if deg_global is not None:
            deg_col[n_l:] = np.asarray(deg_global, np.int64)[halo_gid]
        else:
            deg_col[n_l:] = 1 + np.bincount(col[col >= n_l] - n_l, minlength=n_h)
    dr = np.maximum(counts[rows], 1).astype(np.float64)
    dc = np.maximum(deg_col[col], 1).astype(np.float64)

    # 8. values
    if norm == "gcn":
        vals = (1.0 / np.sqrt(dr * dc)).astype(np.float32)
    elif norm == "mean":
        vals = (1.0 / dr).astype(np.float32)
    else:
        vals = np.ones(rows.size, np.float32)

    A = CSR(n_l, n_l + n_h, indptr, col.astype(np.int32), vals)
    return Built(A, transpose(A), deg_row, deg_col.astype(np.int32),
                 halo_gid.astype(np.int32))


def transpose(A: CSR) -> CSR:
    """Row c of the result lists (r, value) for every entry (r, c) of A, in
    ascending r (a stable sort of A's entries by column)."""
    rows = A.row_ids()
    order = np.argsort(A.indices, kind="stable")
    cols_t = rows[order]
    counts = np.bincount(A.indices, minlength=A.n_cols).astype(np.int64)
    indptr = np.zeros(A.n_cols + 1, np.int64)
    np.cumsum(counts, out=indptr[1:])
    return CSR(A.n_cols, A.n_rows, indptr, cols_t.astype(np.int32), A.values[order])


def gather(src: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """DIGEST "pull": out[k] = src[rows[k]] (a row copy)."""
    return np.asarray(src)[np.asarray(rows, np.int64)]


def halo_rows(built: Built, stale_base: int) -> np.ndarray:
    """Stale-buffer row of each halo node: halo_gid[k] - stale_base."""
    return built.halo_gid.astype(np.int64) - stale_base


def _adjacent_pairs(src, dst, nodes, symmetrize):
    """(v, u) pairs with v in `nodes` aggregating u != v (each once)."""
    src = np.asarray(src, np.int64)
    dst = np.asarray(dst, np.int64)
    nodes = np.unique(np.asarray(nodes, np.int64))
    sel = np.isin(dst, nodes)
    v, u = dst[sel], src[sel]
    if symmetrize:
        sel2 = np.isin(src, nodes)
        v = np.concatenate([v, src[sel2]])
        u = np.concatenate([u, dst[sel2]])
    keep = u != v
    v, u = v[keep], u[keep]
    if v.size == 0:
        return v, u
    n = int(max(v.max(), u.max())) + 1
    key = np.unique(v * n + u)
    return key // n, key % n


def build_rows(src, dst, n_global: int, lo: int, hi: int, symmetrize: bool, self_loops: bool,
               norm: str, rows, deg_global=None):
    """The normalised adjacency restricted to the local rows `rows` (global
    ids in [lo, hi)), from the definition, one row at a time -- for checks
    at sizes where the whole-partition build is too slow.

    Returns a list with, per requested row, (columns, values): the global ids
    of the row's entries (ascending) and their fp32 values, computed exactly
    as in ``build`` (same readings: 0/1 graph, one self connection, degree
    of a halo column = deg_global or 1 + its local entries)."""
    if norm not in NORMS:
        raise ValueError(f"norm must be one of {NORMS}")
    rows = np.asarray(rows, np.int64)
    if rows.size and (rows.min() < lo or rows.max() >= hi):
        raise ValueError("rows must be local")

    def neighbours(nodes):
        v, u = _adjacent_pairs(src, dst, nodes, symmetrize)
        return v, u

    v, u = neighbours(rows)
    cols = {int(r): [] for r in rows}
    for a, b in zip(v.tolist(), u.tolist()):
        cols[a].append(b)
    if self_loops:
        for r in cols:
            cols[r].append(r)
    cols = {r: np.unique(np.asarray(c, np.int64)) for r, c in cols.items()}

    def row_degree(nodes):
        """Entries of local rows `nodes` (their degree in A + I)."""
        nodes = np.unique(np.asarray(nodes, np.int64))
        vv, _ = neighbours(nodes)
        cnt = np.zeros(nodes.size, np.int64)
        if vv.size:
            cnt += np.bincount(np.searchsorted(nodes, vv), minlength=nodes.size)
        if self_loops:
            cnt += 1
        return dict(zip(nodes.tolist(), cnt.tolist()))

    all_cols = np.unique(np.concatenate([c for c in cols.values()])) if cols else np.zeros(0, np.int64)
    local_cols = all_cols[(all_cols >= lo) & (all_cols < hi)]
    halo_cols = all_cols[(all_cols < lo) | (all_cols >= hi)]
    deg = row_degree(np.concatenate([rows, local_cols]))
    if halo_cols.size:
        if deg_global is not None:
            dg = np.asarray(deg_global, np.int64)
            deg.update({int(c): int(dg[c]) for c in halo_cols})
        else:
            # 1 + the number of local rows holding the halo column
            hv, hu = _adjacent_pairs(dst, src, halo_cols, symmetrize)   # (halo c, row r) with r -> c reversed
            local = (hu >= lo) & (hu < hi)
            cnt = np.bincount(np.searchsorted(halo_cols, hv[local]), minlength=halo_cols.size)
            deg.update({int(c): 1 + int(k) for c, k in zip(halo_cols.tolist(), cnt.tolist())})
    out = []
    for r in rows.tolist():
        c = cols[r]
        dr = float(max(deg[r], 1))
        if norm == "gcn":
            dc = np.array([max(deg[int(x)], 1) for x in c], np.float64)
            val = (1.0 / np.sqrt(dr * dc)).astype(np.float32)
        elif norm == "mean":
            val = np.full(c.size, np.float32(1.0 / dr), np.float32)
        else:
            val = np.ones(c.size, np.float32)
        out.append((c, val))
    return out
