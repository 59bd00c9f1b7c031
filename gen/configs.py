"""The five synthetic workloads of the hot path, drawn lazily and seeded.

Stream numbers (seed = 1000*config + stream):
  1 graph, 2 relabel permutation, 3 features, 4 stale buffer, 5 weights,
  6 bias, 7 upstream gradient, 8 halo Bernoulli, 9 remote-id permutation.

``scale`` < 1 draws the same recipe at a smaller size (fewer nodes and edges,
same degree law and widths), for tests that must finish quickly.

Public-benchmark graphs that the pages measure on (Reddit, Amazon,
ogbn-products, a 100M-node / 3B-edge graph) are not available; these
generators stand in for them at the sizes of the workloads below.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from functools import cached_property

import numpy as np

from . import graphs as G

__all__ = ["CONFIGS", "Workload", "make_config"]


@dataclass
class Workload:
    cfg: int
    name: str
    model: str            # "gcn" or "sage"
    dtype: str            # "f32" or "bf16" (storage type of activations)
    n_global: int         # node-id space of the edge list (local + remote)
    lo: int               # local row range [lo, hi)
    hi: int
    symmetrize: bool      # edge list holds each undirected pair once
    self_loops: bool      # add I
    norm: str             # "gcn" (D^-1/2 (A+I) D^-1/2) or "mean"
    dims: list            # [d_0, d_1, ..., d_L]
    relu: list            # per layer
    stale_rows: int = 0   # rows of the stale buffer (0: no halo)
    stale_base: int = 0   # stale row of global id c is c - stale_base
    scale: float = 1.0
    _graph_fn: object = field(default=None, repr=False)

    # ---- lazily drawn tensors -------------------------------------------
    @cached_property
    def edges(self):
        """(src, dst) int32 arrays: edge u -> v means v aggregates u."""
        return self._graph_fn(self)

    @property
    def n_local(self) -> int:
        return self.hi - self.lo

    @property
    def n_layers(self) -> int:
        return len(self.dims) - 1

    def _store(self, x: np.ndarray) -> np.ndarray:
        return G.f32_to_bf16_bits(x) if self.dtype == "bf16" else x

    @cached_property
    def features(self) -> np.ndarray:
        """Local input rows H_local [n_local, d_0] (fp32 or bf16 bits)."""
        return self._store(G.normal_f32((self.n_local, self.dims[0]), G.stream(self.cfg, 3)))

    @cached_property
    def stale(self):
        """Stale-representation buffer [stale_rows, d_0], or None."""
        if not self.stale_rows:
            return None
        return self._store(G.normal_f32((self.stale_rows, self.dims[0]), G.stream(self.cfg, 4)))

    def w_rows(self, layer: int) -> int:
        d_in = self.dims[layer]
        return 2 * d_in if self.model == "sage" else d_in

    @cached_property
    def weights(self):
        """fp32 weights, one [w_rows, d_out] matrix per layer (Glorot uniform,
        fan_in = rows of W)."""
        g = G.stream(self.cfg, 5)
        out = []
        for l in range(self.n_layers):
            k, n = self.w_rows(l), self.dims[l + 1]
            out.append(G.glorot_uniform(k, n, (k, n), g))
        return out

    @cached_property
    def biases(self):
        g = G.stream(self.cfg, 6)
        return [G.uniform_bias(self.dims[l + 1], g) for l in range(self.n_layers)]

    @cached_property
    def grad_out(self) -> np.ndarray:
        """Upstream gradient of the last layer's output [n_local, d_L]."""
        return self._store(G.normal_f32((self.n_local, self.dims[-1]), G.stream(self.cfg, 7)))

    def weights_stored(self, layer: int) -> np.ndarray:
        """The layer's weight in the activation storage type."""
        return self._store(self.weights[layer])


# ---- graph recipes ------------------------------------------------------

def _g_uniform(w: Workload):
    m = int(round(16384 * w.scale))
    return G.uniform_pairs(w.n_global, m, G.stream(w.cfg, 1))


def _chung_lu(mean_deg: float, gamma: float):
    """Chung-Lu power-law graph with n * mean_deg directed edges after
    symmetrisation; kmax = sqrt(sum of weights), the Chung-Lu admissibility
    bound max w^2 <= sum w."""
    def fn(w: Workload):
        n = w.n_global
        mean = min(mean_deg, (n - 1) / 8.0)   # scaled-down draws stay sparse
        target = n * mean
        kmax = math.sqrt(target)
        wt = G.power_law_weights(n, mean, gamma, kmax, G.stream(w.cfg, 1))
        return G.chung_lu_pairs(n, int(round(target / 2)), wt, G.stream(w.cfg, 1))
    return fn


def _rmat_partitioned(scale_bits: int, directed_target: float):
    """R-MAT graph, made undirected (u < v once each), self-loops dropped,
    first distinct pairs kept, then relabelled by a random permutation."""
    def fn(w: Workload):
        n = 1 << scale_bits
        n_pairs = int(round(directed_target / 2))
        g = G.stream(w.cfg, 1)
        keys = np.empty(0, np.int64)
        draws = int(n_pairs * 1.3)
        while True:
            r, c = G.rmat_pairs(scale_bits, draws, 0.57, 0.19, 0.19, g)
            keep = r != c
            k = np.minimum(r, c)[keep] * n + np.maximum(r, c)[keep]
            keys = np.concatenate([keys, k])
            got = G.first_distinct(keys, n_pairs)
            if got is not None:
                break
            draws = n_pairs // 2
        keys = got
        pi = G.permutation(n, G.stream(w.cfg, 2))
        u, v = keys // n, keys % n
        return pi[u].astype(np.int32), pi[v].astype(np.int32)
    return fn


def _rmat_share(scale_bits: int, n_local: int, n_remote: int, p_remote: float,
                directed_target: float):
    """One GPU's share of a large directed R-MAT graph: rows >= n_local are
    rejected; each kept edge's source is remote with probability p_remote
    (remote id = n_local + pi_R(c mod n_remote)) else local
    (pi_L(c mod n_local)); rows are relabelled by pi_L; self-loops dropped and
    the first distinct (dst, src) pairs kept."""
    def fn(w: Workload):
        g = G.stream(w.cfg, 1)
        gb = G.stream(w.cfg, 8)
        pi_l = G.permutation(n_local, G.stream(w.cfg, 2))
        pi_r = G.permutation(n_remote, G.stream(w.cfg, 9))
        n_glob = n_local + n_remote
        keys = np.empty(0, np.int64)
        draws = int(directed_target * 1.6)
        while True:
            r, c = G.rmat_pairs(scale_bits, draws, 0.57, 0.19, 0.19, g)
            keep = r < n_local
            r, c = r[keep], c[keep]
            remote = gb.random(r.size) < p_remote
            src = np.where(remote, n_local + pi_r[c % n_remote], pi_l[c % n_local])
            dst = pi_l[r]
            keep = src != dst
            keys = np.concatenate([keys, dst[keep] * n_glob + src[keep]])
            got = G.first_distinct(keys, int(directed_target))
            if got is not None:
                break
            draws = int(directed_target * 0.5)
        keys = got
        return (keys % n_glob).astype(np.int32), (keys // n_glob).astype(np.int32)
    return fn


def make_config(cfg: int, scale: float = 1.0) -> Workload:
    """Workload ``cfg`` (1..5) at size factor ``scale``."""
    s = float(scale)
    if cfg == 1:
        n = max(64, int(round(4096 * s)))
        return Workload(1, "tiny GCN layer, G(n,m) uniform graph", "gcn", "f32",
                        n, 0, n, True, True, "gcn", [64, 16], [True], scale=s,
                        _graph_fn=_g_uniform)
    if cfg == 2:
        n = max(256, int(round(232_965 * s)))
        return Workload(2, "2-layer GCN on a dense-ish Chung-Lu power-law graph",
                        "gcn", "f32", n, 0, n, True, True, "gcn", [602, 128, 41],
                        [True, False], scale=s,
                        _graph_fn=_chung_lu(491.9, 2.1))
    if cfg == 3:
        bits = max(10, int(round(21 + math.log2(s))))
        n = 1 << bits
        nl = n // 8
        return Workload(3, "GraphSAGE-mean partition of an R-MAT graph with stale halo",
                        "sage", "f32", n, 0, nl, True, False, "mean", [128, 256], [True],
                        stale_rows=n, stale_base=0, scale=s,
                        _graph_fn=_rmat_partitioned(bits, n * 30.0))
    if cfg == 4:
        n = max(1024, int(round(2_450_000 * s)))
        return Workload(4, "3-layer GraphSAGE-mean on a large sparse power-law graph",
                        "sage", "bf16", n, 0, n, True, True, "mean", [100, 256, 256, 47],
                        [True, True, False], scale=s,
                        _graph_fn=_chung_lu(50.49, 2.1))
    if cfg == 5:
        nl = max(4096, int(round(6_250_000 * s)))
        nr = max(2048, int(round(4_000_000 * s)))
        bits = max(12, int(math.ceil(math.log2(nl / 0.745))))
        tgt = 187.5e6 * nl / 6_250_000
        return Workload(5, "GCN on one GPU's share of a 100M-node graph, bf16 stale halo",
                        "gcn", "bf16", nl + nr, 0, nl, False, True, "gcn", [128, 128], [True],
                        stale_rows=nr, stale_base=nl, scale=s,
                        _graph_fn=_rmat_share(bits, nl, nr, 0.35, tgt))
    raise ValueError(f"unknown config {cfg}")


CONFIGS = {i: (lambda i=i, s=1.0: make_config(i, s)) for i in range(1, 6)}
