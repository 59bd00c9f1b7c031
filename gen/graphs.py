"""Random graph, feature and weight draws (numpy PCG64, fully seeded).

Every function takes a ``numpy.random.Generator`` so that callers choose the
stream.  Graphs are returned as raw edge lists (two int32 arrays); nothing here
normalises, symmetrises or aggregates anything.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "stream", "uniform_pairs", "power_law_weights", "chung_lu_pairs",
    "rmat_pairs", "first_distinct", "permutation", "normal_f32",
    "glorot_uniform", "uniform_bias", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "ring_pairs", "circulant_pairs", "random_regular_pairs",
]


def stream(config: int, s: int) -> np.random.Generator:
    """Generator for (config, stream): seed = 1000*config + stream."""
    return np.random.Generator(np.random.PCG64(1000 * int(config) + int(s)))


def first_distinct(keys: np.ndarray, count: int):
    """Return the first ``count`` distinct values of ``keys`` in draw order,
    or None when ``keys`` holds fewer distinct values."""
    uniq, first = np.unique(keys, return_index=True)
    if uniq.size < count:
        return None
    order = np.sort(first)[:count]
    return keys[order]


def _pairs_from_keys(keys: np.ndarray, n: int):
    u = (keys // n).astype(np.int32)
    v = (keys % n).astype(np.int32)
    return u, v


def uniform_pairs(n: int, m: int, g: np.random.Generator):
    """``m`` distinct unordered pairs {u, v}, u != v, uniform over all pairs
    (the G(n, m) model).  Returned once each, with u < v."""
    keys = np.empty(0, np.int64)
    batch = int(m * 1.2) + 1024
    while True:
        a = g.integers(0, n, batch, dtype=np.int64)
        b = g.integers(0, n, batch, dtype=np.int64)
        keep = a != b
        keys = np.concatenate([keys, np.minimum(a, b)[keep] * n + np.maximum(a, b)[keep]])
        got = first_distinct(keys, m)
        if got is not None:
            return _pairs_from_keys(got, n)


def power_law_weights(n: int, mean: float, gamma: float, kmax: float,
                      g: np.random.Generator) -> np.ndarray:
    """i.i.d. expected degrees from a continuous power law p(k) ~ k^-gamma on
    [kmin, kmax]; kmin is solved by bisection so that the law's mean is
    ``mean``.  Returns float64 weights."""
    e = 1.0 - gamma

    def law_mean(kmin):
        # mean of the truncated power law (gamma != 1, 2)
        num = (kmax ** (2.0 - gamma) - kmin ** (2.0 - gamma)) / (2.0 - gamma)
        den = (kmax ** e - kmin ** e) / e
        return num / den

    lo_, hi_ = 1e-6, mean
    for _ in range(200):
        mid = 0.5 * (lo_ + hi_)
        if law_mean(mid) < mean:
            lo_ = mid
        else:
            hi_ = mid
    kmin = 0.5 * (lo_ + hi_)
    u = g.random(n)
    return (kmin ** e + u * (kmax ** e - kmin ** e)) ** (1.0 / e)


def chung_lu_pairs(n: int, n_pairs: int, w: np.ndarray, g: np.random.Generator):
    """Chung-Lu graph by ball dropping: both endpoints of each draw are picked
    with probability proportional to ``w``; draws with u == v are dropped and
    the first ``n_pairs`` distinct unordered pairs (in draw order) are kept.
    Returned once each with u < v."""
    cw = np.cumsum(w)
    total = cw[-1]
    keys = np.empty(0, np.int64)
    batch = int(n_pairs * 1.15) + 4096
    while True:
        a = np.searchsorted(cw, g.random(batch) * total, side="right")
        b = np.searchsorted(cw, g.random(batch) * total, side="right")
        np.minimum(a, n - 1, out=a)
        np.minimum(b, n - 1, out=b)
        keep = a != b
        keys = np.concatenate([keys, np.minimum(a, b)[keep].astype(np.int64) * n
                               + np.maximum(a, b)[keep]])
        got = first_distinct(keys, n_pairs)
        if got is not None:
            return _pairs_from_keys(got, n)
        batch = int(n_pairs * 0.25) + 4096


def rmat_pairs(scale: int, n_draws: int, a: float, b: float, c: float,
               g: np.random.Generator, chunk: int = 1 << 23):
    """R-MAT edge draws (no noise): at each of ``scale`` levels the quadrant
    (a: row 0 col 0, b: row 0 col 1, c: row 1 col 0, d: row 1 col 1) is picked
    from a 16-bit uniform draw, so the quadrant probabilities are quantised to
    multiples of 2^-16.  Returns (row, col) int64 arrays of length n_draws."""
    ta = int(round(a * 65536))
    tb = ta + int(round(b * 65536))
    tc = tb + int(round(c * 65536))
    rows = np.empty(n_draws, np.int64)
    cols = np.empty(n_draws, np.int64)
    for s in range(0, n_draws, chunk):
        m = min(chunk, n_draws - s)
        r = np.zeros(m, np.int64)
        cc = np.zeros(m, np.int64)
        for level in range(scale):
            q = g.integers(0, 65536, m, dtype=np.uint16)
            bit = np.int64(1) << np.int64(scale - 1 - level)
            r |= np.where(q >= tb, bit, 0)
            cc |= np.where(((q >= ta) & (q < tb)) | (q >= tc), bit, 0)
        rows[s:s + m] = r
        cols[s:s + m] = cc
    return rows, cols


def permutation(n: int, g: np.random.Generator) -> np.ndarray:
    return g.permutation(n).astype(np.int64)


def normal_f32(shape, g: np.random.Generator) -> np.ndarray:
    return g.standard_normal(shape, dtype=np.float32)


def glorot_uniform(fan_in: int, fan_out: int, shape, g: np.random.Generator) -> np.ndarray:
    lim = np.sqrt(6.0 / (fan_in + fan_out))
    return g.uniform(-lim, lim, shape).astype(np.float32)


def uniform_bias(d: int, g: np.random.Generator, lim: float = 0.1) -> np.ndarray:
    return g.uniform(-lim, lim, d).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even, returned as uint16 bits.
    (Input encoding only: inputs are drawn in fp32 and stored as bf16.)"""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---- structured graphs with closed-form spectra -------------------------

def ring_pairs(n: int):
    """Cycle C_n as unordered pairs {i, i+1 mod n}."""
    i = np.arange(n, dtype=np.int32)
    return i, ((i + 1) % n).astype(np.int32)


def circulant_pairs(n: int, offsets):
    """Circulant graph: i ~ i+o (mod n) for each o in ``offsets`` (each
    unordered pair listed once when o < n/2; o == n/2 lists each pair twice,
    which a simple-graph build collapses)."""
    i = np.arange(n, dtype=np.int64)
    us, vs = [], []
    for o in offsets:
        us.append(i)
        vs.append((i + o) % n)
    return np.concatenate(us).astype(np.int32), np.concatenate(vs).astype(np.int32)


def random_regular_pairs(n: int, k: int, g: np.random.Generator, swaps: int = 20):
    """Random simple k-regular graph (n even when k is odd): a circulant
    k-regular graph, randomly relabelled, then ``swaps`` * (edges) random
    double-edge swaps (a-b, c-d -> a-d, c-b) that keep it simple.  Returns
    unordered pairs once each."""
    assert n > k and n * k % 2 == 0
    offs = list(range(1, k // 2 + 1))
    i = np.arange(n)
    us = [i for _ in offs]
    vs = [(i + o) % n for o in offs]
    if k % 2:
        h = np.arange(n // 2)
        us.append(h)
        vs.append(h + n // 2)
    u = np.concatenate(us)
    v = np.concatenate(vs)
    perm = g.permutation(n)
    u, v = perm[u], perm[v]
    edges = {(min(a, b), max(a, b)) for a, b in zip(u.tolist(), v.tolist())}
    el = list(edges)
    for _ in range(swaps * len(el)):
        x, y = g.integers(0, len(el), 2)
        if x == y:
            continue
        a, b = el[x]
        c, d = el[y]
        if g.random() < 0.5:
            c, d = d, c
        e1, e2 = (min(a, d), max(a, d)), (min(c, b), max(c, b))
        if a == d or c == b or e1 in edges or e2 in edges:
            continue
        edges.discard(el[x]); edges.discard(el[y])
        edges.add(e1); edges.add(e2)
        el[x], el[y] = e1, e2
    arr = np.array(sorted(edges), dtype=np.int32)
    return arr[:, 0].copy(), arr[:, 1].copy()
