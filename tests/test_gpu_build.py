"""GPU CSR build, halo map, transpose and schedule against the oracle:
bit-exact on every array."""
import numpy as np
import pytest
import torch

import gen
from oracle import csr as ocsr

pytestmark = pytest.mark.gpu

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from gpu_util import DEV, say, to_dev  # noqa: E402


def _cmp_built(gb, ob):
    A, AT = gb.A, gb.AT
    assert A.n_rows == ob.A.n_rows and A.n_cols == ob.A.n_cols
    assert np.array_equal(A.indptr.cpu().numpy(), ob.A.indptr)
    assert np.array_equal(A.indices.cpu().numpy(), ob.A.indices)
    assert np.array_equal(A.values.cpu().numpy().view(np.uint32), ob.A.values.view(np.uint32))
    assert np.array_equal(gb.halo_gid.cpu().numpy(), ob.halo_gid)
    assert np.array_equal(gb.deg.cpu().numpy(), ob.deg_col)
    if AT is not None:
        assert np.array_equal(AT.indptr.cpu().numpy(), ob.AT.indptr)
        assert np.array_equal(AT.indices.cpu().numpy(), ob.AT.indices)
        assert np.array_equal(AT.values.cpu().numpy().view(np.uint32), ob.AT.values.view(np.uint32))


def _edges(seed, n, m):
    g = np.random.default_rng(seed)
    src = g.integers(0, n, m).astype(np.int32)
    dst = g.integers(0, n, m).astype(np.int32)
    k = m // 5   # duplicates and explicit self-loops
    src = np.concatenate([src, src[:k], np.arange(min(3, n), dtype=np.int32)])
    dst = np.concatenate([dst, dst[:k], np.arange(min(3, n), dtype=np.int32)])
    return src, dst


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("norm", ["gcn", "mean", "none"])
def test_random_partitions(seed, norm):
    g = np.random.default_rng(100 + seed)
    n = int(g.integers(2, 3000))
    m = int(g.integers(0, 6 * n))
    src, dst = _edges(seed, n, m)
    lo = int(g.integers(0, n))
    hi = int(g.integers(lo, n + 1))
    sym, loops = bool(seed % 2), bool((seed // 2) % 2)
    say(f"build random seed={seed} n={n} m={m} lo={lo} hi={hi} sym={sym} loops={loops} norm={norm}")
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), n, lo, hi, sym, loops, norm)
    ob = ocsr.build(src, dst, n, lo, hi, sym, loops, norm)
    _cmp_built(gb, ob)


def test_given_halo_degrees():
    g = np.random.default_rng(7)
    n = 5000
    src, dst = _edges(7, n, 20000)
    dg = g.integers(1, 500, n).astype(np.int32)
    say("build with given global degrees")
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), n, 1000, 3000, False, True, "gcn",
                                 deg_global=to_dev(dg))
    ob = ocsr.build(src, dst, n, 1000, 3000, False, True, "gcn", deg_global=dg)
    _cmp_built(gb, ob)


@pytest.mark.parametrize("cfg,scale", [(1, 1.0), (2, 0.01), (3, 1 / 64), (4, 0.004), (5, 0.002)])
def test_workload_graphs(cfg, scale):
    w = gen.make_config(cfg, scale)
    src, dst = w.edges
    say(f"build config {cfg} scale {scale}: n_global={w.n_global} edges={src.size}")
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), w.n_global, w.lo, w.hi, w.symmetrize,
                                 w.self_loops, w.norm)
    ob = ocsr.build(src, dst, w.n_global, w.lo, w.hi, w.symmetrize, w.self_loops, w.norm)
    _cmp_built(gb, ob)


def test_empty_and_degenerate():
    e = np.zeros(0, np.int32)
    say("build empty graphs")
    for lo, hi, loops in [(0, 0, True), (0, 5, False), (0, 5, True), (2, 4, True)]:
        gb = sag.csr_build_normalize(to_dev(e), to_dev(e), 5, lo, hi, True, loops, "gcn")
        ob = ocsr.build(e, e, 5, lo, hi, True, loops, "gcn")
        _cmp_built(gb, ob)
    # only self-loops in the input: all dropped
    s = np.arange(6, dtype=np.int32)
    gb = sag.csr_build_normalize(to_dev(s), to_dev(s), 6, 0, 6, True, False, "mean")
    ob = ocsr.build(s, s, 6, 0, 6, True, False, "mean")
    _cmp_built(gb, ob)


def test_out_of_range_id_is_reported():
    src = np.array([0, 1, 7], np.int32)
    dst = np.array([1, 2, 3], np.int32)
    say("build with an id out of range")
    with pytest.raises(sag._lib.SagError) as ei:
        sag.csr_build_normalize(to_dev(src), to_dev(dst), 5, 0, 5, True, True, "gcn")
    assert ei.value.status == sag._lib.SAG_E_RANGE
    src = np.array([0, -1], np.int32)
    dst = np.array([1, 2], np.int32)
    with pytest.raises(sag._lib.SagError):
        sag.csr_build_normalize(to_dev(src), to_dev(dst), 5, 0, 5, True, True, "gcn")


@pytest.mark.parametrize("seed", range(6))
def test_query_sizes_match_the_build(seed):
    """sag_csr_build_normalize_query returns the entry count and halo size
    that the build then produces (and the oracle's), without outputs; an
    exact-size build from those sizes matches the oracle bit for bit."""
    g = np.random.default_rng(300 + seed)
    n = int(g.integers(2, 4000))
    src, dst = _edges(seed, n, int(g.integers(0, 5 * n)))
    lo = int(g.integers(0, n))
    hi = int(g.integers(lo, n + 1))
    sym, loops = bool(seed % 2), bool((seed // 2) % 2)
    say(f"build query seed={seed} n={n} lo={lo} hi={hi} sym={sym} loops={loops}")
    nnz, n_halo = sag.csr_build_normalize_query(to_dev(src), to_dev(dst), n, lo, hi, sym, loops)
    ob = ocsr.build(src, dst, n, lo, hi, sym, loops, "gcn")
    assert (nnz, n_halo) == (ob.A.nnz, ob.n_halo)
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), n, lo, hi, sym, loops, "gcn", max_halo=n_halo)
    _cmp_built(gb, ob)


def test_query_reports_out_of_range_ids():
    src = np.array([0, 1, 9], np.int32)
    dst = np.array([1, 2, 3], np.int32)
    say("build query with an id out of range")
    with pytest.raises(sag._lib.SagError) as ei:
        sag.csr_build_normalize_query(to_dev(src), to_dev(dst), 5, 0, 5, True, True)
    assert ei.value.status == sag._lib.SAG_E_RANGE


def test_capacity_too_small_reports_sizes():
    src, dst = _edges(3, 200, 800)
    say("build with a small halo capacity")
    with pytest.raises(sag._lib.SagError) as ei:
        sag.csr_build_normalize(to_dev(src), to_dev(dst), 200, 0, 50, True, True, "gcn", max_halo=3)
    assert ei.value.status == sag._lib.SAG_E_WORKSPACE


def test_deterministic_repeat():
    w = gen.make_config(2, 0.005)
    src, dst = w.edges
    say("build twice")
    a = sag.csr_build_normalize(to_dev(src), to_dev(dst), w.n_global, 0, w.n_global, True, True, "gcn")
    b = sag.csr_build_normalize(to_dev(src), to_dev(dst), w.n_global, 0, w.n_global, True, True, "gcn")
    assert torch.equal(a.A.indices, b.A.indices) and torch.equal(a.AT.values, b.AT.values)


@pytest.mark.parametrize("seg_len", [64, 256, 1024])
def test_schedule_covers_rows(seg_len):
    # power-law rows: Chung-Lu plus one hub row of 5000 entries
    w = gen.make_config(2, 0.01)
    src, dst = w.edges
    hub_src = np.arange(1, 5001, dtype=np.int32) % w.n_global
    src = np.concatenate([src, hub_src])
    dst = np.concatenate([dst, np.zeros(5000, np.int32)])
    say(f"schedule seg_len={seg_len}")
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), w.n_global, 0, w.n_global, True, True, "gcn")
    A = sag.csr_schedule(gb.A, seg_len)
    info = sag.csr_info(A)
    indptr = A.indptr.cpu().numpy()
    lens = np.diff(indptr)
    n = A.n_rows
    rec = A.sched[: 16 * n].cpu().view(torch.int32).numpy().reshape(n, 4)
    # every row exactly once, records consistent with indptr
    assert np.array_equal(np.sort(rec[:, 0]), np.arange(n))
    assert np.array_equal(rec[:, 1], lens[rec[:, 0]])
    start = rec[:, 2].astype(np.int64) & 0xFFFFFFFF | (rec[:, 3].astype(np.int64) << 32)
    assert np.array_equal(start, indptr[rec[:, 0]])
    ns, nm, nl = info["n_short"], info["n_medium"], info["n_long"]
    assert ns + nm + nl == n
    assert np.all(rec[:ns, 1] <= 32)
    assert np.all((rec[ns:ns + nm, 1] > 32) & (rec[ns:ns + nm, 1] <= seg_len))
    assert np.all(rec[ns + nm:, 1] > seg_len)
    # within a bin, by length class then row id
    key = np.where(rec[:, 1] == 0, 0, np.floor(np.log2(np.maximum(rec[:, 1], 1))).astype(int) + 1)
    bins = np.repeat([0, 1, 2], [ns, nm, nl])
    order = np.lexsort((rec[:, 0], key, bins))
    assert np.array_equal(order, np.arange(n))
    # segments tile each long row in order
    nseg = info["n_seg"]
    seg = A.sched[16 * n: 16 * (n + nseg)].cpu().view(torch.int32).numpy().reshape(nseg, 4)
    seg0 = A.sched[16 * (n + nseg): 16 * (n + nseg) + 4 * (nl + 1)].cpu().view(torch.int32).numpy()
    assert seg0[0] == 0 and seg0[-1] == nseg
    for j in range(nl):
        r = rec[ns + nm + j]
        s = seg[seg0[j]:seg0[j + 1]]
        assert np.all(s[:, 0] == j)
        st = s[:, 1].astype(np.int64) & 0xFFFFFFFF | (s[:, 2].astype(np.int64) << 32)
        assert st[0] == indptr[r[0]] and np.all(np.diff(st) == seg_len)
        assert s[:, 3].sum() == r[1] and np.all(s[:-1, 3] == seg_len)
