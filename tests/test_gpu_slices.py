"""Products in 128-byte column slices of X (a matrix's col_slices flag).

Rows of X wider than 256 bytes are gathered one cache line per pass; each
pass writes its own columns of Y with the epilogue.  The products are
compared with the oracle (the one-pass SpMM's bounds) across widths that
leave a ragged last slice, both dtypes and the bf16 -> fp32 pair, the
mean-normalised A (values not read) and its transpose; bit for bit with
exact sums on small-integer data (long rows, empty rows); the addend on the
first rows lands in the right columns; rows of at most 256 bytes and split
matrices ignore the flag (bitwise equal to the product without it); the
allocation-free entry takes the same slices (bitwise equal); the tuner
leaves the flag as it measured."""
import numpy as np
import pytest
import torch

import gen
from oracle import csr as ocsr, native

pytestmark = pytest.mark.gpu

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from gpu_util import DEV, f64, say, to_dev, to_dev_dense, tol  # noqa: E402


def _built(cfg, scale, norm, transpose=True):
    w = gen.make_config(cfg, scale)
    src, dst = w.edges
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), w.n_global, w.lo, w.hi, w.symmetrize, w.self_loops, norm,
                                 transpose=transpose)
    ob = ocsr.build(src, dst, w.n_global, w.lo, w.hi, w.symmetrize, w.self_loops, norm)
    return gb, ob


def _x(n, d, dt, seed):
    X = gen.normal_f32((n, d), np.random.default_rng(seed))
    return to_dev_dense(X if dt == "f32" else gen.f32_to_bf16_bits(X), dt)


def _err(Y, M, X64):
    ref = native.spmm(M.indptr, M.indices, M.values, X64)
    den = native.spmm(M.indptr, M.indices, M.values, np.abs(X64), abs_mode=True)
    return np.max(np.abs(f64(Y) - ref) / (den + 1e-30)) if ref.size else 0.0


@pytest.mark.parametrize("dt,out_dt,d", [("f32", "f32", 65), ("f32", "f32", 128), ("f32", "f32", 200),
                                         ("f32", "f32", 1000), ("bf16", "bf16", 129), ("bf16", "bf16", 256),
                                         ("bf16", "bf16", 300), ("bf16", "f32", 256), ("bf16", "f32", 777)])
@pytest.mark.parametrize("cfg,scale,norm", [(4, 0.002, "mean"), (2, 0.004, "gcn"), (3, 1 / 64, "mean")])
def test_sliced_spmm_against_oracle(dt, out_dt, d, cfg, scale, norm):
    gb, ob = _built(cfg, scale, norm)
    for M in (gb.A, gb.AT):
        sag.csr_schedule(M, 64)
        sag.csr_set_col_slices(M, True)
    assert sag.col_slices_apply(gb.A, d, torch.float32 if dt == "f32" else torch.bfloat16)
    odt = torch.float32 if out_dt == "f32" else torch.bfloat16
    bound = 1e-5 if out_dt == "f32" else tol("bf16")
    X = _x(gb.A.n_cols, d, dt, d + cfg)
    say(f"sliced spmm cfg={cfg} {dt}->{out_dt} d={d}")
    e = _err(sag.spmm_csr(gb.A, X, out_dtype=odt), ob.A, f64(X))
    assert e <= bound, f"A: err {e:.3e}"
    XT = _x(gb.AT.n_cols, d, dt, d + cfg + 1)
    e = _err(sag.spmm_csr_t(gb.AT, XT, out_dtype=odt), ob.AT, f64(XT))
    assert e <= bound, f"A^T: err {e:.3e}"


@pytest.mark.parametrize("scheduled", [True, False])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_sliced_exact_small_integers_with_long_and_empty_rows(dt, scheduled):
    """Star centres far longer than a segment, rows without entries, values 1
    and integer features: every sum is exact, so each slice's columns equal
    the exact result bit for bit (a slice reading the wrong columns of X or
    writing the wrong columns of Y fails here)."""
    n = 9000
    g = np.random.default_rng(4)
    src = np.concatenate([np.arange(10, n, dtype=np.int32)] * 3 + [g.integers(10, n, 20000).astype(np.int32)])
    dst = np.concatenate([np.full(n - 10, c, np.int32) for c in (0, 1, 2)] +
                         [g.integers(3, n - 50, 20000).astype(np.int32)])
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), n, 0, n, False, False, "none", transpose=False)
    if scheduled:   # else every row is summed as a medium row, in natural order
        sag.csr_schedule(gb.A, 64)
        assert sag.csr_info(gb.A)["n_long"] > 0
    sag.csr_set_col_slices(gb.A, True)
    ob = ocsr.build(src, dst, n, 0, n, False, False, "none")
    d = 150 if dt == "f32" else 230
    X = g.integers(-4, 5, (n, d)).astype(np.float32)
    Xd = to_dev_dense(X if dt == "f32" else gen.f32_to_bf16_bits(X), dt)
    say(f"sliced exact integers dt={dt} d={d} scheduled={scheduled}")
    Y = sag.spmm_csr(gb.A, Xd, out_dtype=torch.float32)
    assert np.array_equal(f64(Y), native.spmm(ob.A.indptr, ob.A.indices, ob.A.values, X.astype(np.float64)))


def test_sliced_addend_on_the_first_rows():
    gb, ob = _built(2, 0.004, "gcn", transpose=False)
    sag.csr_schedule(gb.A, 64)
    sag.csr_set_col_slices(gb.A, True)
    g = np.random.default_rng(2)
    n, d = gb.A.n_rows, 170
    X = g.standard_normal((gb.A.n_cols, d)).astype(np.float32)
    add = g.standard_normal((n // 3, d)).astype(np.float32)
    say("sliced addend")
    Z = f64(sag.spmm_csr(gb.A, to_dev_dense(X), addend=to_dev_dense(add)))
    ref = native.spmm(ob.A.indptr, ob.A.indices, ob.A.values, X.astype(np.float64))
    ref[: n // 3] += add
    den = native.spmm(ob.A.indptr, ob.A.indices, ob.A.values, np.abs(X.astype(np.float64)), abs_mode=True)
    den[: n // 3] += np.abs(add)
    assert np.max(np.abs(Z - ref) / (den + 1e-30)) <= 1e-5


def test_flag_ignored_by_narrow_rows_and_split_matrices():
    """Rows of at most 256 bytes and products over a hub split take whole
    rows whatever the flag: bit for bit the product without it."""
    gb, _ = _built(2, 0.004, "gcn", transpose=False)
    sag.csr_schedule(gb.A, 64)
    say("col_slices ignored: narrow rows, split matrix")
    for dt, d in (("f32", 64), ("bf16", 128), ("bf16", 100)):
        X = _x(gb.A.n_cols, d, dt, d)
        a = sag.spmm_csr(gb.A, X)
        sag.csr_set_col_slices(gb.A, True)
        b = sag.spmm_csr(gb.A, X)
        sag.csr_set_col_slices(gb.A, False)
        assert torch.equal(a, b)
    X = _x(gb.A.n_cols, 128, "f32", 7)
    sag.csr_hub_split(gb.A, 100, 64, levels=2)
    a = sag.spmm_csr(gb.A, X)
    sag.csr_set_col_slices(gb.A, True)
    assert torch.equal(a, sag.spmm_csr(gb.A, X))


@pytest.mark.parametrize("dt,d", [("f32", 130), ("bf16", 256)])
def test_sliced_deterministic_and_noalloc_takes_the_same_slices(dt, d):
    gb, _ = _built(4, 0.002, "mean", transpose=False)
    sag.csr_schedule(gb.A, 64)
    sag.csr_set_col_slices(gb.A, True)
    X = _x(gb.A.n_cols, d, dt, 3)
    say(f"sliced determinism / noalloc dt={dt} d={d}")
    a = sag.spmm_csr(gb.A, X)
    assert torch.equal(a, sag.spmm_csr(gb.A, X))
    Y = sag.empty_dense(gb.A.n_rows, d, X.dtype, DEV)
    sag.spmm_csr_noalloc(gb.A, X, Y)
    assert torch.equal(Y, a)


def test_tuner_sets_the_flag_it_measured():
    gb, ob = _built(4, 0.002, "mean", transpose=False)
    sag.csr_schedule(gb.A, 64)
    say("col_slices tuner")
    r = sag.csr_tune_col_slices(gb.A, 100, torch.bfloat16)   # 200-byte rows: not eligible, nothing timed
    assert r == {"on": False, "whole_ms": None, "sliced_ms": None} and not gb.A.col_slices
    r = sag.csr_tune_col_slices(gb.A, 256, torch.bfloat16)
    assert r["whole_ms"] > 0 and r["sliced_ms"] > 0
    assert r["on"] == (r["sliced_ms"] < (1 - sag.ops.COL_SLICE_MARGIN) * r["whole_ms"])
    assert gb.A.col_slices == r["on"] and gb.A.raw.col_slices == int(r["on"])
    X = _x(gb.A.n_cols, 256, "bf16", 5)
    assert _err(sag.spmm_csr(gb.A, X), ob.A, f64(X)) <= tol("bf16")
