"""The oracle's C product built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, host code only) and run on edge cases:
an empty matrix, rows without entries, a long row, no values, d = 1, a row
pitch wider than d, no selected rows and repeated selected rows.  Every
buffer the driver hands it has its exact size, so any read or write past
one aborts the run.  The results are also checked against numpy."""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("san") / "spmm_san")
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fopenmp", "-ffp-contract=off",
           os.path.join(HERE, "sanitized_spmm_driver.c"), os.path.join(ROOT, "oracle", "spmm_f64.c"),
           "-lm", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("sanitizer build unavailable: " + r.stderr[-300:])
    return out


def _run(driver, tmp_path, indptr, indices, val, X, d, rows):
    n_rows, nnz = len(indptr) - 1, len(indices)
    n_cols, ldx = X.shape
    path_in, path_out = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    with open(path_in, "wb") as f:
        np.array([n_rows, n_cols, nnz, d, ldx, val is not None, len(rows)], np.int64).tofile(f)
        np.asarray(indptr, np.int64).tofile(f)
        np.asarray(indices, np.int32).tofile(f)
        if val is not None:
            np.asarray(val, np.float32).tofile(f)
        np.ascontiguousarray(X, np.float64).tofile(f)
        np.asarray(rows, np.int64).tofile(f)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([driver, path_in, path_out], capture_output=True, text=True, env=env)
    assert r.returncode == 0, f"sanitized run failed ({r.returncode}):\n{r.stderr[-3000:]}"
    raw = np.fromfile(path_out, np.float64)
    ny, ns = n_rows * d, len(rows) * d
    assert raw.size == 3 * ny + ns
    Y, Ya, Ys, Yf = (raw[:ny], raw[ny:2 * ny], raw[2 * ny:2 * ny + ns], raw[2 * ny + ns:])
    return (Y.reshape(n_rows, d), Ya.reshape(n_rows, d), Ys.reshape(len(rows), d), Yf.reshape(n_rows, d))


def _dense(indptr, indices, val, n_cols):
    """The matrix and the matrix of |entry| sums (repeated entries add up)."""
    n_rows = len(indptr) - 1
    A, Aabs = np.zeros((n_rows, n_cols)), np.zeros((n_rows, n_cols))
    for r in range(n_rows):
        for p in range(indptr[r], indptr[r + 1]):
            v = 1.0 if val is None else float(np.float32(val[p]))
            A[r, indices[p]] += v
            Aabs[r, indices[p]] += abs(v)
    return A, Aabs


def _check(driver, tmp_path, indptr, indices, val, X, d, rows):
    Y, Ya, Ys, Yf = _run(driver, tmp_path, indptr, indices, val, X, d, rows)
    A, Aabs = _dense(indptr, indices, val, X.shape[0])
    Xd = X[:, :d]
    ref, ref_abs = A @ Xd, Aabs @ np.abs(Xd)
    scale = ref_abs + 1e-300
    assert np.all(np.abs(Y - ref) <= 1e-12 * scale)
    assert np.all(np.abs(Ya - ref_abs) <= 1e-12 * scale)
    assert np.array_equal(Ys, Y[np.asarray(rows, np.int64)]) if len(rows) else Ys.size == 0
    assert np.all(np.abs(Yf - ref) <= 1e-5 * scale)


def _csr(g, n_rows, n_cols, lens):
    indptr = np.zeros(n_rows + 1, np.int64)
    indptr[1:] = np.cumsum(lens)
    indices = np.concatenate([np.sort(g.choice(n_cols, size=k, replace=True)) for k in lens]) \
        if sum(lens) else np.zeros(0, np.int32)
    return indptr, indices.astype(np.int32)


def test_empty_matrix(driver, tmp_path):
    X = np.random.default_rng(0).standard_normal((5, 4))
    _check(driver, tmp_path, np.zeros(1, np.int64), np.zeros(0, np.int32), None, X, 3, [])


def test_empty_rows_long_row_values_and_wide_pitch(driver, tmp_path):
    g = np.random.default_rng(1)
    lens = [0, 3, 0, 0, 7, 1] + [300] + list(g.integers(0, 5, 43))
    indptr, indices = _csr(g, len(lens), 40, lens)
    val = g.uniform(-2, 2, len(indices)).astype(np.float32)
    X = g.standard_normal((40, 8))
    _check(driver, tmp_path, indptr, indices, val, X, 7, [6, 0, 6, 49, 2])


def test_no_values_single_column(driver, tmp_path):
    g = np.random.default_rng(2)
    lens = list(g.integers(0, 9, 64))
    indptr, indices = _csr(g, 64, 17, lens)
    X = g.standard_normal((17, 1))
    _check(driver, tmp_path, indptr, indices, None, X, 1, list(range(63, -1, -1)))


def test_last_column_and_last_row(driver, tmp_path):
    # every entry in the last column, read through a pitch equal to d
    g = np.random.default_rng(3)
    n_rows, n_cols = 33, 29
    lens = [2] * n_rows
    indptr = np.arange(0, 2 * n_rows + 1, 2, dtype=np.int64)
    indices = np.full(2 * n_rows, n_cols - 1, np.int32)
    val = g.uniform(-1, 1, 2 * n_rows).astype(np.float32)
    X = g.standard_normal((n_cols, 5))
    assert sum(lens) == len(indices)
    _check(driver, tmp_path, indptr, indices, val, X, 5, [n_rows - 1])
