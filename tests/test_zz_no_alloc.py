"""The allocation-free SpMM (sag_spmm_csr_noalloc) against the SpMM with a
caller workspace (sag_spmm_csr), through the C ABI: two calls in a row on
one GPU, the second with a smaller input, each bitwise equal to the
workspace entry point (same kernels, partials in the library's fixed device
scratch instead of the workspace) and within the oracle's bound; a matrix
whose partial sums exceed the fixed scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import gen
from oracle import csr as ocsr, native

pytestmark = pytest.mark.gpu

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from gpu_util import DEV, bits16, f64, say, to_dev, to_dev_dense, tol  # noqa: E402


def _graph(scale, seed):
    w = gen.make_config(2, scale)
    src, dst = w.edges
    return src, dst, w.n_global


def _case(src, dst, n, d, dt, seg_len, seed, with_addend):
    say(f"noalloc spmm n={n} d={d} dt={dt} seg_len={seg_len} addend={with_addend}")
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), n, 0, n, True, True, "gcn")
    sag.csr_schedule(gb.A, seg_len)
    assert gb.A.raw.n_long > 0, "the case must have long rows (partials in the scratch)"
    need = sag._lib.lib().sag_spmm_workspace_bytes(gb.A.ref, d)
    assert 0 < need <= sag.spmm_noalloc_scratch_bytes()
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, d)).astype(np.float32)
    if dt == "bf16":
        xs = gen.f32_to_bf16_bits(x)
        tdt = torch.bfloat16
    else:
        xs = x
        tdt = torch.float32
    X = to_dev_dense(xs, dt)
    add = to_dev_dense(gen.f32_to_bf16_bits(x[: n // 2]) if dt == "bf16" else x[: n // 2], dt) if with_addend else None
    Y_ws = sag.empty_dense(n, d, tdt, DEV, fill=0.0)
    Y_na = sag.empty_dense(n, d, tdt, DEV, fill=7.0)
    sag.spmm_csr(gb.A, X, Y=Y_ws, addend=add)
    sag.spmm_csr_noalloc(gb.A, X, Y_na, addend=add)
    torch.cuda.synchronize()
    if dt == "bf16":
        assert np.array_equal(bits16(Y_na), bits16(Y_ws))
    else:
        assert np.array_equal(f64(Y_na), f64(Y_ws))
    # and the oracle's bound
    ob = ocsr.build(src, dst, n, 0, n, True, True, "gcn")
    x64 = f64(X)
    ref = native.spmm(ob.A.indptr, ob.A.indices, ob.A.values, x64)
    den = native.spmm(ob.A.indptr, ob.A.indices, ob.A.values, np.abs(x64), abs_mode=True)
    if with_addend:
        a64 = f64(add)
        ref[: n // 2] += a64
        den[: n // 2] += np.abs(a64)
    err = float(np.max(np.abs(f64(Y_na) - ref) / (den + 1e-30)))
    assert err <= tol(dt), err
    return need


def test_two_calls_in_a_row_second_smaller():
    src, dst, n = _graph(0.02, 1)
    need1 = _case(src, dst, n, 256, "bf16", 64, 11, True)
    src2, dst2, n2 = _graph(0.006, 2)
    need2 = _case(src2, dst2, n2, 40, "f32", 64, 12, False)
    assert need2 < need1


def test_oversized_partials_are_refused_before_any_launch():
    """A schedule whose long rows need more partial-sum memory than the fixed
    scratch: SAG_E_WORKSPACE from the host-side check (no kernel runs)."""
    L = sag._lib
    lib = L.lib()
    fake = ctypes.c_void_p(1 << 20)
    A = L.SagCsr()
    A.n_rows, A.n_cols, A.nnz = 200_000, 200_000, 50_000_000
    A.indptr = A.indices = A.values = A.sched = fake
    A.n_short, A.n_medium, A.n_long, A.n_seg, A.seg_len = 100_000, 0, 100_000, 100_000, 64
    d = 256
    assert lib.sag_spmm_workspace_bytes(ctypes.byref(A), d) > lib.sag_spmm_noalloc_scratch_bytes()
    st = lib.sag_spmm_csr_noalloc(ctypes.byref(A), fake, d, L.SAG_BF16, d, fake, d, L.SAG_BF16, None, 0, 0,
                                  None)
    assert st == L.SAG_E_WORKSPACE
    assert b"scratch" in lib.sag_last_error()
