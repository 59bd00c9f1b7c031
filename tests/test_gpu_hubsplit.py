"""Hub split of a CSR (one level or a chain) and the products over it.

The split's structure is checked against its definition on the host: the
hub columns are the n_hub columns holding the most entries (ties to the
lower id), every row's hub and cold entries are its entries in those
columns and in the others, in their order, with their values.  Products
over a split matrix are compared with the oracle (the same bounds as the
one-pass SpMM), bit for bit with exact sums on small-integer data, with
the one-pass product on every edge case of the split (one hub column,
every column a hub, rows with entries in one part only, rows longer than a
segment), and with themselves for determinism.  A chain splits each cold
part again: every level's hub columns are the busiest of what remains."""
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
    return w, src, dst, gb


def _host(A):
    return (A.indptr.cpu().numpy(), A.indices.cpu().numpy(),
            A.values.cpu().numpy() if A.values is not None else None)


def _check_structure(A, n_hub):
    ip, ix, vv = _host(A)
    cnt = np.bincount(ix, minlength=A.n_cols)
    order = np.lexsort((np.arange(A.n_cols), -cnt))       # most entries first, then lower id
    hub = np.zeros(A.n_cols, bool)
    hub[order[:n_hub]] = True
    hp, hi, hv = _host(A.hub_part)
    cp, ci, cv = _host(A.cold_part)
    assert A.hub_part.nnz == int(hub[ix].sum()) and A.hub_part.nnz + A.cold_part.nnz == A.nnz
    for r in range(A.n_rows):
        e = slice(ip[r], ip[r + 1])
        m = hub[ix[e]]
        assert np.array_equal(hi[hp[r]:hp[r + 1]], ix[e][m])
        assert np.array_equal(ci[cp[r]:cp[r + 1]], ix[e][~m])
        if vv is not None:
            assert np.array_equal(hv[hp[r]:hp[r + 1]], vv[e][m])
            assert np.array_equal(cv[cp[r]:cp[r + 1]], vv[e][~m])


@pytest.mark.parametrize("n_hub", [1, 37, 512, 10 ** 9])
@pytest.mark.parametrize("cfg,scale,norm", [(2, 0.004, "gcn"), (4, 0.002, "mean"), (3, 1 / 128, "none")])
def test_split_structure(n_hub, cfg, scale, norm):
    w, _, _, gb = _built(cfg, scale, norm)
    say(f"hub split structure cfg={cfg} n_hub={n_hub}")
    sag.csr_hub_split(gb.A, n_hub, 64, levels=1)
    _check_structure(gb.A, min(n_hub, gb.A.n_cols))
    sag.csr_hub_split(gb.AT, n_hub, 64, levels=1)
    _check_structure(gb.AT, min(n_hub, gb.AT.n_cols))


@pytest.mark.parametrize("levels", [3, None])
def test_chain_structure(levels):
    """Each level of a chain is the split of the previous level's cold part."""
    w, _, _, gb = _built(2, 0.004, "gcn", transpose=False)
    say(f"hub chain structure levels={levels}")
    sag.csr_hub_split(gb.A, 40, 64, levels=levels)
    chain = sag.hub_chain(gb.A)
    assert sum(chain) == gb.A.nnz and len(chain) >= 2
    if levels:
        assert len(chain) == levels + 1
    else:
        # the automatic depth stops after the first group under 2% of the
        # entries (or when nothing is left to split)
        assert chain[-2] < 0.02 * gb.A.nnz or chain[-1] == 0
        assert all(c >= 0.02 * gb.A.nnz for c in chain[:-2])
    M = gb.A
    while M.hub_part is not None:
        _check_structure(M, min(40, M.n_cols))
        M = M.cold_part


@pytest.mark.parametrize("n_hub,levels", [(16, 1), (300, 1), (30, 5), (60, None)])
@pytest.mark.parametrize("dt,out_dt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("d", [1, 41, 128, 256])
def test_two_pass_spmm_against_oracle(n_hub, levels, dt, out_dt, d):
    w, src, dst, gb = _built(2, 0.004, "gcn")
    sag.csr_schedule(gb.A, 128)
    sag.csr_hub_split(gb.A, n_hub, 128, levels=levels)
    ob = ocsr.build(src, dst, w.n_global, 0, w.n_global, True, True, "gcn")
    X = gen.normal_f32((ob.A.n_cols, d), np.random.default_rng(d + n_hub))
    Xd = to_dev_dense(X if dt == "f32" else gen.f32_to_bf16_bits(X), dt)
    X64 = f64(Xd)
    say(f"two-pass spmm n_hub={n_hub} levels={levels} {dt}->{out_dt} d={d}")
    Y = sag.spmm_csr(gb.A, Xd, out_dtype=torch.float32 if out_dt == "f32" else torch.bfloat16)
    ref = native.spmm(ob.A.indptr, ob.A.indices, ob.A.values, X64)
    den = native.spmm(ob.A.indptr, ob.A.indices, ob.A.values, np.abs(X64), abs_mode=True)
    err = np.max(np.abs(f64(Y) - ref) / (den + 1e-30))
    bound = 1e-5 if out_dt == "f32" else tol("bf16")
    assert err <= bound, f"err {err:.3e} > {bound}"


def test_two_pass_addend_epilogue_and_transpose():
    """The caller's addend on the first rows, the transposed product over a
    split A^T, and <Y, A X> = <A^T Y, X> across the two split matrices."""
    w, src, dst, gb = _built(2, 0.004, "mean")
    for M in (gb.A, gb.AT):
        sag.csr_schedule(M, 64)
        sag.csr_hub_split(M, 100, 64, levels=3)
    ob = ocsr.build(src, dst, w.n_global, 0, w.n_global, True, True, "mean")
    g = np.random.default_rng(2)
    n, d = gb.A.n_rows, 40
    X = g.standard_normal((n, d)).astype(np.float32)
    Yv = g.standard_normal((n, d)).astype(np.float32)
    add = g.standard_normal((n // 3, d)).astype(np.float32)
    say("two-pass addend and transpose")
    Z = f64(sag.spmm_csr(gb.A, to_dev_dense(X), addend=to_dev_dense(add)))
    ref = native.spmm(ob.A.indptr, ob.A.indices, ob.A.values, X.astype(np.float64))
    ref[: n // 3] += add
    den = native.spmm(ob.A.indptr, ob.A.indices, ob.A.values, np.abs(X.astype(np.float64)), abs_mode=True)
    den[: n // 3] += np.abs(add)
    assert np.max(np.abs(Z - ref) / (den + 1e-30)) <= 1e-5
    AX = f64(sag.spmm_csr(gb.A, to_dev_dense(X)))
    ATY = f64(sag.spmm_csr_t(gb.AT, to_dev_dense(Yv)))
    rt = native.spmm(ob.AT.indptr, ob.AT.indices, ob.AT.values, Yv.astype(np.float64))
    dt_ = native.spmm(ob.AT.indptr, ob.AT.indices, ob.AT.values, np.abs(Yv.astype(np.float64)), abs_mode=True)
    assert np.max(np.abs(ATY - rt) / (dt_ + 1e-30)) <= 1e-5
    assert abs(np.sum(Yv * AX) - np.sum(ATY * X)) <= 1e-5 * np.sum(np.abs(Yv) * f64(sag.spmm_csr(gb.A, to_dev_dense(np.abs(X)))))


@pytest.mark.parametrize("n_hub,levels", [(1, 1), (5, 1), (250, 1), (10 ** 6, 1), (1, 6), (50, None)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_two_pass_exact_small_integers(n_hub, levels, dt):
    """Values 1 (no normalisation) and integer features: every sum is exact,
    so the two-pass product equals the exact result bit for bit, whatever the
    split (one hub column, a few, every column)."""
    w, src, dst, gb = _built(2, 0.004, "none", transpose=False)
    sag.csr_schedule(gb.A, 64)
    sag.csr_hub_split(gb.A, n_hub, 64, levels=levels)
    ob = ocsr.build(src, dst, w.n_global, 0, w.n_global, True, True, "none")
    X = np.random.default_rng(n_hub).integers(-8, 9, (gb.A.n_cols, 72)).astype(np.float32)
    Xd = to_dev_dense(X if dt == "f32" else gen.f32_to_bf16_bits(X), dt)
    say(f"two-pass exact n_hub={n_hub} levels={levels} dt={dt}")
    Y = sag.spmm_csr(gb.A, Xd, out_dtype=torch.float32)
    ref = native.spmm(ob.A.indptr, ob.A.indices, ob.A.values, X.astype(np.float64))
    assert np.array_equal(f64(Y), ref)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_two_pass_long_rows_and_one_part_rows(dt):
    """Star centres with rows far longer than a segment in both parts, rows
    whose entries all fall in one part, and rows without entries."""
    n = 9000
    g = np.random.default_rng(4)
    src = np.concatenate([np.arange(10, n, dtype=np.int32)] * 3 + [g.integers(10, n, 20000).astype(np.int32)])
    dst = np.concatenate([np.full(n - 10, c, np.int32) for c in (0, 1, 2)] + [g.integers(3, n - 50, 20000).astype(np.int32)])
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), n, 0, n, False, False, "none", transpose=False)
    sag.csr_schedule(gb.A, 64)
    sag.csr_hub_split(gb.A, 900, 64, levels=2)
    assert sag.csr_info(gb.A.hub_part)["n_long"] > 0 and sag.csr_info(gb.A.cold_part)["n_long"] > 0
    assert sag.csr_info(gb.A.cold_part.cold_part)["n_long"] > 0
    ip = gb.A.indptr.cpu().numpy()
    assert np.any(np.diff(ip) == 0)
    ob = ocsr.build(src, dst, n, 0, n, False, False, "none")
    X = g.integers(-4, 5, (n, 24)).astype(np.float32)
    Xd = to_dev_dense(X if dt == "f32" else gen.f32_to_bf16_bits(X), dt)
    say(f"two-pass long rows dt={dt}")
    Y = sag.spmm_csr(gb.A, Xd, out_dtype=torch.float32)
    ref = native.spmm(ob.A.indptr, ob.A.indices, ob.A.values, X.astype(np.float64))
    assert np.array_equal(f64(Y), ref)


def test_two_pass_deterministic_and_noalloc_one_pass():
    """Two runs of the two-pass product agree bit for bit; the allocation-free
    entry multiplies the same matrix in one pass over its own arrays, bit for
    bit like the matrix without its split."""
    w, src, dst, gb = _built(2, 0.004, "gcn", transpose=False)
    sag.csr_schedule(gb.A, 64)
    X = to_dev_dense(gen.normal_f32((gb.A.n_cols, 100), np.random.default_rng(0)))
    say("two-pass determinism / noalloc")
    one = sag.spmm_csr(gb.A, X)
    sag.csr_hub_split(gb.A, 100, 64)
    a = sag.spmm_csr(gb.A, X)
    b = sag.spmm_csr(gb.A, X)
    assert torch.equal(a, b)
    Y = sag.empty_dense(gb.A.n_rows, 100, torch.float32, DEV)
    sag.spmm_csr_noalloc(gb.A, X, Y)
    assert torch.equal(Y, one)


def _gat_pass(gb, H, W, asrc, adst, b, G):
    out, ctx = sag.gat_layer_forward(gb.A, H, W, asrc, adst, b, heads=4, relu=True)
    dW, das, dad, db, dH = sag.gat_layer_backward(ctx, gb.A, gb.AT, out, G)
    return [out, dW, das, dad, db, dH]


def test_gat_reads_the_matrix_itself():
    """GAT works on the matrix's own arrays, so a split changes none of its
    bits (forward and backward)."""
    w, _, _, gb = _built(2, 0.004, "none")
    for M in (gb.A, gb.AT):
        sag.csr_schedule(M, 64)
    g = torch.Generator(device=DEV)
    g.manual_seed(8)
    n, d, F = gb.A.n_cols, 64, 64
    H = sag.empty_dense(n, d, torch.float32, DEV)
    H.copy_(torch.randn(n, d, device=DEV, generator=g))
    W = (torch.randn(d, F, device=DEV, generator=g) * 0.1).contiguous()
    asrc = torch.randn(4, 16, device=DEV, generator=g) * 0.3
    adst = torch.randn(4, 16, device=DEV, generator=g) * 0.3
    b = torch.randn(F, device=DEV, generator=g) * 0.1
    G = sag.empty_dense(gb.A.n_rows, F, torch.float32, DEV)
    G.copy_(torch.randn(gb.A.n_rows, F, device=DEV, generator=g))
    say("gat over a split matrix")
    ref = [t.clone() for t in _gat_pass(gb, H, W, asrc, adst, b, G)]
    for M in (gb.A, gb.AT):
        sag.csr_hub_split(M, 50, 64, levels=3)
    got = _gat_pass(gb, H, W, asrc, adst, b, G)
    for a, r in zip(got, ref):
        assert torch.equal(a, r)
