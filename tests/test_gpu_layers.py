"""GPU GCN and GraphSAGE-mean layers (forward and backward) against the
oracle, on the workloads' graphs at reduced size and on synthetic shapes
that take each association order (aggregate first when d_in <= d_out,
transform first otherwise).

Each case pulls the halo rows from a seeded stale buffer on the GPU
(halo gather), builds the CSR on the GPU, runs the layer, and compares
Out / Y_pre, then dW, db and dH_ext, with the error measured against the
same expressions on absolute values: <= 1e-5 for fp32 storage, <= 2e-2 for
bf16.  The backward of both sides gets the same ReLU mask input: the
oracle's forward Y in the storage type."""
import numpy as np
import pytest
import torch

import gen
from oracle import csr as ocsr, layers as olay

pytestmark = pytest.mark.gpu

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from gpu_util import DEV, elementwise_rel, f64, round_to, say, to_dev, to_dev_dense, tol  # noqa: E402


def _err(got, ref, den):
    return float(np.max(np.abs(got - ref) / (den + 1e-30))) if np.size(ref) else 0.0


def _bits_or_f32(x, dt):
    return gen.f32_to_bf16_bits(np.asarray(x, np.float32)) if dt == "bf16" else np.asarray(x, np.float32)


def run_case(model, dt, src, dst, n_global, lo, hi, sym, loops, norm, d_in, d_out, relu,
             stale_rows=0, stale_base=0, seed=0, seg_len=256, label="", fused=False, hub_cols=None,
             col_slices=False):
    g = np.random.default_rng(seed)
    n_l = hi - lo
    say(f"layer {label} model={model} dt={dt} n_global={n_global} [{lo},{hi}) {d_in}->{d_out}")
    ob = ocsr.build(src, dst, n_global, lo, hi, sym, loops, norm)
    n_h = ob.n_halo
    H_loc = _bits_or_f32(g.standard_normal((n_l, d_in)), dt)
    stale = _bits_or_f32(g.standard_normal((max(stale_rows, 1), d_in)), dt)
    w_rows = 2 * d_in if model == "sage" else d_in
    lim = np.sqrt(6.0 / (w_rows + d_out))
    W = _bits_or_f32(g.uniform(-lim, lim, (w_rows, d_out)), dt)
    b = g.uniform(-0.1, 0.1, d_out).astype(np.float32)
    G = _bits_or_f32(g.standard_normal((n_l, d_out)), dt)

    # ---- GPU: build, pull the halo rows, forward
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), n_global, lo, hi, sym, loops, norm)
    assert gb.n_halo == n_h
    if seg_len:
        sag.csr_schedule(gb.A, seg_len)
        sag.csr_schedule(gb.AT, seg_len)
    if hub_cols:
        # both products of the layer take two passes (hub part, cold part)
        sag.csr_hub_split(gb.A, hub_cols, seg_len or 1024)
        sag.csr_hub_split(gb.AT, hub_cols, seg_len or 1024)
    if col_slices:
        # products with rows over 256 bytes take one pass per 128-byte column slice
        sag.csr_set_col_slices(gb.A, True)
        sag.csr_set_col_slices(gb.AT, True)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    H_ext = sag.empty_dense(n_l + n_h, d_in, tdt, DEV)
    H_ext[:n_l].copy_(to_dev_dense(H_loc, dt))
    if n_h:
        sag.halo_gather(to_dev_dense(stale, dt), gb.halo_gid, H_ext[n_l:], row_base=stale_base)
    Wd = to_dev_dense(W, dt).contiguous()
    bd = to_dev(b)
    fwd = sag.gcn_layer_forward if model == "gcn" else sag.sage_layer_forward
    Out, Ypre, ctx = fwd(gb.A, H_ext, Wd, bd, relu=relu, want_pre=True, fused=fused)

    # ---- oracle forward
    H64 = olay.as_f64(np.concatenate([H_loc, ocsr.gather(stale, ocsr.halo_rows(ob, stale_base))]), dt)
    W64 = olay.as_f64(W, dt)
    if model == "gcn":
        Zr, Yr, Outr = olay.gcn_forward(ob.A, H64, W64, b, relu)
        _, Yd = olay.gcn_forward_den(ob.A, H64, W64, b)
    else:
        Mr, Yr, Outr = olay.sage_forward(ob.A, H64, n_l, W64, b, relu)
        _, Yd = olay.sage_forward_den(ob.A, H64, n_l, W64, b)
    e_out = _err(f64(Out), Outr, Yd)
    e_pre = _err(f64(Ypre), Yr, Yd)
    say(f"  forward err {e_pre:.2e} of the bound; per element {elementwise_rel(f64(Ypre), Yr):.2e}")
    assert e_out <= tol(dt) and e_pre <= tol(dt), f"{label}: forward err out {e_out:.2e} pre {e_pre:.2e}"

    # ---- backward with the same mask input on both sides
    Ymask = round_to(Yr, dt)
    Ym64 = olay.as_f64(Ymask, dt)
    G64 = olay.as_f64(G, dt)
    bwd = sag.gcn_layer_backward if model == "gcn" else sag.sage_layer_backward
    dW, db, dH = bwd(ctx, gb.AT, n_l, to_dev_dense(Ymask, dt), to_dev_dense(G, dt))
    if model == "gcn":
        rdW, rdb, _, rdH = olay.gcn_backward(ob.AT, Zr, W64, Ym64, relu, G64)
        dWd, dbd, _, dHd = olay.gcn_backward_den(ob.AT, Zr, W64, Ym64, relu, G64)
    else:
        rdW, rdb, rdH = olay.sage_backward(ob.AT, H64[:n_l], Mr, W64, Ym64, relu, G64)
        dWd, dbd, dHd = olay.sage_backward_den(ob.AT, H64[:n_l], Mr, W64, Ym64, relu, G64)
    errs = {"dW": _err(f64(dW), rdW, dWd), "db": _err(f64(db), rdb, dbd), "dH": _err(f64(dH), rdH, dHd)}
    for k, e in errs.items():
        assert e <= tol(dt), f"{label}: {k} err {e:.2e}"
    return e_out, errs


# ---- the workloads' recipes at reduced size --------------------------------------

def test_tiny_gcn_layer_full_size():
    """4,096-node uniform graph, GCN 64 -> 16 fp32, one forward + backward."""
    w = gen.make_config(1)
    src, dst = w.edges
    run_case("gcn", "f32", src, dst, w.n_global, 0, w.n_global, True, True, "gcn", 64, 16, True,
             label="tiny GCN")


@pytest.mark.parametrize("d_in,d_out,relu", [(602, 128, True), (128, 41, False)])
def test_power_law_gcn_layers(d_in, d_out, relu):
    w = gen.make_config(2, 0.005)
    src, dst = w.edges
    run_case("gcn", "f32", src, dst, w.n_global, 0, w.n_global, True, True, "gcn", d_in, d_out, relu,
             seed=d_in, label="power-law GCN")


@pytest.mark.parametrize("hub_cols", [1, 64, 700])
@pytest.mark.parametrize("model,dt,d_in,d_out,relu", [("gcn", "f32", 602, 128, True), ("gcn", "f32", 128, 41, False),
                                                      ("sage", "bf16", 100, 256, True), ("sage", "f32", 256, 47, False)])
def test_layers_over_hub_split(hub_cols, model, dt, d_in, d_out, relu):
    """The dense power-law graph with both of the layer's matrices split
    (the SAGE cases: the mean-normalised A, whose parts carry its values)."""
    w = gen.make_config(2, 0.004)
    src, dst = w.edges
    run_case(model, dt, src, dst, w.n_global, 0, w.n_global, True, True, "gcn" if model == "gcn" else "mean",
             d_in, d_out, relu, seed=hub_cols + d_in, seg_len=128, label="hub split", hub_cols=hub_cols)


def test_fused_layer_over_hub_split():
    """The fused aggregate -> transform kernel reads the matrix's own arrays,
    so it runs (and matches the oracle) over a split matrix too."""
    w = gen.make_config(2, 0.004)
    src, dst = w.edges
    run_case("sage", "bf16", src, dst, w.n_global, 0, w.n_global, True, True, "mean", 100, 256, True, seed=9,
             seg_len=128, label="fused over hub split", fused=True, hub_cols=64)


@pytest.mark.parametrize("model,dt,d_in,d_out,relu", [("gcn", "f32", 602, 128, True), ("gcn", "f32", 96, 200, False),
                                                      ("sage", "bf16", 256, 256, True), ("sage", "f32", 256, 160, True),
                                                      ("sage", "bf16", 300, 47, False)])
def test_layers_over_column_slices(model, dt, d_in, d_out, relu):
    """Both of the layer's matrices gather in 128-byte column slices: the
    epilogue (bias, Y_pre, ReLU, the SAGE self-term addend) lands on each
    slice's own columns."""
    w = gen.make_config(4, 0.002)
    src, dst = w.edges
    run_case(model, dt, src, dst, w.n_global, 0, w.n_global, True, True, "gcn" if model == "gcn" else "mean",
             d_in, d_out, relu, seed=d_in + d_out, seg_len=64, label="column slices", col_slices=True)


def test_partition_with_halo_over_hub_split():
    w = gen.make_config(3, 1 / 64)
    src, dst = w.edges
    run_case("sage", "f32", src, dst, w.n_global, w.lo, w.hi, True, False, "mean", 64, 96, True,
             stale_rows=w.stale_rows, stale_base=w.stale_base, seed=5, seg_len=64, label="partition hub split",
             hub_cols=300)


def test_rmat_partition_sage_with_stale_halo():
    w = gen.make_config(3, 1 / 64)
    src, dst = w.edges
    run_case("sage", "f32", src, dst, w.n_global, w.lo, w.hi, True, False, "mean", 128, 256, True,
             stale_rows=w.stale_rows, stale_base=w.stale_base, label="R-MAT partition SAGE")


@pytest.mark.parametrize("d_in,d_out,relu", [(100, 256, True), (256, 256, True), (256, 47, False)])
def test_large_sparse_sage_bf16(d_in, d_out, relu):
    w = gen.make_config(4, 0.002)
    src, dst = w.edges
    run_case("sage", "bf16", src, dst, w.n_global, 0, w.n_global, True, True, "mean", d_in, d_out, relu,
             seed=d_out, label="large sparse SAGE")


def test_share_of_large_graph_gcn_bf16():
    w = gen.make_config(5, 0.001)
    src, dst = w.edges
    run_case("gcn", "bf16", src, dst, w.n_global, w.lo, w.hi, False, True, "gcn", 128, 128, True,
             stale_rows=w.stale_rows, stale_base=w.stale_base, label="GCN share with halo")


# ---- both association orders, both storage types, halo and no halo ------------------

@pytest.mark.parametrize("model", ["gcn", "sage"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("d_in,d_out", [(16, 64), (64, 16), (41, 41), (100, 47), (8, 300), (96, 200), (200, 160)])
@pytest.mark.parametrize("halo", [False, True])
def test_orders_and_partitions(model, dt, d_in, d_out, halo):
    g = np.random.default_rng(d_in * 1000 + d_out)
    n = 3000
    m = 12000
    src = g.integers(0, n, m).astype(np.int32)
    dst = g.integers(0, n, m).astype(np.int32)
    lo, hi = (700, 2100) if halo else (0, n)
    norm = "gcn" if model == "gcn" else "mean"
    run_case(model, dt, src, dst, n, lo, hi, True, True, norm, d_in, d_out, True,
             stale_rows=n, stale_base=0, seed=d_in + d_out, seg_len=64, label=f"orders halo={halo}")


def test_no_schedule_path():
    g = np.random.default_rng(0)
    n = 1500
    src = g.integers(0, n, 8000).astype(np.int32)
    dst = g.integers(0, n, 8000).astype(np.int32)
    run_case("sage", "f32", src, dst, n, 0, n, True, True, "mean", 32, 64, True, seg_len=0,
             label="no schedule")


def test_partition_consistency_with_fresh_halo():
    """DIGEST's P_m = P_in + P_out: with the stale buffer equal to the fresh
    features, the local rows of every partition equal the full-graph layer."""
    g = np.random.default_rng(21)
    n, d_in, d_out = 4000, 32, 24
    src = g.integers(0, n, 20000).astype(np.int32)
    dst = g.integers(0, n, 20000).astype(np.int32)
    H = g.standard_normal((n, d_in)).astype(np.float32)
    W = g.uniform(-0.3, 0.3, (d_in, d_out)).astype(np.float32)
    b = g.uniform(-0.1, 0.1, d_out).astype(np.float32)
    Hd = to_dev_dense(H)
    Wd = to_dev(W)
    bd = to_dev(b)
    say("partition consistency: full graph")
    full = sag.csr_build_normalize(to_dev(src), to_dev(dst), n, 0, n, True, True, "gcn")
    ref, _, _ = sag.gcn_layer_forward(full.A, Hd, Wd, bd, relu=True)
    ref = f64(ref)
    parts = []
    for p in range(4):
        lo, hi = p * n // 4, (p + 1) * n // 4
        say(f"partition consistency: part {p}")
        gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), n, lo, hi, True, True, "gcn",
                                     deg_global=full.deg)
        H_ext = sag.empty_dense(gb.A.n_cols, d_in, torch.float32, DEV)
        H_ext[: hi - lo].copy_(Hd[lo:hi])
        if gb.n_halo:
            sag.halo_gather(Hd, gb.halo_gid, H_ext[hi - lo:])
        out, _, _ = sag.gcn_layer_forward(gb.A, H_ext, Wd, bd, relu=True)
        parts.append(f64(out))
    got = np.concatenate(parts)
    assert np.max(np.abs(got - ref)) <= 1e-5 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("model", ["gcn", "sage"])
@pytest.mark.parametrize("d_in,d_out", [(24, 40), (40, 24)])
def test_empty_partition(model, d_in, d_out):
    """A partition with no local rows (lo == hi): nothing to aggregate, the
    outputs have no rows, and the weight and bias gradients -- sums over no
    rows -- are exactly zero (not whatever their buffers held)."""
    g = np.random.default_rng(5)
    n = 300
    src = g.integers(0, n, 900).astype(np.int32)
    dst = g.integers(0, n, 900).astype(np.int32)
    say(f"empty partition {model} {d_in}->{d_out}")
    norm = "gcn" if model == "gcn" else "mean"
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), n, 120, 120, True, True, norm)
    assert gb.n_local == 0 and gb.n_halo == 0
    H = sag.empty_dense(0, d_in, torch.float32, DEV)
    w_rows = 2 * d_in if model == "sage" else d_in
    W = torch.randn(w_rows, d_out, device=DEV)
    b = torch.randn(d_out, device=DEV)
    fwd = sag.gcn_layer_forward if model == "gcn" else sag.sage_layer_forward
    bwd = sag.gcn_layer_backward if model == "gcn" else sag.sage_layer_backward
    Out, _, ctx = fwd(gb.A, H, W, b, relu=True)
    assert Out.shape[0] == 0
    G = sag.empty_dense(0, d_out, torch.float32, DEV)
    dW, db, dH = bwd(ctx, gb.AT, 0, Out, G)
    torch.cuda.synchronize()
    assert dW.shape == (w_rows, d_out) and torch.count_nonzero(dW).item() == 0
    assert torch.count_nonzero(db).item() == 0
    assert dH.shape[0] == 0


@pytest.mark.parametrize("model", ["gcn", "sage"])
def test_rows_without_entries(model):
    """Local rows that aggregate nothing (no edges into the range, no self
    connections): the aggregate is zero, so Out = act(b) (GraphSAGE: act of
    the self term plus b) and the gradients follow, against the oracle."""
    g = np.random.default_rng(6)
    n = 1000
    src = g.integers(0, 500, 3000).astype(np.int32)
    dst = g.integers(0, 500, 3000).astype(np.int32)      # rows 600..899 receive nothing
    run_case(model, "f32", src, dst, n, 600, 900, False, False, "gcn" if model == "gcn" else "mean", 16, 32,
             True, seed=7, label="rows without entries")
