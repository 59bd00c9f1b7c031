"""GPU graph-attention layer (forward and backward) against the oracle.

Each case builds the CSR and its transpose on the GPU (pattern only, with
self connections unless stated), pulls the halo rows from a seeded stale
buffer, runs the layer and its backward, and compares Out, dW, da_src,
da_dst, db and dH_ext with the oracle's.  The error is measured against the
same expressions on absolute values with the softmax weights scaled by the
sensitivity of their exponent (oracle ``*_den``): <= 1e-5 for fp32 storage,
<= 2e-2 for bf16.  Both backward passes get the same ReLU mask input, the
oracle's forward Y in the storage type.  Cases cover one and many heads,
head widths from one 16-byte vector to 64 of them, rows in every bin of the
schedule (short, medium, segmented long rows), no schedule, rows without
entries, and the workloads' graphs at reduced size."""
import numpy as np
import pytest
import torch

import gen
from oracle import csr as ocsr, gat as ogat, layers as olay

pytestmark = pytest.mark.gpu

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from gpu_util import DEV, f64, round_to, say, to_dev, to_dev_dense, tol  # noqa: E402


def _err(got, ref, den):
    return float(np.max(np.abs(got - ref) / (den + 1e-30))) if np.size(ref) else 0.0


def _stored(x, dt):
    return gen.f32_to_bf16_bits(np.asarray(x, np.float32)) if dt == "bf16" else np.asarray(x, np.float32)


def run_gat(dt, src, dst, n_global, lo, hi, sym, loops, d_in, heads, dh, relu, slope=0.2, stale_rows=0,
            stale_base=0, seed=0, seg_len=256, label=""):
    g = np.random.default_rng(seed)
    n_l = hi - lo
    F = heads * dh
    say(f"gat {label} dt={dt} n_global={n_global} [{lo},{hi}) d_in={d_in} heads={heads}x{dh} relu={relu} "
        f"seg_len={seg_len}")
    ob = ocsr.build(src, dst, n_global, lo, hi, sym, loops, "none")
    n_h = ob.n_halo
    H_loc = _stored(g.standard_normal((n_l, d_in)), dt)
    stale = _stored(g.standard_normal((max(stale_rows, 1), d_in)), dt)
    lim = np.sqrt(6.0 / (d_in + F))
    W = _stored(g.uniform(-lim, lim, (d_in, F)), dt)
    la = np.sqrt(6.0 / (dh + 1))
    a_src = g.uniform(-la, la, (heads, dh)).astype(np.float32)
    a_dst = g.uniform(-la, la, (heads, dh)).astype(np.float32)
    b = g.uniform(-0.1, 0.1, F).astype(np.float32)
    G = _stored(g.standard_normal((n_l, F)), dt)

    # ---- GPU: build, schedule, pull the halo rows, forward
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), n_global, lo, hi, sym, loops, "none")
    assert gb.n_halo == n_h
    if seg_len:
        sag.csr_schedule(gb.A, seg_len)
        sag.csr_schedule(gb.AT, seg_len)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    H_ext = sag.empty_dense(n_l + n_h, d_in, tdt, DEV)
    H_ext[:n_l].copy_(to_dev_dense(H_loc, dt))
    if n_h:
        sag.halo_gather(to_dev_dense(stale, dt), gb.halo_gid, H_ext[n_l:], row_base=stale_base)
    Out, ctx = sag.gat_layer_forward(gb.A, H_ext, to_dev_dense(W, dt).contiguous(), to_dev(a_src), to_dev(a_dst),
                                     to_dev(b), heads=heads, slope=slope, relu=relu)

    # ---- oracle forward
    H64 = olay.as_f64(np.concatenate([H_loc, ocsr.gather(stale, ocsr.halo_rows(ob, stale_base))]), dt)
    W64 = olay.as_f64(W, dt)
    f = ogat.gat_forward(ob.A, H64, W64, a_src, a_dst, b, heads, slope, relu, store=dt)
    sw = score_weight(d_in, dh, dt)
    Yd = ogat.gat_forward_den(ob.A, f, b, heads, H64, W64, a_src, a_dst, sw)
    e_out = _err(f64(Out), f["Out"], Yd)
    e_plain = _err(f64(Out), f["Out"], ogat.gat_forward_den(ob.A, f, b, heads, H64, W64, a_src, a_dst))
    assert e_out <= tol(dt), f"{label}: forward err {e_out:.2e}"

    # ---- backward with the same mask input on both sides
    Ymask = round_to(f["Y"], dt)
    Ym64 = olay.as_f64(Ymask, dt)
    G64 = olay.as_f64(G, dt)
    dW, da_src, da_dst, db, dH = sag.gat_layer_backward(ctx, gb.A, gb.AT, to_dev_dense(Ymask, dt),
                                                        to_dev_dense(G, dt))
    r = ogat.gat_backward(ob.A, H64, W64, a_src, a_dst, heads, slope, relu, f, Ym64, G64, store=dt)
    d = ogat.gat_backward_den(ob.A, H64, W64, a_src, a_dst, heads, slope, relu, f, Ym64, G64, sw)
    errs = {k: _err(f64(v), r[k], d[k]) for k, v in
            (("dW", dW), ("da_src", da_src), ("da_dst", da_dst), ("db", db), ("dH_ext", dH))}
    say(f"  errors: out {e_out:.1e} (plain {e_plain:.1e}) " + " ".join(f"{k} {e:.1e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= tol(dt), f"{label}: {k} err {e:.2e}"
    return e_out, errs


def score_weight(d_in, dh, dt):
    """Weight of the score magnitude in the error bound: the exponent of a
    softmax weight comes from fp32 sums of d_in (transform) and d_head
    (score) terms and a few more operations, so its absolute error is at
    most about (d_in + d_head + 8) eps32 S; relative to the allowed error."""
    return (d_in + dh + 8) * 2.0 ** -24 / tol(dt)


def _uniform_partition(seed, n=3000, m=24000, lo=500, hi=2700):
    g = np.random.default_rng(seed)
    return g.integers(0, n, m).astype(np.int32), g.integers(0, n, m).astype(np.int32), n, lo, hi


# ---- head layouts, both storage types, a partition with halo rows -------------------------

@pytest.mark.parametrize("dt,heads,dh,relu", [
    ("f32", 1, 4, True), ("f32", 2, 8, False), ("f32", 4, 16, True), ("f32", 2, 32, True),
    ("f32", 8, 4, False),
    ("bf16", 1, 8, True), ("bf16", 4, 8, False), ("bf16", 2, 32, True), ("bf16", 4, 64, True),
    ("bf16", 1, 128, False),
])
def test_heads_on_a_partition(dt, heads, dh, relu):
    src, dst, n, lo, hi = _uniform_partition(heads * 100 + dh)
    stale_rows = n
    run_gat(dt, src, dst, n, lo, hi, True, True, 24, heads, dh, relu, stale_rows=stale_rows, stale_base=0,
            seed=heads + dh, label="uniform partition")


@pytest.mark.parametrize("dt,heads,dh", [("f32", 4, 256), ("bf16", 2, 512), ("f32", 16, 16)])
def test_widest_rows(dt, heads, dh):
    """F at the widest the lanes take (1024 fp32 / bf16 rows of 64 and 128
    vectors, head widths of 64 vectors) and many heads."""
    src, dst, n, lo, hi = _uniform_partition(7, n=600, m=3000, lo=100, hi=500)
    run_gat(dt, src, dst, n, lo, hi, True, True, 16, heads, dh, True, stale_rows=n, seed=dh,
            label="widest rows")


@pytest.mark.parametrize("seg_len", [64, 0])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_power_law_rows_in_every_bin(seg_len, dt):
    """A dense-ish power-law graph: short, medium and segmented long rows
    (seg_len 64), and the same graph without a schedule (all rows one
    wavefront each)."""
    w = gen.make_config(2, 0.005)
    src, dst = w.edges
    run_gat(dt, src, dst, w.n_global, 0, w.n_global, True, True, 32, 4, 16 if dt == "f32" else 32, True,
            seg_len=seg_len, seed=seg_len + 1, label="power-law")


def test_rows_without_entries_and_slope():
    """No self connections and isolated nodes: empty rows give act(b) and no
    gradient through the attention; a small negative slope."""
    g = np.random.default_rng(3)
    n = 800
    src = g.integers(0, 400, 1500).astype(np.int32)
    dst = g.integers(0, 400, 1500).astype(np.int32)     # rows 400..799 have no entries
    run_gat("f32", src, dst, n, 0, n, False, False, 20, 2, 8, True, slope=0.01, label="empty rows")


# ---- the workloads' graphs at reduced size ------------------------------------------------

def test_rmat_partition_with_stale_halo():
    w = gen.make_config(3, 1 / 64)
    src, dst = w.edges
    run_gat("f32", src, dst, w.n_global, w.lo, w.hi, True, False, 128, 8, 16, True,
            stale_rows=w.stale_rows, stale_base=w.stale_base, label="R-MAT partition")


def test_large_sparse_graph_bf16():
    w = gen.make_config(4, 0.002)
    src, dst = w.edges
    run_gat("bf16", src, dst, w.n_global, 0, w.n_global, True, True, 256, 4, 64, True, label="large sparse")


def test_share_of_large_graph_bf16():
    w = gen.make_config(5, 0.001)
    src, dst = w.edges
    run_gat("bf16", src, dst, w.n_global, w.lo, w.hi, False, True, 128, 4, 32, True,
            stale_rows=w.stale_rows, stale_base=w.stale_base, label="share with halo")


def test_empty_partition():
    """No local rows: every gradient is a sum over nothing, exactly zero."""
    g = np.random.default_rng(8)
    n, d_in, heads, dh = 300, 16, 2, 8
    src = g.integers(0, n, 900).astype(np.int32)
    dst = g.integers(0, n, 900).astype(np.int32)
    say("gat empty partition")
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), n, 50, 50, True, True, "none")
    assert gb.n_local == 0 and gb.n_halo == 0
    H = sag.empty_dense(0, d_in, torch.float32, DEV)
    W = torch.randn(d_in, heads * dh, device=DEV)
    a = torch.randn(heads, dh, device=DEV)
    Out, ctx = sag.gat_layer_forward(gb.A, H, W, a, a, torch.randn(heads * dh, device=DEV), heads=heads)
    assert Out.shape[0] == 0
    G = sag.empty_dense(0, heads * dh, torch.float32, DEV)
    dW, da_src, da_dst, db, dH = sag.gat_layer_backward(ctx, gb.A, gb.AT, Out, G)
    torch.cuda.synchronize()
    for t in (dW, da_src, da_dst, db):
        assert torch.count_nonzero(t).item() == 0
    assert dH.shape[0] == 0
