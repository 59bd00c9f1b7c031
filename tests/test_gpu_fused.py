"""GPU fused aggregate -> transform kernel against the oracle.

sag_aggregate_transform computes Z = A H_ext and [H_local | Z] W + b (or
Z W + b) in one kernel.  Its Out, Y_pre and stored Z are compared with the
oracle's GCN / GraphSAGE forward (Z against the SpMM, Out against the
layer), with the error measured against the same expressions on absolute
values: <= 1e-5 for fp32 storage, <= 2e-2 for bf16.  Cases cover rows in
every bin of the schedule (short, medium, and long rows summed by segment
kernels first), no schedule, a partition with halo columns, widths that are
not whole vectors, and the layers with the switch on and off."""
import numpy as np
import pytest
import torch

import gen
from oracle import csr as ocsr, layers as olay

pytestmark = pytest.mark.gpu

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from gpu_util import DEV, f64, say, to_dev, to_dev_dense, tol  # noqa: E402


def _err(got, ref, den):
    return float(np.max(np.abs(got - ref) / (den + 1e-30))) if np.size(ref) else 0.0


def _stored(x, dt):
    return gen.f32_to_bf16_bits(np.asarray(x, np.float32)) if dt == "bf16" else np.asarray(x, np.float32)


def run_fused(dt, src, dst, n_global, lo, hi, sym, loops, norm, d_in, d_out, self_rows, relu, stale_rows=0,
              stale_base=0, seg_len=256, seed=0, label=""):
    g = np.random.default_rng(seed)
    n_l = hi - lo
    say(f"fused {label} dt={dt} [{lo},{hi}) of {n_global} {norm} {d_in}->{d_out} self={self_rows} "
        f"seg_len={seg_len}")
    ob = ocsr.build(src, dst, n_global, lo, hi, sym, loops, norm)
    n_h = ob.n_halo
    H_loc = _stored(g.standard_normal((n_l, d_in)), dt)
    stale = _stored(g.standard_normal((max(stale_rows, 1), d_in)), dt)
    w_rows = 2 * d_in if self_rows else d_in
    lim = np.sqrt(6.0 / (w_rows + d_out))
    W = _stored(g.uniform(-lim, lim, (w_rows, d_out)), dt)
    b = g.uniform(-0.1, 0.1, d_out).astype(np.float32)

    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), n_global, lo, hi, sym, loops, norm)
    if seg_len:
        sag.csr_schedule(gb.A, seg_len)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    H_ext = sag.empty_dense(n_l + n_h, d_in, tdt, DEV)
    H_ext[:n_l].copy_(to_dev_dense(H_loc, dt))
    if n_h:
        sag.halo_gather(to_dev_dense(stale, dt), gb.halo_gid, H_ext[n_l:], row_base=stale_base)
    Out, Ypre, Z = sag.aggregate_transform(gb.A, H_ext, to_dev_dense(W, dt).contiguous(), to_dev(b),
                                           self_rows=self_rows, relu=relu, want_pre=True)

    H64 = olay.as_f64(np.concatenate([H_loc, ocsr.gather(stale, ocsr.halo_rows(ob, stale_base))]), dt)
    W64 = olay.as_f64(W, dt)
    if self_rows:
        Zr, Yr, Or = olay.sage_forward(ob.A, H64, n_l, W64, b, relu)
        Zd, Yd = olay.sage_forward_den(ob.A, H64, n_l, W64, b)
    else:
        Zr, Yr, Or = olay.gcn_forward(ob.A, H64, W64, b, relu)
        Zd, Yd = olay.gcn_forward_den(ob.A, H64, W64, b)
    errs = {"Z": _err(f64(Z), Zr, Zd), "Y_pre": _err(f64(Ypre), Yr, Yd), "Out": _err(f64(Out), Or, Yd)}
    say("  errors: " + " ".join(f"{k} {e:.1e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= tol(dt), f"{label}: {k} err {e:.2e}"
    return errs


def _uniform(seed, n=3000, m=30000):
    g = np.random.default_rng(seed)
    return g.integers(0, n, m).astype(np.int32), g.integers(0, n, m).astype(np.int32), n


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("self_rows", [False, True])
@pytest.mark.parametrize("d_in,d_out", [(16, 64), (100, 256), (128, 128), (37, 41), (8, 150)])
def test_shapes_on_a_partition(dt, self_rows, d_in, d_out):
    src, dst, n = _uniform(d_in + d_out)
    run_fused(dt, src, dst, n, 400, 2600, True, True, "mean" if self_rows else "gcn", d_in, d_out, self_rows,
              relu=d_out % 2 == 0, stale_rows=n, seed=d_in, label="uniform partition")


@pytest.mark.parametrize("seg_len", [64, 0])
@pytest.mark.parametrize("dt,d_in,d_out", [("f32", 64, 128), ("bf16", 256, 256), ("bf16", 100, 256)])
def test_power_law_rows_in_every_bin(seg_len, dt, d_in, d_out):
    """Short, medium and long rows (seg_len 64: segmented first), and no
    schedule."""
    w = gen.make_config(2, 0.005)
    src, dst = w.edges
    run_fused(dt, src, dst, w.n_global, 0, w.n_global, True, True, "mean", d_in, d_out, True, True,
              seg_len=seg_len, seed=seg_len, label="power-law SAGE")
    run_fused(dt, src, dst, w.n_global, 0, w.n_global, True, True, "gcn", d_in, d_out, False, False,
              seg_len=seg_len, seed=seg_len + 1, label="power-law GCN")


def test_workload_shapes():
    """The large sparse graph's aggregate-first SAGE layers and the share's
    GCN layer, at reduced size."""
    w = gen.make_config(4, 0.002)
    src, dst = w.edges
    for d_in, d_out in [(100, 256), (256, 256)]:
        run_fused("bf16", src, dst, w.n_global, 0, w.n_global, True, True, "mean", d_in, d_out, True, True,
                  seg_len=1024, label="large sparse SAGE")
    w = gen.make_config(5, 0.001)
    src, dst = w.edges
    run_fused("bf16", src, dst, w.n_global, w.lo, w.hi, False, True, "gcn", 128, 128, False, True,
              stale_rows=w.stale_rows, stale_base=w.stale_base, seg_len=1024, label="share GCN")


def test_unsupported_width_is_refused():
    src, dst, n = _uniform(3, n=200, m=800)
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), n, 0, n, True, True, "gcn")
    H = sag.empty_dense(n, 16, torch.float32, DEV, fill=0)
    W = torch.zeros((16, 300), dtype=torch.float32, device=DEV)
    with pytest.raises(Exception, match="aggregate_transform"):
        sag.aggregate_transform(gb.A, H, W)


@pytest.mark.parametrize("fusion", [True, False])
def test_layers_with_and_without_fusion(fusion):
    """The GCN and SAGE layers (aggregate first, forward + backward) agree
    with the oracle both through the fused kernel (SAG_LAYER_FUSED) and
    through the separate SpMM and product."""
    from test_gpu_layers import run_case
    src, dst, n = _uniform(11)
    for model, norm in (("gcn", "gcn"), ("sage", "mean")):
        for dt in ("f32", "bf16"):
            run_case(model, dt, src, dst, n, 300, 2700, True, True, norm, 64, 128, True, stale_rows=n,
                     seed=5, label=f"fusion={fusion}", fused=fusion)


@pytest.mark.parametrize("fusion", [True, False])
@pytest.mark.parametrize("norm", ["none", "gcn"])
def test_sage_layer_on_a_csr_that_is_not_a_mean(fusion, norm):
    """A GraphSAGE layer over a CSR built without the mean normalisation
    (not tagged row_mean) aggregates with the stored values -- a sum for
    SAG_NORM_NONE -- in the fused and the separate forward and in the
    backward alike, as the oracle does with the same CSR."""
    from test_gpu_layers import run_case
    src, dst, n = _uniform(17)
    for dt in ("f32", "bf16"):
        run_case("sage", dt, src, dst, n, 200, 2500, True, True, norm, 48, 96, True, stale_rows=n, seed=9,
                 label=f"sage over a {norm} CSR, fusion={fusion}", fused=fusion)
