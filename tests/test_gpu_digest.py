"""DIGEST's stale-representation exchange (sparse_aggregation_gemm_amd.digest)
against the oracle: a two-layer model on one partition whose layer inputs
take their halo rows from per-layer stale stores (pull), whose fresh local
rows go into the next layer's store (push) and whose halo input gradients
are added into gradient stores (accumulating push), over two consecutive
steps, with the exchanges on a second stream and on one stream.

Per step, from the GPU stores as they stood before the step: each layer's
output and weight/bias/input gradients match the oracle layers (error
relative to the absolute-value bound, 1e-5 fp32 / 2e-2 bf16), each layer fed
the GPU's previous layer output and the same ReLU mask; the stores after the
step equal the oracle push of the GPU's fresh rows (bit for bit) and the
gradient stores the fp32 sum of their old rows and the GPU's halo gradient
rows, rounded once; the overlapped and one-stream runs give the same bits."""
import numpy as np
import pytest
import torch

import gen
from oracle import csr as ocsr, layers as olay, lowbit as olb

pytestmark = pytest.mark.gpu

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from sparse_aggregation_gemm_amd.digest import StaleExchange  # noqa: E402
from gpu_util import DEV, f64, say, to_dev, to_dev_dense, tol  # noqa: E402


def _bits(t):
    t = t.detach().contiguous()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).cpu().numpy()


def _store_bits(vals_f32, dt):
    v = np.asarray(vals_f32, np.float32)
    if dt == "bf16":
        r = olay.round_bf16(v.astype(np.float64)).astype(np.float32)
        return (r.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)
    return v.view(np.int32)


def _stored(x, dt):
    return gen.f32_to_bf16_bits(np.asarray(x, np.float32)) if dt == "bf16" else np.asarray(x, np.float32)


def _err(got, ref, den):
    return float(np.max(np.abs(got - ref) / (den + 1e-30))) if np.size(ref) else 0.0


def _oracle_layer(model, A, AT, H_ext, n_l, W, b, relu, Ymask, G, want_dH):
    """Oracle forward and backward of one layer: (Out, Yden, dW, db, dH, dens)."""
    if model == "gcn":
        Z, Y, Out = olay.gcn_forward(A, H_ext, W, b, relu)
        _, Yd = olay.gcn_forward_den(A, H_ext, W, b)
        dW, db, _, dH = olay.gcn_backward(AT, Z, W, Ymask, relu, G, want_dH)
        dWd, dbd, _, dHd = olay.gcn_backward_den(AT, Z, W, Ymask, relu, G, want_dH)
    else:
        M, Y, Out = olay.sage_forward(A, H_ext, n_l, W, b, relu)
        _, Yd = olay.sage_forward_den(A, H_ext, n_l, W, b)
        dW, db, dH = olay.sage_backward(AT, H_ext[:n_l], M, W, Ymask, relu, G, want_dH)
        dWd, dbd, dHd = olay.sage_backward_den(AT, H_ext[:n_l], M, W, Ymask, relu, G, want_dH)
    return Out, Yd, dW, db, dH, (dWd, dbd, dHd)


def run_exchange(cfg, scale, model, dt, dims, relu, seed):
    w = gen.make_config(cfg, scale)
    src, dst = w.edges
    norm = "gcn" if model == "gcn" else "mean"
    say(f"digest cfg={cfg} scale={scale} {model} {dt} dims={dims}")
    ob = ocsr.build(src, dst, w.n_global, w.lo, w.hi, w.symmetrize, w.self_loops, norm)
    gb = sag.csr_build_normalize(to_dev(src), to_dev(dst), w.n_global, w.lo, w.hi, w.symmetrize, w.self_loops,
                                 norm)
    sag.csr_schedule(gb.A, 256)
    sag.csr_schedule(gb.AT, 256)
    n_l, n_h, L = ob.n_local, ob.n_halo, len(dims) - 1
    assert n_h > 0
    g = np.random.default_rng(seed)
    base, n_store = 0, w.n_global            # stores over every global id of the share
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    stores0 = [_stored(g.standard_normal((n_store, dims[l])), dt) for l in range(L)]
    gstores0 = [None] + [_stored(g.standard_normal((n_store, dims[l])), dt) for l in range(1, L)]
    H0 = _stored(g.standard_normal((n_l, dims[0])), dt)
    Ws, bs = [], []
    for l in range(L):
        k = (2 if model == "sage" else 1) * dims[l]
        lim = np.sqrt(6.0 / (k + dims[l + 1]))
        Ws.append(_stored(g.uniform(-lim, lim, (k, dims[l + 1])), dt))
        bs.append(g.uniform(-0.1, 0.1, dims[l + 1]).astype(np.float32))
    Gs = [_stored(g.standard_normal((n_l, dims[L])), dt) for _ in range(2)]
    local_ids = np.arange(w.lo, w.hi, dtype=np.int32)

    results = {}
    for overlap in (True, False):
        stores = [to_dev_dense(s, dt) for s in stores0]
        gstores = [None] + [to_dev_dense(s, dt) for s in gstores0[1:]]
        ex = StaleExchange(gb, model, dims, relu, stores, gstores, to_dev(local_ids), store_base=base)
        Wd = [to_dev_dense(x, dt).contiguous() for x in Ws]
        bd = [to_dev(x) for x in bs]
        H0d = to_dev_dense(H0, dt)
        trace = []
        for step in range(2):
            before = [f64(s) for s in stores]
            gbefore = [None] + [f64(s) for s in gstores[1:]]
            res = ex.step(H0d, Wd, bd, to_dev_dense(Gs[step], dt), overlap=overlap)
            torch.cuda.synchronize()
            outs = [f64(ex.H[l + 1][:n_l]) for l in range(L - 1)] + [f64(res.out)]
            trace.append([_bits(x) for x in (res.out, *res.dW, *res.db, *[s for s in stores],
                                             *[s for s in gstores[1:]])])
            if not overlap:
                continue
            # ---- the oracle, layer by layer, on the GPU's layer inputs
            halo_rows = ocsr.halo_rows(ob, base)
            G = olay.as_f64(Gs[step], dt)
            H_ext = []
            for l in range(L):
                local = olay.as_f64(H0, dt) if l == 0 else outs[l - 1]
                H_ext.append(np.concatenate([local, before[l][halo_rows]]))
            grads_in = G
            for l in reversed(range(L)):
                W64, want = olay.as_f64(Ws[l], dt), l > 0
                Out, Yd, dW, db, dH, (dWd, dbd, dHd) = _oracle_layer(
                    model, ob.A, ob.AT, H_ext[l], n_l, W64, bs[l], relu[l], outs[l], grads_in, want)
                e = _err(outs[l], Out, Yd)
                assert e <= tol(dt), f"step {step} layer {l} forward {e:.2e}"
                for name, got, ref, den in (("dW", res.dW[l], dW, dWd), ("db", res.db[l], db, dbd)):
                    e = _err(f64(got), ref, den)
                    assert e <= tol(dt), f"step {step} layer {l} {name} {e:.2e}"
                if want:
                    gdH = f64(res.dH[l])
                    e = _err(gdH, dH, dHd)
                    assert e <= tol(dt), f"step {step} layer {l} dH_ext {e:.2e}"
                    # the returned halo gradients: old rows plus the GPU's halo rows, one rounding
                    exp = gbefore[l].astype(np.float32)
                    exp[halo_rows] = (exp[halo_rows] + gdH[n_l:].astype(np.float32)).astype(np.float32)
                    assert np.array_equal(_bits(gstores[l]), _store_bits(exp, dt)), f"grad store {l}"
                    grads_in = gdH[:n_l]
            # the pushes: store l + 1 holds layer l's fresh local rows, the rest unchanged
            for l in range(L - 1):
                exp = olb.push(before[l + 1], outs[l], local_ids, base)
                assert np.array_equal(_bits(stores[l + 1]), _store_bits(exp, dt)), f"store {l + 1}"
            assert np.array_equal(_bits(stores[0]), _store_bits(before[0], dt))
        results[overlap] = trace
    for a, b in zip(results[True], results[False]):
        for x, y in zip(a, b):
            assert np.array_equal(x, y), "overlapped and one-stream runs differ"


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gcn_share_two_layers(dt):
    """The 100M-graph share's GCN at reduced size (aggregate first, then
    transform first)."""
    run_exchange(5, 0.002, "gcn", dt, [48, 64, 24], [True, False], seed=1)


def test_sage_partition_two_layers():
    """The R-MAT partition's GraphSAGE-mean at reduced size."""
    run_exchange(3, 1 / 64, "sage", "f32", [32, 64, 16], [True, True], seed=2)
