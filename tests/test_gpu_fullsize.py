"""Parity at the workloads' full sizes, in the configuration bench.py times
(GPU CSR build with the degree-binned schedule, each matrix's automatic
segment length (1024 or 4096 entries by its size), the chain of
hub splits on matrices whose rows average at least 128 entries: the dense
GCN graph's, and column slices on every other A: the choice the bench's
set-up timing makes for the A of the workloads whose rows are wide enough),
on outputs the oracle can compute one row at a time.

For each workload the graph is drawn at full size and built on the GPU; the
halo list is compared whole, and a sample of rows (random ones plus the
longest and the shortest) entry by entry.  Each layer shape then runs with
seeded inputs of its own width: the forward is compared on the sampled rows;
the backward gets an upstream gradient that is zero except on a second row
sample, so dW, db and every row of dH_ext have exact references built from
those rows alone (a small CSR of the sampled rows and their neighbours,
passed to the oracle's layer functions); every dH_ext row outside those
neighbourhoods must be exactly zero.  On the 2.45M-node graph the oracle
also builds the whole CSR and its transpose (compared with the GPU build bit
for bit) and the d = 256 products over both are compared element by element
in full against its OpenMP fp64 SpMM on the host's cores."""
import numpy as np
import pytest
import torch

import gen
from oracle import csr as ocsr, gat as ogat, layers as olay, native

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from gpu_util import DEV, f64, round_to, say, to_dev, to_dev_dense, tol  # noqa: E402

SEG_LEN = None   # each matrix's own auto_seg_len, as the bench schedules


def _bits_or_f32(x, dt):
    return gen.f32_to_bf16_bits(np.asarray(x, np.float32)) if dt == "bf16" else np.asarray(x, np.float32)


class Full:
    """One workload at full size: edges, GPU build, halo list by definition."""

    def __init__(self, cfg):
        self.w = w = gen.make_config(cfg)
        say(f"full-size workload {cfg}: drawing the graph")
        self.src, self.dst = w.edges
        say(f"full-size workload {cfg}: {self.src.size} edge records; GPU build")
        self.gb = sag.csr_build_normalize(to_dev(self.src), to_dev(self.dst), w.n_global, w.lo, w.hi,
                                          w.symmetrize, w.self_loops, w.norm)
        sag.csr_schedule(self.gb.A, SEG_LEN)
        sag.csr_schedule(self.gb.AT, SEG_LEN)
        for M in (self.gb.A, self.gb.AT):
            if sag.hub_split_pays(M):
                sag.csr_hub_split(M, seg_len=SEG_LEN)
                say(f"full-size workload {cfg}: hub chain of {len(sag.hub_chain(M)) - 1} groups")
        if self.gb.A.hub_part is None:
            sag.csr_set_col_slices(self.gb.A, True)
        torch.cuda.synchronize()
        self.n_l = w.hi - w.lo
        # HALO list by definition: distinct sources outside [lo, hi) of edges into the range
        s = self.src.astype(np.int64)
        d = self.dst.astype(np.int64)
        into = (d >= w.lo) & (d < w.hi)
        rem = s[into & ((s < w.lo) | (s >= w.hi)) & (s != d)]
        if w.symmetrize:
            into2 = (s >= w.lo) & (s < w.hi)
            rem = np.concatenate([rem, d[into2 & ((d < w.lo) | (d >= w.hi)) & (s != d)]])
        self.halo = np.unique(rem)
        # degree proxy (edge records per local row) to pick long and short rows
        cnt = np.bincount(d[into] - w.lo, minlength=self.n_l)
        if w.symmetrize:
            cnt = cnt + np.bincount(s[(s >= w.lo) & (s < w.hi)] - w.lo, minlength=self.n_l)
        self.count = cnt

    def sample(self, n_random, seed, n_extreme=4):
        g = np.random.default_rng(seed)
        order = np.argsort(self.count, kind="stable")
        pick = np.concatenate([g.choice(self.n_l, n_random, replace=False), order[-n_extreme:],
                               order[:n_extreme]])
        return np.unique(pick) + self.w.lo

    def global_id(self, c):
        """Global id of the build's column c (local columns first, then the
        halo in ascending global id)."""
        c = np.asarray(c, np.int64)
        out = c + self.w.lo
        h = c >= self.n_l
        out[h] = self.halo[c[h] - self.n_l]
        return out

    def gpu_row(self, gid):
        gid = np.asarray(gid, np.int64)
        local = (gid >= self.w.lo) & (gid < self.w.hi)
        return np.where(local, gid - self.w.lo, self.n_l + np.searchsorted(self.halo, gid))

    def mini(self, rows):
        """CSR of `rows` over [rows ; their neighbours] (global ids) from the
        oracle's row-by-row build."""
        w = self.w
        rr = ocsr.build_rows(self.src, self.dst, w.n_global, w.lo, w.hi, w.symmetrize, w.self_loops, w.norm,
                             rows)
        nb = np.unique(np.concatenate([c for c, _ in rr]))
        ext = np.concatenate([np.asarray(rows, np.int64), nb])
        indptr = np.zeros(len(rows) + 1, np.int64)
        indptr[1:] = np.cumsum([c.size for c, _ in rr])
        indices = np.concatenate([len(rows) + np.searchsorted(nb, c) for c, _ in rr]).astype(np.int32)
        values = np.concatenate([v for _, v in rr]).astype(np.float32)
        A = ocsr.CSR(len(rows), ext.size, indptr, indices, values)
        return A, ext


_CACHE = {}


def _full(cfg):
    """The workload's Full, kept while consecutive cases use it."""
    if cfg not in _CACHE:
        _CACHE.clear()
        torch.cuda.empty_cache()
        _CACHE[cfg] = Full(cfg)
    return _CACHE[cfg]


@pytest.fixture(scope="module", autouse=True)
def _release():
    yield
    _CACHE.clear()
    torch.cuda.empty_cache()


# (workload, layer): layer None is the build check; each workload's cases are
# consecutive so its graph is drawn and built once; "gat" runs a graph-
# attention layer on the same graph (its pattern only)
CASES = [(2, None), (2, 0), (2, 1), (3, None), (3, 0), (4, None), (4, 0), (4, 1), (4, 2), (4, "fused"),
         (4, "gat"), (4, "full_output"), (5, None), (5, 0), (5, "fused"), (5, "gat")]
# "fused" runs the fused aggregate -> transform kernel at the widest
# aggregate-first layer of the workload
# graph-attention layer per workload: (d_in, heads, d_head)
GAT = {4: (256, 4, 64), 5: (128, 4, 32)}


def _case_id(c, l):
    return f"workload{c}-" + ("build" if l is None else (l if isinstance(l, str) else f"layer{l}"))


@pytest.mark.parametrize("cfg,layer", CASES, ids=[_case_id(c, l) for c, l in CASES])
def test_full_size(cfg, layer):
    full = _full(cfg)
    assert full.w.n_layers == max(l for c, l in CASES if c == cfg and isinstance(l, int)) + 1
    if layer is None:
        check_build(full)
    elif layer == "gat":
        check_gat(full, *GAT[cfg])
    elif layer == "fused":
        check_fused(full)
    elif layer == "full_output":
        check_full_output(full)
    else:
        check_layer(full, layer)


def check_build(full):
    w = full.w
    gb = full.gb
    say(f"full-size build check, workload {w.cfg}")
    assert np.array_equal(gb.halo_gid.cpu().numpy().astype(np.int64), full.halo)
    assert gb.A.n_cols == full.n_l + full.halo.size
    indptr = gb.A.indptr.cpu().numpy()
    assert indptr[0] == 0 and np.all(np.diff(indptr) >= 0) and indptr[-1] == gb.A.nnz
    assert gb.AT.nnz == gb.A.nnz
    rows = full.sample(200, seed=7)
    ref = ocsr.build_rows(full.src, full.dst, w.n_global, w.lo, w.hi, w.symmetrize, w.self_loops, w.norm, rows)
    idx = gb.A.indices.cpu().numpy()
    val = gb.A.values.cpu().numpy()
    for r, (cols, vals) in zip(rows, ref):
        i = r - w.lo
        s, e = indptr[i], indptr[i + 1]
        c = idx[s:e].astype(np.int64)
        assert np.all(np.diff(c) > 0)
        glob = full.global_id(c)
        order = np.argsort(glob)
        assert np.array_equal(glob[order], cols), f"row {r}"
        assert np.array_equal(val[s:e][order].view(np.uint32), vals.view(np.uint32)), f"row {r}"


def _layer_shapes(w):
    return [(l, w.dims[l], w.dims[l + 1], w.relu[l]) for l in range(w.n_layers)]


def check_layer(full, layer):
    w = full.w
    _, d_in, d_out, relu = _layer_shapes(w)[layer]
    dt = w.dtype
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    g = np.random.default_rng(100 * w.cfg + layer)
    n_l, n_h = full.n_l, full.halo.size
    say(f"full-size layer {layer} of workload {w.cfg}: {d_in} -> {d_out} {dt}")
    feats = _bits_or_f32(g.standard_normal((n_l, d_in), dtype=np.float32), dt)
    stale = _bits_or_f32(g.standard_normal((max(w.stale_rows, 1), d_in), dtype=np.float32), dt) \
        if n_h else None
    w_rows = 2 * d_in if w.model == "sage" else d_in
    lim = np.sqrt(6.0 / (w_rows + d_out))
    W = _bits_or_f32(g.uniform(-lim, lim, (w_rows, d_out)), dt)
    b = g.uniform(-0.1, 0.1, d_out).astype(np.float32)

    # ---- GPU: pull the halo, forward over the whole partition
    H_ext = sag.empty_dense(n_l + n_h, d_in, tdt, DEV)
    H_ext[:n_l].copy_(to_dev_dense(feats, dt))
    if n_h:
        sag.halo_gather(to_dev_dense(stale, dt), full.gb.halo_gid, H_ext[n_l:], row_base=w.stale_base)
    Wd = to_dev_dense(W, dt).contiguous()
    fwd = sag.gcn_layer_forward if w.model == "gcn" else sag.sage_layer_forward
    Out, Ypre, ctx = fwd(full.gb.A, H_ext, Wd, to_dev(b), relu=relu, want_pre=True)

    def h_of(gid):
        gid = np.asarray(gid, np.int64)
        local = (gid >= w.lo) & (gid < w.hi)
        out = np.empty((gid.size, d_in), np.float64)
        out[local] = olay.as_f64(feats[gid[local] - w.lo], dt)
        if (~local).any():
            out[~local] = olay.as_f64(stale[gid[~local] - w.stale_base], dt)
        return out

    W64 = olay.as_f64(W, dt)
    # ---- forward on sampled rows
    rows = full.sample(300, seed=11 + layer)
    A_s, ext = full.mini(rows)
    H_s = h_of(ext)
    if w.model == "gcn":
        _, Yr, Or = olay.gcn_forward(A_s, H_s, W64, b, relu)
        _, Yd = olay.gcn_forward_den(A_s, H_s, W64, b)
    else:
        _, Yr, Or = olay.sage_forward(A_s, H_s, len(rows), W64, b, relu)
        _, Yd = olay.sage_forward_den(A_s, H_s, len(rows), W64, b)
    li = rows - w.lo
    e_out = np.max(np.abs(f64(Out)[li] - Or) / (Yd + 1e-30))
    e_pre = np.max(np.abs(f64(Ypre)[li] - Yr) / (Yd + 1e-30))
    assert e_out <= tol(dt) and e_pre <= tol(dt), f"forward err {e_out:.2e} {e_pre:.2e}"

    # ---- backward with the upstream gradient supported on a row sample
    rows_b = full.sample(120, seed=21 + layer, n_extreme=2)
    A_b, ext_b = full.mini(rows_b)
    H_b = h_of(ext_b)
    if w.model == "gcn":
        Zb, Yb, _ = olay.gcn_forward(A_b, H_b, W64, b, relu)
    else:
        Mb, Yb, _ = olay.sage_forward(A_b, H_b, len(rows_b), W64, b, relu)
    Gb = _bits_or_f32(g.standard_normal((len(rows_b), d_out), dtype=np.float32), dt)
    Ymask = round_to(Yb, dt)
    G_full = np.zeros((n_l, d_out), np.uint16 if dt == "bf16" else np.float32)
    Y_full = np.zeros_like(G_full)
    G_full[rows_b - w.lo] = Gb
    Y_full[rows_b - w.lo] = Ymask
    bwd = sag.gcn_layer_backward if w.model == "gcn" else sag.sage_layer_backward
    dW, db, dH = bwd(ctx, full.gb.AT, n_l, to_dev_dense(Y_full, dt), to_dev_dense(G_full, dt))
    AT_b = ocsr.transpose(A_b)
    Ym64, G64 = olay.as_f64(Ymask, dt), olay.as_f64(Gb, dt)
    if w.model == "gcn":
        rdW, rdb, _, rdH = olay.gcn_backward(AT_b, Zb, W64, Ym64, relu, G64)
        dWd, dbd, _, dHd = olay.gcn_backward_den(AT_b, Zb, W64, Ym64, relu, G64)
    else:
        rdW, rdb, rdH = olay.sage_backward(AT_b, H_b[:len(rows_b)], Mb, W64, Ym64, relu, G64)
        dWd, dbd, dHd = olay.sage_backward_den(AT_b, H_b[:len(rows_b)], Mb, W64, Ym64, relu, G64)
    e_dw = np.max(np.abs(f64(dW) - rdW) / (dWd + 1e-30))
    e_db = np.max(np.abs(f64(db) - rdb) / (dbd + 1e-30))
    assert e_dw <= tol(dt) and e_db <= tol(dt), f"dW err {e_dw:.2e} db err {e_db:.2e}"
    # dH_ext: reference by global id (a sampled row can also be another's neighbour)
    uniq, inv = np.unique(ext_b, return_inverse=True)
    ref = np.zeros((uniq.size, d_in))
    den = np.zeros((uniq.size, d_in))
    np.add.at(ref, inv, rdH)
    np.add.at(den, inv, dHd)
    got = f64(dH)
    gi = full.gpu_row(uniq)
    e_dh = np.max(np.abs(got[gi] - ref) / (den + 1e-30))
    assert e_dh <= tol(dt), f"dH err {e_dh:.2e}"
    others = np.ones(got.shape[0], bool)
    others[gi] = False
    assert np.all(got[others] == 0.0), "rows outside the sampled neighbourhoods must be zero"


def check_gat(full, d_in, heads, dh):
    """The graph-attention layer over the whole partition; the forward on
    sampled rows, the backward with an upstream gradient supported on a
    second row sample (its exact references come from the small CSR of
    those rows and their neighbours: entries of other rows carry zero
    gradient and contribute nothing)."""
    w = full.w
    dt = w.dtype
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    F = heads * dh
    g = np.random.default_rng(1000 + w.cfg)
    n_l, n_h = full.n_l, full.halo.size
    say(f"full-size GAT layer of workload {w.cfg}: {d_in} -> {heads} x {dh} {dt}")
    feats = _bits_or_f32(g.standard_normal((n_l, d_in), dtype=np.float32), dt)
    stale = _bits_or_f32(g.standard_normal((max(w.stale_rows, 1), d_in), dtype=np.float32), dt) \
        if n_h else None
    lim = np.sqrt(6.0 / (d_in + F))
    W = _bits_or_f32(g.uniform(-lim, lim, (d_in, F)), dt)
    la = np.sqrt(6.0 / (dh + 1))
    a_src = g.uniform(-la, la, (heads, dh)).astype(np.float32)
    a_dst = g.uniform(-la, la, (heads, dh)).astype(np.float32)
    b = g.uniform(-0.1, 0.1, F).astype(np.float32)

    H_ext = sag.empty_dense(n_l + n_h, d_in, tdt, DEV)
    H_ext[:n_l].copy_(to_dev_dense(feats, dt))
    if n_h:
        sag.halo_gather(to_dev_dense(stale, dt), full.gb.halo_gid, H_ext[n_l:], row_base=w.stale_base)
    Out, ctx = sag.gat_layer_forward(full.gb.A, H_ext, to_dev_dense(W, dt).contiguous(), to_dev(a_src),
                                     to_dev(a_dst), to_dev(b), heads=heads, relu=True)

    def h_of(gid):
        gid = np.asarray(gid, np.int64)
        local = (gid >= w.lo) & (gid < w.hi)
        out = np.empty((gid.size, d_in), np.float64)
        out[local] = olay.as_f64(feats[gid[local] - w.lo], dt)
        if (~local).any():
            out[~local] = olay.as_f64(stale[gid[~local] - w.stale_base], dt)
        return out

    W64 = olay.as_f64(W, dt)
    rows = full.sample(300, seed=31)
    A_s, ext = full.mini(rows)
    H_s = h_of(ext)
    f = ogat.gat_forward(A_s, H_s, W64, a_src, a_dst, b, heads, 0.2, True, store=dt)
    sw = (d_in + dh + 8) * 2.0 ** -24 / tol(dt)     # rounding of the softmax weights' exponent
    Yd = ogat.gat_forward_den(A_s, f, b, heads, H_s, W64, a_src, a_dst, sw)
    e_out = np.max(np.abs(f64(Out)[rows - w.lo] - f["Out"]) / (Yd + 1e-30))
    say(f"  forward err {e_out:.1e}")
    assert e_out <= tol(dt), f"forward err {e_out:.2e}"

    rows_b = full.sample(120, seed=41, n_extreme=2)
    A_b, ext_b = full.mini(rows_b)
    H_b = h_of(ext_b)
    fb = ogat.gat_forward(A_b, H_b, W64, a_src, a_dst, b, heads, 0.2, True, store=dt)
    Gb = _bits_or_f32(g.standard_normal((len(rows_b), F), dtype=np.float32), dt)
    Ymask = round_to(fb["Y"], dt)
    G_full = np.zeros((n_l, F), np.uint16 if dt == "bf16" else np.float32)
    Y_full = np.zeros_like(G_full)
    G_full[rows_b - w.lo] = Gb
    Y_full[rows_b - w.lo] = Ymask
    dW, da_src, da_dst, db, dH = sag.gat_layer_backward(ctx, full.gb.A, full.gb.AT, to_dev_dense(Y_full, dt),
                                                        to_dev_dense(G_full, dt))
    Ym64, G64 = olay.as_f64(Ymask, dt), olay.as_f64(Gb, dt)
    r = ogat.gat_backward(A_b, H_b, W64, a_src, a_dst, heads, 0.2, True, fb, Ym64, G64, store=dt)
    d = ogat.gat_backward_den(A_b, H_b, W64, a_src, a_dst, heads, 0.2, True, fb, Ym64, G64, sw)
    errs = {k: float(np.max(np.abs(f64(v) - r[k]) / (d[k] + 1e-30)))
            for k, v in (("dW", dW), ("da_src", da_src), ("da_dst", da_dst), ("db", db))}
    # dH_ext by global id (a sampled row is also a column of the small CSR)
    uniq, inv = np.unique(ext_b, return_inverse=True)
    ref = np.zeros((uniq.size, d_in))
    den = np.zeros((uniq.size, d_in))
    np.add.at(ref, inv, r["dH_ext"])
    np.add.at(den, inv, d["dH_ext"])
    got = f64(dH)
    gi = full.gpu_row(uniq)
    errs["dH_ext"] = float(np.max(np.abs(got[gi] - ref) / (den + 1e-30)))
    say("  backward errors: " + " ".join(f"{k} {e:.1e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e <= tol(dt), f"{k} err {e:.2e}"
    others = np.ones(got.shape[0], bool)
    others[gi] = False
    assert np.all(got[others] == 0.0), "rows outside the sampled neighbourhoods must be zero"


def check_fused(full):
    """The fused aggregate -> transform kernel over the whole partition at the
    workload's widest aggregate-first layer; Out and the stored Z on ~300
    sampled rows against the oracle's layer on the small CSR of those rows."""
    w = full.w
    shapes = [(l, d_in, d_out, relu) for l, d_in, d_out, relu in _layer_shapes(w) if d_in <= d_out]
    _, d_in, d_out, relu = max(shapes, key=lambda t: t[1])
    self_rows = w.model == "sage"
    dt = w.dtype
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    g = np.random.default_rng(2000 + w.cfg)
    n_l, n_h = full.n_l, full.halo.size
    say(f"full-size fused aggregate -> transform, workload {w.cfg}: {d_in} -> {d_out} {dt}")
    feats = _bits_or_f32(g.standard_normal((n_l, d_in), dtype=np.float32), dt)
    stale = _bits_or_f32(g.standard_normal((max(w.stale_rows, 1), d_in), dtype=np.float32), dt) \
        if n_h else None
    w_rows = 2 * d_in if self_rows else d_in
    lim = np.sqrt(6.0 / (w_rows + d_out))
    W = _bits_or_f32(g.uniform(-lim, lim, (w_rows, d_out)), dt)
    b = g.uniform(-0.1, 0.1, d_out).astype(np.float32)
    H_ext = sag.empty_dense(n_l + n_h, d_in, tdt, DEV)
    H_ext[:n_l].copy_(to_dev_dense(feats, dt))
    if n_h:
        sag.halo_gather(to_dev_dense(stale, dt), full.gb.halo_gid, H_ext[n_l:], row_base=w.stale_base)
    Out, _, Z = sag.aggregate_transform(full.gb.A, H_ext, to_dev_dense(W, dt).contiguous(), to_dev(b),
                                        self_rows=self_rows, relu=relu)

    def h_of(gid):
        gid = np.asarray(gid, np.int64)
        local = (gid >= w.lo) & (gid < w.hi)
        out = np.empty((gid.size, d_in), np.float64)
        out[local] = olay.as_f64(feats[gid[local] - w.lo], dt)
        if (~local).any():
            out[~local] = olay.as_f64(stale[gid[~local] - w.stale_base], dt)
        return out

    W64 = olay.as_f64(W, dt)
    rows = full.sample(300, seed=51)
    A_s, ext = full.mini(rows)
    H_s = h_of(ext)
    if self_rows:
        Zr, _, Or = olay.sage_forward(A_s, H_s, len(rows), W64, b, relu)
        Zd, Yd = olay.sage_forward_den(A_s, H_s, len(rows), W64, b)
    else:
        Zr, _, Or = olay.gcn_forward(A_s, H_s, W64, b, relu)
        Zd, Yd = olay.gcn_forward_den(A_s, H_s, W64, b)
    li = rows - w.lo
    e_out = np.max(np.abs(f64(Out)[li] - Or) / (Yd + 1e-30))
    e_z = np.max(np.abs(f64(Z)[li] - Zr) / (Zd + 1e-30))
    say(f"  errors: out {e_out:.1e} Z {e_z:.1e}")
    assert e_out <= tol(dt) and e_z <= tol(dt), f"fused err out {e_out:.2e} Z {e_z:.2e}"


def check_full_output(full, d=256):
    """The whole build against the oracle's, bit for bit, then the d = 256
    products of the forward (A, mean-normalised: the pattern-only path) and
    of the backward (A^T, with values) compared in full, every element,
    against the oracle's fp64 SpMM (bf16 inputs and outputs, fp32
    accumulation: within 2e-2 of the same product on absolute values), each
    both in whole rows and in 128-byte column slices."""
    w = full.w
    gb = full.gb
    say(f"full-size whole build and full-output products, workload {w.cfg}: oracle build of {gb.A.nnz} entries")
    ob = ocsr.build(full.src, full.dst, w.n_global, w.lo, w.hi, w.symmetrize, w.self_loops, w.norm)
    for name, G, O in (("A", gb.A, ob.A), ("AT", gb.AT, ob.AT)):
        assert np.array_equal(G.indptr.cpu().numpy(), O.indptr), f"{name} indptr"
        assert np.array_equal(G.indices.cpu().numpy(), O.indices), f"{name} indices"
        assert np.array_equal(G.values.cpu().numpy().view(np.uint32), O.values.view(np.uint32)), f"{name} values"
    assert np.array_equal(gb.deg.cpu().numpy(), ob.deg_col)
    g = np.random.default_rng(4242)
    X = gen.f32_to_bf16_bits(g.standard_normal((ob.A.n_cols, d), dtype=np.float32))
    Xd = to_dev_dense(X, "bf16")
    X64 = olay.as_f64(X, "bf16")
    for name, Gm, Om, fn in (("A X", gb.A, ob.A, sag.spmm_csr), ("A^T X", gb.AT, ob.AT, sag.spmm_csr_t)):
        say(f"  {name}: GPU products, then the oracle's fp64 product and bound ({native.num_threads()} threads)")
        kept = Gm.col_slices
        Ys = {}
        for sliced in (False, True):
            sag.csr_set_col_slices(Gm, sliced)
            Ys[sliced] = f64(fn(Gm, Xd))
        sag.csr_set_col_slices(Gm, kept)
        ref = native.spmm(Om.indptr, Om.indices, Om.values, X64)
        den = native.spmm(Om.indptr, Om.indices, Om.values, np.abs(X64), abs_mode=True)
        step = 1 << 18
        for sliced, Y in Ys.items():
            err = 0.0
            for r0 in range(0, Y.shape[0], step):
                sl = slice(r0, r0 + step)
                err = max(err, float(np.max(np.abs(Y[sl] - ref[sl]) / (den[sl] + 1e-30))))
            how = "column slices" if sliced else "whole rows"
            say(f"  {name} ({how}): max error {err:.2e} of the bound over {Y.size} elements")
            assert err <= tol("bf16"), f"{name} ({how}) err {err:.2e}"
        del Ys, ref, den
