"""Layer steps captured into a HIP graph and replayed.

A forward + backward pass through the library (halo pull, layer forwards
and backwards; every output and workspace given or allocated by the
binding) is run eagerly, then captured once with torch.cuda.graph and
replayed three times, with eager steps, unrelated torch work and
synchronisations between the replays.  Every replay's outputs (layer
outputs, weight and bias gradients, input gradients) must equal the eager
pass bit for bit: the kernels are deterministic, and a graph that recorded
something it should not (a memset node, a stale pointer) shows up here."""
import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from gpu_util import DEV, say, to_dev, to_dev_dense  # noqa: E402


class Pass:
    """One forward + backward pass of an L-layer model on one partition:
    every layer's input holds the local rows and then the halo rows, pulled
    from a per-layer store (constant here, so that every pass computes the
    same values); layer l writes its output into the local rows of layer
    l + 1's input."""

    def __init__(self, w, dt, dims, relu, seed, hub_cols=None, col_slices=False):
        src, dst = w.edges
        norm = "gcn" if w.model == "gcn" else "mean"
        self.b = sag.csr_build_normalize(to_dev(src), to_dev(dst), w.n_global, w.lo, w.hi, w.symmetrize,
                                         w.self_loops, norm)
        sag.csr_schedule(self.b.A, 256)
        sag.csr_schedule(self.b.AT, 256)
        if hub_cols:
            sag.csr_hub_split(self.b.A, hub_cols, 256)
            sag.csr_hub_split(self.b.AT, hub_cols, 256)
        if col_slices:
            sag.csr_set_col_slices(self.b.A, True)
            sag.csr_set_col_slices(self.b.AT, True)
        A = self.b.A
        self.n_l, self.n_ext = A.n_rows, A.n_cols
        self.n_h = self.n_ext - self.n_l
        g = np.random.default_rng(seed)
        stored = (lambda x: gen.f32_to_bf16_bits(np.asarray(x, np.float32))) if dt == "bf16" else \
            (lambda x: np.asarray(x, np.float32))
        L = len(dims) - 1
        self.stores = [to_dev_dense(stored(g.standard_normal((w.n_global, dims[l]))), dt) for l in range(L)]
        tdt = self.stores[0].dtype
        self.H = [sag.empty_dense(self.n_ext, dims[l], tdt, DEV, fill=0.0) for l in range(L)]
        self.H[0][: self.n_l].copy_(to_dev_dense(stored(g.standard_normal((self.n_l, dims[0]))), dt))
        self.W, self.bias = [], []
        for l in range(L):
            k = (2 if w.model == "sage" else 1) * dims[l]
            lim = np.sqrt(6.0 / (k + dims[l + 1]))
            self.W.append(to_dev_dense(stored(g.uniform(-lim, lim, (k, dims[l + 1]))), dt).contiguous())
            self.bias.append(to_dev(g.uniform(-0.1, 0.1, dims[l + 1]).astype(np.float32)))
        self.G = to_dev_dense(stored(g.standard_normal((self.n_l, dims[-1]))), dt)
        self.last = sag.empty_dense(self.n_l, dims[-1], tdt, DEV)
        self.dH = [sag.empty_dense(self.n_ext, dims[l], tdt, DEV) for l in range(L)]
        self.model, self.relu, self.dims = w.model, relu, dims

    def run(self):
        """The pass; returns every output tensor it produced."""
        fwd = sag.gcn_layer_forward if self.model == "gcn" else sag.sage_layer_forward
        bwd = sag.gcn_layer_backward if self.model == "gcn" else sag.sage_layer_backward
        L = len(self.dims) - 1
        if self.n_h:
            for l in range(L):
                sag.halo_gather(self.stores[l], self.b.halo_gid, self.H[l][self.n_l:])
        outs, ctxs, ys = [], [], []
        for l in range(L):
            Out = self.H[l + 1][: self.n_l] if l + 1 < L else self.last
            _, _, ctx = fwd(self.b.A, self.H[l], self.W[l], self.bias[l], relu=self.relu[l], Out=Out)
            ctxs.append(ctx)
            ys.append(Out)
            outs.append(Out)
        g = self.G
        for l in reversed(range(L)):
            dW, db, dH = bwd(ctxs[l], self.b.AT, self.n_l, ys[l], g, want_dH=True, dH=self.dH[l])
            outs += [dW, db, dH]
            g = dH[: self.n_l]
        return outs


def _bits(t):
    t = t.detach().contiguous()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def check_graph(p: Pass):
    ref = [_bits(t) for t in p.run()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        p.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = p.run()
    torch.cuda.synchronize()
    junk = torch.empty(1 << 22, dtype=torch.float32, device=DEV)
    for rep in range(3):
        # eager work between the replays: an eager pass (same buffers) and
        # unrelated kernels over other memory
        p.run()
        junk.normal_()
        _ = float(junk.sum())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [_bits(t) for t in captured]
        assert len(got) == len(ref)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert np.array_equal(a, b), f"replay {rep}: output {i} differs from the eager pass"
    say(f"graph: {len(ref)} outputs equal over 3 replays")


def test_sage_three_layers_bf16():
    """The large sparse graph's 3-layer GraphSAGE at reduced size (the
    headline step's kernels: ring and register NN products, TN, SpMMs)."""
    w = gen.make_config(4, 0.01)
    say("graph capture: sage 3 layers bf16")
    check_graph(Pass(w, "bf16", [100, 256, 256, 47], [True, True, False], seed=3))


def test_gcn_share_with_halo_pull_bf16():
    """The 100M-graph share's GCN at reduced size, with the halo pull in the
    graph."""
    w = gen.make_config(5, 0.002)
    say("graph capture: gcn share with halo bf16")
    check_graph(Pass(w, "bf16", [128, 128, 64], [True, False], seed=4))


def test_tiny_gcn_f32():
    w = gen.make_config(1, 1.0)
    say("graph capture: tiny gcn f32")
    check_graph(Pass(w, "f32", [64, 16], [True], seed=5))


def test_dense_gcn_over_hub_split_f32():
    """The dense power-law graph's GCN with both matrices split: every
    product takes two passes through the partial rows in the workspace."""
    w = gen.make_config(2, 0.004)
    say("graph capture: dense gcn over a hub split f32")
    check_graph(Pass(w, "f32", [64, 32, 16], [True, False], seed=6, hub_cols=100))


def test_sage_over_column_slices_bf16():
    """The large power-law graph's SAGE (reduced) with both matrices in
    column slices: every 256-wide product is four launches in the graph."""
    w = gen.make_config(4, 0.002)
    say("graph capture: sage over column slices bf16")
    check_graph(Pass(w, "bf16", [100, 256, 256, 47], [True, True, False], seed=7, col_slices=True))
