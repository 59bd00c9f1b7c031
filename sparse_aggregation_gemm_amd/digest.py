"""DIGEST's stale-representation exchange around a multi-layer GCN or
GraphSAGE-mean model on one partition, on one GPU.

The DIGEST page's system design keeps, for every layer, a representation
store of all nodes; a partition "pulls" the rows of its out-of-subgraph
neighbours (its halo) from the store before that layer and "pushes" its own
freshly computed rows back for the next epoch, and its I/O section overlaps
the pull of layer l with the forward pass of layer l - 1 and the push with
layer l + 1.  Sylvie's "Backward Propagation" returns the halo rows of each
layer's input gradient to their owners, which add them to their own.

``StaleExchange.step`` runs one forward and backward pass of the model with
these exchanges: the pulls of every layer's halo rows, the pushes of the
fresh local rows into the next layer's store, and the accumulating return of
halo gradients into per-layer gradient stores.  With ``overlap`` the pulls
and pushes run on a second stream, ordered against the layers by events
(the pulls of the next step wait for this step's end, the layers wait for
their pull, each push for the layer that produced its rows); without it
every call runs on the current stream.  Both orders give the same bits.

This module only orders calls into the library (halo gather, layer forward
and backward, halo push); every step of the arithmetic runs in its kernels.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import ops


@dataclass
class StepResult:
    out: torch.Tensor          # the last layer's output rows [n_local, d_L]
    dW: list                   # fp32 weight gradients per layer
    db: list                   # fp32 bias gradients per layer
    dH: list                   # each layer's input gradient [n_local + n_halo, d_l] (None for
                               # layer 0 unless want_dH0); halo rows are what was returned


class StaleExchange:
    """One partition's L-layer model with per-layer stale stores.

    built      : ops.Built of the partition (A with its halo list, and AT).
    model      : "gcn" or "sage".
    dims       : [d_0, ..., d_L]; relu: per layer.
    stores     : L device tensors, store l [n_store, dims[l]] holding the
                 representations of layer l's input for node ids
                 store_base .. store_base + n_store - 1 (store 0: the stale
                 input features of the halo nodes).
    grad_stores: gradient stores [n_store, dims[l]] per layer (None where no
                 gradient is returned; entry 0 is used only with want_dH0),
                 added to by the halo rows of each layer's input gradient.
    local_ids  : int32 global ids of the local rows (lo .. hi - 1), where the
                 pushes write.
    """

    def __init__(self, built: ops.Built, model: str, dims, relu, stores, grad_stores, local_ids,
                 store_base: int = 0):
        if model not in ("gcn", "sage"):
            raise ValueError("model must be gcn or sage")
        L = len(dims) - 1
        if len(stores) != L or len(grad_stores) != L or len(relu) != L:
            raise ValueError("one store, gradient store and ReLU flag per layer")
        self.built, self.model, self.dims, self.relu = built, model, list(dims), list(relu)
        self.stores, self.grad_stores = stores, grad_stores
        self.local_ids = local_ids.to(torch.int32).contiguous()
        self.base = store_base
        A = built.A
        self.n_l, self.n_h = A.n_rows, built.n_halo
        dev = A.device
        dt = stores[0].dtype
        # layer inputs [local ; halo]; layer l's output is written into the
        # local rows of layer l + 1's input
        self.H = [ops.empty_dense(self.n_l + self.n_h, dims[l], dt, dev, fill=0.0) for l in range(L)]
        self.out = ops.empty_dense(self.n_l, dims[L], dt, dev)
        self.fwd = ops.gcn_layer_forward if model == "gcn" else ops.sage_layer_forward
        self.bwd = ops.gcn_layer_backward if model == "gcn" else ops.sage_layer_backward
        self.side = torch.cuda.Stream(device=dev)
        self.e_end = torch.cuda.Event()
        self.e_end.record()

    def step(self, H0_local: torch.Tensor, W, b, G_out: torch.Tensor, overlap: bool = True,
             want_dH0: bool = False) -> StepResult:
        """One forward + backward pass.  H0_local: the local input rows
        [n_local, d_0]; W, b: per-layer weights and fp32 biases; G_out: the
        upstream gradient of the last layer's output."""
        L = len(self.dims) - 1
        n_l = self.n_l
        halo = self.built.halo_gid
        main = torch.cuda.current_stream()
        side = self.side if overlap else main
        pulled = [torch.cuda.Event() for _ in range(L)]
        produced = [torch.cuda.Event() for _ in range(L)]
        pushed = [torch.cuda.Event() for _ in range(L)]
        # pulls of every layer's halo rows (they read only the stale stores)
        with torch.cuda.stream(side):
            side.wait_event(self.e_end)
            for l in range(L):
                if self.n_h:
                    ops.halo_gather(self.stores[l], halo, self.H[l][n_l:], row_base=self.base)
                pulled[l].record(side)
        self.H[0][:n_l].copy_(H0_local)
        ctxs = []
        for l in range(L):
            main.wait_event(pulled[l])
            Out = self.H[l + 1][:n_l] if l + 1 < L else self.out
            _, _, ctx = self.fwd(self.built.A, self.H[l], W[l], b[l], relu=self.relu[l], Out=Out)
            ctxs.append(ctx)
            produced[l].record(main)
            if l + 1 < L:
                # the fresh local rows go to the next layer's store (next epoch)
                with torch.cuda.stream(side):
                    side.wait_event(produced[l])
                    ops.halo_push(Out, self.local_ids, self.stores[l + 1], row_base=self.base)
                    pushed[l].record(side)
        dW, db, dHs = [None] * L, [None] * L, [None] * L
        g = G_out
        for l in reversed(range(L)):
            Y = self.H[l + 1][:n_l] if l + 1 < L else self.out
            want = l > 0 or want_dH0
            dW[l], db[l], dH = self.bwd(ctxs[l], self.built.AT, n_l, Y, g, want_dH=want)
            if want:
                if self.n_h and self.grad_stores[l] is not None:
                    ops.halo_push(dH[n_l:], halo, self.grad_stores[l], row_base=self.base, accumulate=True)
                g = dH[:n_l]
                dHs[l] = dH
        for l in range(L - 1):
            main.wait_event(pushed[l])
        self.e_end.record(main)
        return StepResult(self.out, dW, db, dHs)
