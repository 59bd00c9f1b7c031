"""DIGEST's pull overlapped with compute (the two-layer GCN on the
100M-graph share that bench.py times, at reduced size): running the pulls
and the push on a second stream, ordered by events, gives the same bits as
running every step on one stream -- the gradients, the layer-1 store after
the push of the fresh local rows, and the store of returned halo gradients
(accumulating push) -- over two consecutive steps."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from gpu_util import say  # noqa: E402


def _state(net):
    return [t.clone() for t in (net.stores[0], net.stores[1], net.grad_store, net.H[0])]


def _restore(net, st):
    for dst, src in zip((net.stores[0], net.stores[1], net.grad_store, net.H[0]), st):
        dst.copy_(src)
    torch.cuda.synchronize()


def _bits(t):
    t = t.detach().contiguous()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).cpu().numpy()


@pytest.mark.parametrize("scale", [0.002, 0.01])
def test_overlapped_pull_matches_one_stream(scale):
    import bench
    say(f"overlapped pull, 2-layer share at scale {scale}")
    net = bench.TwoLayerShare(sag, torch, np, scale)
    assert net.n_h > 0
    st = _state(net)
    results = {}
    for overlap in (False, True):
        _restore(net, st)
        for _ in range(2):
            net.step(overlap)
        torch.cuda.synchronize()
        results[overlap] = [_bits(x) for x in (*net.grads, net.stores[1], net.grad_store, net.Out)]
    for a, b in zip(results[False], results[True]):
        assert np.array_equal(a, b)
    # the push wrote the fresh local rows into the layer-1 store, the pull read
    # the same store's halo rows, and halo gradients were returned
    assert np.array_equal(_bits(net.stores[1][: net.n_l]), _bits(net.H[1][: net.n_l]))
    assert np.any(_bits(net.grad_store[net.n_l:]) != 0)
