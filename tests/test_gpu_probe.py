"""The row-gather probe reads exactly the rows it is given: the sum of its
sink's words equals, word by word and modulo 2^32, the sum of the same words
of every 16-byte vector of the named rows (computed on the host from the
buffer's bits, padding included).  Cases cover every lane layout (one vector
per row up to four per lane), an empty id list, fewer ids than wavefronts,
and the large sparse graph's own column ids at reduced size."""
import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from gpu_util import DEV, say, to_dev  # noqa: E402


def _buffer(g, n_rows, d, dtype):
    es = torch.empty(0, dtype=dtype).element_size()
    ld = sag.padded_ld(d, dtype)
    words = g.integers(0, 2 ** 32, size=(n_rows, ld * es // 4), dtype=np.uint64).astype(np.uint32)
    X = torch.from_numpy(words.view(np.int32)).to(DEV).view(dtype)
    assert X.shape == (n_rows, ld)
    return X[:, :d], words, -(-d * es // 16)


def _check(X, words, C, ids):
    sink = sag.gather_probe(X, to_dev(ids))
    got = sink.view(torch.int32).cpu().numpy().view(np.uint32).reshape(-1, 4).astype(np.uint64).sum(axis=0)
    want = words[ids][:, :4 * C].reshape(len(ids), C, 4).astype(np.uint64).sum(axis=(0, 1))
    assert want.shape == (4,)
    assert np.array_equal(got % 2 ** 32, want % 2 ** 32)


@pytest.mark.parametrize("dt,d", [(torch.float32, 1), (torch.bfloat16, 8), (torch.float32, 41),
                                  (torch.bfloat16, 100), (torch.bfloat16, 256), (torch.float32, 128),
                                  (torch.bfloat16, 1000), (torch.float32, 700)])
@pytest.mark.parametrize("n", [0, 5, 20_011])
def test_probe_sums_the_named_rows(dt, d, n):
    g = np.random.default_rng(d * 7 + n)
    X, words, C = _buffer(g, 3001, d, dt)
    ids = g.integers(0, 3001, n).astype(np.int32)
    say(f"gather probe dt={dt} d={d} n={n}")
    _check(X, words, C, ids)


def test_probe_over_the_graph_column_ids():
    w = gen.make_config(4, 0.01)
    src, dst = w.edges
    b = sag.csr_build_normalize(to_dev(src), to_dev(dst), w.n_global, w.lo, w.hi, w.symmetrize, w.self_loops,
                                "mean")
    ids = b.A.indices.cpu().numpy()
    g = np.random.default_rng(4)
    X, words, C = _buffer(g, b.A.n_cols, 256, torch.bfloat16)
    say(f"gather probe over {ids.size} column ids")
    _check(X, words, C, ids)
