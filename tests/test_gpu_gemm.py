"""GPU MFMA products against float64 matrix products on the same stored
inputs (the oracle's dense step is a library matmul in float64)."""
import numpy as np
import pytest
import torch

import gen
from oracle import layers as olay

pytestmark = pytest.mark.gpu

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from gpu_util import DEV, f64, say, to_dev, to_dev_dense, tol  # noqa: E402


def _mat(g, shape, dt, integers=False):
    x = g.integers(-4, 5, shape).astype(np.float32) if integers else g.standard_normal(shape).astype(np.float32)
    stored = gen.f32_to_bf16_bits(x) if dt == "bf16" else x
    return stored, to_dev_dense(stored, dt)


def _err(got, ref, den):
    return float(np.max(np.abs(got - ref) / (den + 1e-30))) if ref.size else 0.0


# (1031, 128, 111) and (517, 100, 64): bf16 products over a 128-element K
# with at most 128 columns take the weights-in-registers kernel
SHAPES = [(1, 1, 1), (5, 3, 7), (130, 64, 16), (257, 100, 256), (1000, 200, 47), (333, 512, 48),
          (700, 128, 602), (4099, 602, 128), (129, 41, 300), (1031, 128, 111), (517, 100, 64)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_gemm_nn(dt, M, K, N):
    g = np.random.default_rng(M * 7 + K * 3 + N)
    As, A = _mat(g, (M, K), dt)
    Ws, W = _mat(g, (K, N), dt)
    W = W.contiguous()
    b = g.uniform(-0.1, 0.1, N).astype(np.float32)
    say(f"gemm nn dt={dt} M={M} K={K} N={N}")
    C, pre = sag.gemm(A, W, bias=to_dev(b), relu=True, want_pre=True)
    A64, W64 = f64(A), f64(W)
    ref = A64 @ W64 + b
    den = np.abs(A64) @ np.abs(W64) + np.abs(b)
    assert _err(f64(pre), ref, den) <= tol(dt)
    assert _err(f64(C), np.maximum(ref, 0), den) <= tol(dt)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gemm_two_blocks_mask_addend_transposed(dt):
    g = np.random.default_rng(3)
    M, K1, K2, N = 517, 100, 100, 256
    _, A1 = _mat(g, (M, K1), dt)
    _, A2 = _mat(g, (M, K2), dt)
    _, Mk = _mat(g, (M, K1), dt)
    _, Bt = _mat(g, (N, K1 + K2), dt)          # B given transposed
    Bt = Bt.contiguous()
    _, add = _mat(g, (M, N), dt)
    say(f"gemm two blocks dt={dt}")
    C = sag.gemm(A1, Bt, A2=A2, mask=Mk, trans_b=True, addend=add)
    A64 = np.concatenate([f64(A1) * (f64(Mk) > 0), f64(A2)], 1)
    B64 = f64(Bt).T
    ref = A64 @ B64 + f64(add)
    den = np.abs(A64) @ np.abs(B64) + np.abs(f64(add))
    assert _err(f64(C), ref, den) <= tol(dt)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("K1,K2,N,masked", [(256, 256, 256, False), (100, 100, 256, False), (256, 0, 512, True),
                                            (47, 47, 150, False), (200, 0, 300, True)])
def test_gemm_wide_outputs(dt, K1, K2, N, masked):
    """Outputs wider than 128 columns (bf16 takes the kernel that keeps the
    weight fragments in registers): two K blocks, the ReLU mask, ragged M
    and N, pre-activation and output."""
    g = np.random.default_rng(K1 + K2 + N)
    M = 1031
    _, A1 = _mat(g, (M, K1), dt)
    A2 = _mat(g, (M, K2), dt)[1] if K2 else None
    Mk = _mat(g, (M, K1), dt)[1] if masked else None
    _, W = _mat(g, (K1 + K2, N), dt)
    W = W.contiguous()
    b = g.uniform(-0.1, 0.1, N).astype(np.float32)
    say(f"gemm wide dt={dt} K={K1}+{K2} N={N} masked={masked}")
    C, pre = sag.gemm(A1, W, A2=A2, mask=Mk, bias=to_dev(b), relu=True, want_pre=True)
    A64 = f64(A1) * (f64(Mk) > 0) if masked else f64(A1)
    if K2:
        A64 = np.concatenate([A64, f64(A2)], 1)
    W64 = f64(W)
    ref = A64 @ W64 + b
    den = np.abs(A64) @ np.abs(W64) + np.abs(b)
    assert _err(f64(pre), ref, den) <= tol(dt)
    assert _err(f64(C), np.maximum(ref, 0), den) <= tol(dt)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("M", [1, 33, 97])
@pytest.mark.parametrize("K,N", [(128, 256), (256, 256), (512, 256), (256, 512), (96, 100)])
def test_gemm_few_rows(dt, M, K, N):
    """Fewer row tiles than the persistent kernels' workgroups and their
    prefetch depth: the steps past a workgroup's last tile must store
    nothing.  Exact small integers, so any stray or missing store shows."""
    g = np.random.default_rng(M + K + N)
    _, A = _mat(g, (M, K), dt, integers=True)
    _, W = _mat(g, (K, N), dt, integers=True)
    W = W.contiguous()
    say(f"gemm few rows dt={dt} M={M} K={K} N={N}")
    C = sag.gemm(A, W)
    exact = f64(A) @ f64(W)
    ref = olay.round_bf16(exact) if dt == "bf16" else exact
    assert np.array_equal(f64(C), ref)


@pytest.mark.parametrize("M,K1,K2,N", [(2053, 512, 0, 200), (777, 100, 100, 136), (64, 128, 0, 256),
                                        (100_003, 300, 100, 256), (120_001, 256, 256, 248), (50_000, 100, 100, 160)])
def test_gemm_streamed_tiles(M, K1, K2, N):
    """bf16 products with 128 < N <= 256 (N a multiple of 8) and a packed K of
    256 or 512, whose row tiles stream through an LDS ring (and one at a
    packed K of 128, which takes the register-prefetch kernel): column
    blocks past N (wavefronts with no block in either half of the
    workgroup, one block half outside), rows past M, partly covered 16-byte
    units in both K blocks at both packed K, and enough tiles per workgroup
    for the ring to wrap many times.  Exact small integers (every
    sum is exact in fp32), so the result is the exact product rounded once
    to bf16, bit for bit."""
    g = np.random.default_rng(M + K1 + K2 + N)
    _, A1 = _mat(g, (M, K1), "bf16", integers=True)
    A2 = _mat(g, (M, K2), "bf16", integers=True)[1] if K2 else None
    _, W = _mat(g, (K1 + K2, N), "bf16", integers=True)
    W = W.contiguous()
    b = g.integers(-3, 4, N).astype(np.float32)
    say(f"gemm streamed tiles M={M} K={K1}+{K2} N={N}")
    C = sag.gemm(A1, W, A2=A2, bias=to_dev(b), relu=True)
    A64 = f64(A1) if not K2 else np.concatenate([f64(A1), f64(A2)], 1)
    exact = A64 @ f64(W) + b
    assert np.array_equal(f64(C), olay.round_bf16(np.maximum(exact, 0)))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N", [80, 300])
def test_gemm_exact_integers(dt, N):
    g = np.random.default_rng(4)
    _, A = _mat(g, (300, 96), dt, integers=True)
    _, W = _mat(g, (96, N), dt, integers=True)
    W = W.contiguous()
    say(f"gemm exact dt={dt}")
    C = sag.gemm(A, W)
    exact = f64(A) @ f64(W)   # every partial sum is an integer below 2^24
    # one rounding of the exact result to the stored type
    ref = olay.round_bf16(exact) if dt == "bf16" else exact
    assert np.array_equal(f64(C), ref)


TN_SHAPES = [(1, 1, 1), (33, 17, 5), (1000, 100, 256), (5000, 256, 47), (20000, 128, 128),
             (70000, 512, 48), (3, 602, 128)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("M,K,N", TN_SHAPES)
def test_gemm_tn(dt, M, K, N):
    g = np.random.default_rng(M + K + N)
    _, A = _mat(g, (M, K), dt)
    _, B = _mat(g, (M, N), dt)
    _, Mk = _mat(g, (M, N), dt)
    say(f"gemm tn dt={dt} M={M} K={K} N={N}")
    C, cs = sag.gemm_tn(A, B, mask=Mk)
    Bm = f64(B) * (f64(Mk) > 0)
    A64 = f64(A)
    ref = A64.T @ Bm
    den = np.abs(A64).T @ np.abs(Bm)
    assert _err(f64(C), ref, den) <= 1e-5   # inputs are exact values; only fp32 sums round
    assert _err(f64(cs), Bm.sum(0), np.abs(Bm).sum(0)) <= 1e-5


def test_gemm_tn_two_blocks():
    g = np.random.default_rng(8)
    M, K1, K2, N = 3001, 100, 100, 256
    _, A1 = _mat(g, (M, K1), "bf16")
    _, A2 = _mat(g, (M, K2), "bf16")
    _, B = _mat(g, (M, N), "bf16")
    say("gemm tn two blocks")
    C, cs = sag.gemm_tn(A1, B, A2=A2)
    A64 = np.concatenate([f64(A1), f64(A2)], 1)
    ref = A64.T @ f64(B)
    den = np.abs(A64).T @ np.abs(f64(B))
    assert _err(f64(C), ref, den) <= 1e-5


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("masked,N", [(False, 96), (True, 96), (False, 256)])
def test_gemm_tight_row_pitch(dt, masked, N):
    """Operands whose row pitch is the width rounded to 16 bytes only (e.g.
    100 bf16 in rows of 104) and that end exactly at the end of their
    allocation: the padded k-steps must not read past the rows."""
    g = np.random.default_rng(31 + N)
    M, K1, K2 = 333, 100, 42
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    v = 4 if dt == "f32" else 8

    def tight(rows, cols):
        ld = (cols + v - 1) // v * v
        buf = torch.empty(rows * ld, dtype=tdt, device=DEV)
        t = buf.view(rows, ld)[:, :cols]
        t.copy_(torch.from_numpy(g.standard_normal((rows, cols)).astype(np.float32)).to(tdt).to(DEV))
        return t

    A1, A2 = tight(M, K1), tight(M, K2)
    Mk = tight(M, K1) if masked else None
    W = torch.from_numpy(g.standard_normal((K1 + K2, N)).astype(np.float32)).to(tdt).to(DEV)
    say(f"gemm tight pitch dt={dt} masked={masked}")
    C = sag.gemm(A1, W, A2=A2, mask=Mk)
    a1 = f64(A1) * ((f64(Mk) > 0) if masked else 1.0)
    A64 = np.concatenate([a1, f64(A2)], 1)
    ref = A64 @ f64(W)
    den = np.abs(A64) @ np.abs(f64(W))
    assert _err(f64(C), ref, den) <= tol(dt)
