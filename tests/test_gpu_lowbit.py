"""GPU push and low-bit halo messages against the oracle, bit for bit.

Quantization draws come from the same counter-based generator on both
sides, and both take each rounding decision in fp32 in the same order, so
codes, scales, zero-points and recovered rows must match exactly; pushes
are bitwise copies, or fp32 sums rounded once."""
import numpy as np
import pytest
import torch

import gen
from oracle import csr as ocsr, layers as olay, lowbit as olb

pytestmark = pytest.mark.gpu

sag = pytest.importorskip("sparse_aggregation_gemm_amd")
from gpu_util import DEV, f64, say, tol, to_dev, to_dev_dense  # noqa: E402


def _stored(x, dt):
    """(stored array: fp32 values or bf16 bits, the same values as float32)."""
    x = np.asarray(x, np.float32)
    if dt == "bf16":
        bits = gen.f32_to_bf16_bits(x)
        return bits, olay.as_f64(bits, "bf16").astype(np.float32)
    return x, x


def _bits_of(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    return t.detach().contiguous().cpu().numpy().view(np.uint32)


def _expected_bits(vals_f32: np.ndarray, dt: str) -> np.ndarray:
    """Oracle fp32 values in the storage type, as bits (bf16: nearest, ties
    to even, from the fp32 value)."""
    v = np.asarray(vals_f32, np.float32)
    if dt == "bf16":
        r = olay.round_bf16(v.astype(np.float64)).astype(np.float32)
        return (r.view(np.uint32) >> 16).astype(np.uint16)
    return v.view(np.uint32)


def _rows(g, n, d, dt):
    x = (g.standard_normal((n, d)) * g.uniform(0.01, 50, (n, 1)) + g.uniform(-5, 5, (n, 1))).astype(np.float32)
    return _stored(x, dt)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [1, 7, 8, 37, 64, 100, 128, 600])
def test_quantize_matches_oracle(dt, bits, d):
    g = np.random.default_rng(1000 * bits + d)
    n_src, n = 700, 500
    stored, vals = _rows(g, n_src, d, dt)
    rows = g.choice(n_src, n, replace=False).astype(np.int32)
    nodes = g.integers(0, 2 ** 31 - 1, n).astype(np.int32)
    seed, epoch = int(g.integers(0, 2 ** 63)), int(g.integers(0, 2 ** 32))
    say(f"quantize dt={dt} bits={bits} d={d}")
    src = to_dev_dense(stored, dt)
    codes, scale, zero = sag.quantize_rows(src, bits, seed, epoch, rows=to_dev(rows), nodes=to_dev(nodes))
    q, s_ref, z_ref = olb.quantize_rows(vals[rows], nodes, epoch, seed, bits)
    nb = olb.code_bytes(d, bits)
    got = codes.cpu().numpy()
    assert np.array_equal(got[:, :nb], olb.pack_codes(q, bits))
    assert np.all(got[:, nb:((d + 7) // 8) * bits] == 0)
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(zero.cpu().numpy().view(np.uint32), z_ref.view(np.uint32))
    # recovery into a fresh buffer (dst[k]) and into scattered rows
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    out = sag.empty_dense(n, d, tdt, DEV, fill=0)
    sag.dequantize_rows(codes, scale, zero, d, bits, out)
    ref = olb.dequantize_rows(q, s_ref, z_ref)
    assert np.array_equal(_bits_of(out), _expected_bits(ref, dt))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_quantize_special_rows(dt):
    """Constant rows, single elements, rows on the grid (exact), stream ids
    defaulting to the message row, identity row mapping, and an index
    outside the source (an all-zero message)."""
    g = np.random.default_rng(5)
    d, bits = 40, 4
    x = g.standard_normal((6, d)).astype(np.float32)
    x[0] = 2.5                                   # constant
    x[1] = 0.0
    x[1, 17] = 3.0                               # one non-zero element
    x[2] = (np.arange(d) % 16).astype(np.float32) * 0.125 - 1.0   # grid, scale 1/8
    stored, vals = _stored(x, dt)
    src = to_dev_dense(stored, dt)
    codes, scale, zero = sag.quantize_rows(src, bits, 77, 3)
    q, s_ref, z_ref = olb.quantize_rows(vals, np.arange(6), 3, 77, bits)
    assert np.array_equal(codes.cpu().numpy()[:, :olb.code_bytes(d, bits)], olb.pack_codes(q, bits))
    assert np.array_equal(scale.cpu().numpy(), s_ref) and np.array_equal(zero.cpu().numpy(), z_ref)
    assert np.all(q[0] == 0) and s_ref[0] == 0 and z_ref[0] == 2.5
    assert np.array_equal(q[2], (np.arange(d) % 16))
    rows = to_dev(np.array([3, -1, 6, 0], np.int32))
    c2, s2, z2 = sag.quantize_rows(src, bits, 77, 3, rows=rows)
    written = ((d + 7) // 8) * bits          # bytes a row's codes occupy; the rest is not touched
    assert np.all(c2.cpu().numpy()[1:3, :written] == 0) and np.all(s2.cpu().numpy()[1:3] == 0)
    assert np.all(z2.cpu().numpy()[1:3] == 0)
    q3, _, _ = olb.quantize_rows(vals[[3]], [0], 3, 77, bits)
    assert np.array_equal(c2.cpu().numpy()[0, :olb.code_bytes(d, bits)], olb.pack_codes(q3, bits)[0])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [1, 8])
def test_dequantize_scatter_and_accumulate(dt, bits):
    """The pull into listed rows and the accumulating gradient return."""
    g = np.random.default_rng(bits)
    n, d, n_dst, base = 300, 96, 1000, 50
    stored, vals = _rows(g, n, d, dt)
    src = to_dev_dense(stored, dt)
    codes, scale, zero = sag.quantize_rows(src, bits, 11, 2)
    q, s_ref, z_ref = olb.quantize_rows(vals, np.arange(n), 2, 11, bits)
    rec = olb.dequantize_rows(q, s_ref, z_ref)
    ids = (g.choice(n_dst, n, replace=False) + base).astype(np.int32)
    ids[:3] = [base - 1, base + n_dst, base + n_dst + 7]      # outside: skipped
    dst_stored, dst_vals = _rows(g, n_dst, d, dt)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    for acc in (False, True):
        say(f"dequantize dt={dt} bits={bits} accumulate={acc}")
        dst = to_dev_dense(dst_stored, dt)
        sag.dequantize_rows(codes, scale, zero, d, bits, dst, ids=to_dev(ids), row_base=base, accumulate=acc)
        want = _expected_bits(dst_vals, dt).copy()
        t = ids[3:] - base
        new = (dst_vals[t] + rec[3:]).astype(np.float32) if acc else rec[3:]
        want[t] = _expected_bits(new, dt)
        assert np.array_equal(_bits_of(dst), want)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("d", [5, 64, 100, 600])
def test_push_then_pull_and_accumulate(dt, d):
    """DIGEST push then pull round-trips bitwise; the accumulating push adds
    in fp32 with one rounding; targets outside the store are skipped."""
    g = np.random.default_rng(d)
    n_store, n, base = 2000, 400, 100
    store_stored, store_vals = _rows(g, n_store, d, dt)
    src_stored, src_vals = _rows(g, n, d, dt)
    ids = (g.choice(n_store, n, replace=False) + base).astype(np.int32)
    ids[0] = base + n_store                       # outside: skipped
    say(f"push dt={dt} d={d}")
    store = to_dev_dense(store_stored, dt)
    src = to_dev_dense(src_stored, dt)
    sag.halo_push(src, to_dev(ids), store, row_base=base)
    want = _expected_bits(store_vals, dt).copy()
    want[ids[1:] - base] = _expected_bits(src_vals[1:], dt)
    assert np.array_equal(_bits_of(store), want)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    back = sag.empty_dense(n - 1, d, tdt, DEV)
    sag.halo_gather(store, to_dev(ids[1:]), back, row_base=base)
    assert np.array_equal(_bits_of(back), _bits_of(src[1:]))
    store = to_dev_dense(store_stored, dt)
    sag.halo_push(src, to_dev(ids), store, row_base=base, accumulate=True)
    want = _expected_bits(store_vals, dt).copy()
    t = ids[1:] - base
    want[t] = _expected_bits((store_vals[t] + src_vals[1:]).astype(np.float32), dt)
    assert np.array_equal(_bits_of(store), want)


@pytest.mark.parametrize("bits", [1, 8])
def test_layer_on_low_bit_halo(bits):
    """Sylvie's forward on one partition: the halo rows arrive as b-bit
    messages quantized from the stale buffer and are recovered into H_ext
    on the GPU; the layer then matches the oracle layer run on the oracle's
    recovered rows (same codes, bit for bit)."""
    w = gen.make_config(3, 1 / 64)
    src_e, dst_e = w.edges
    n_l = w.hi - w.lo
    ob = ocsr.build(src_e, dst_e, w.n_global, w.lo, w.hi, True, False, "mean")
    g = np.random.default_rng(bits)
    d_in, d_out = 128, 256
    H_loc = g.standard_normal((n_l, d_in)).astype(np.float32)
    stale = g.standard_normal((w.stale_rows, d_in)).astype(np.float32)
    say(f"low-bit halo layer bits={bits} n_halo={ob.n_halo}")
    gb = sag.csr_build_normalize(to_dev(src_e), to_dev(dst_e), w.n_global, w.lo, w.hi, True, False, "mean")
    sag.csr_schedule(gb.A, 256)
    sag.csr_schedule(gb.AT, 256)
    stale_d = to_dev_dense(stale)
    rows = gb.halo_gid.to(torch.int64) - w.stale_base
    codes, scale, zero = sag.quantize_rows(stale_d, bits, 123, 9, rows=rows.to(torch.int32), nodes=gb.halo_gid)
    H_ext = sag.empty_dense(n_l + gb.n_halo, d_in, torch.float32, DEV)
    H_ext[:n_l].copy_(to_dev_dense(H_loc))
    sag.dequantize_rows(codes, scale, zero, d_in, bits, H_ext[n_l:])
    W = g.uniform(-0.1, 0.1, (2 * d_in, d_out)).astype(np.float32)
    b = g.uniform(-0.1, 0.1, d_out).astype(np.float32)
    Out, _, _ = sag.sage_layer_forward(gb.A, H_ext, to_dev(W), to_dev(b), relu=True)
    q, s_ref, z_ref = olb.quantize_rows(stale[ob.halo_gid - w.stale_base], ob.halo_gid, 9, 123, bits)
    halo = olb.dequantize_rows(q, s_ref, z_ref)
    assert np.array_equal(f64(H_ext[n_l:]), halo.astype(np.float64))
    H64 = np.concatenate([H_loc, halo]).astype(np.float64)
    _, _, ref = olay.sage_forward(ob.A, H64, n_l, W.astype(np.float64), b, True)
    _, den = olay.sage_forward_den(ob.A, H64, n_l, W.astype(np.float64), b)
    assert np.max(np.abs(f64(Out) - ref) / (den + 1e-30)) <= tol("f32")
