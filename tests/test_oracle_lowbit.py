"""Pins of the oracle's low-bit halo messages and store updates against facts
outside the oracle: the counter-based generator's published known answers,
the unbiasedness the Sylvie page states for its Low-bit Module, exact cases
that need no rounding, the quantization error bound, and round trips."""
import numpy as np
import pytest

from oracle import lowbit as olb


def test_philox_known_answers():
    """Philox4x32-10 known-answer vectors published with the generator
    (Salmon, Moraes, Dror and Shaw, SC'11; the Random123 distribution's
    known-answer tests)."""
    cases = [
        ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
        ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
        ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
         (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
    ]
    for ctr, key, want in cases:
        got = olb.philox4x32_10(np.array([ctr], np.uint32), key)[0]
        assert [int(x) for x in got] == list(want)


def test_uniforms_are_uniform_and_keyed():
    u = olb.uniforms(np.arange(2000), 3, 64, seed=12345)
    assert u.dtype == np.float32 and u.min() >= 0.0 and u.max() < 1.0
    # mean 1/2, variance 1/12 of U[0,1)
    assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / u.size)
    assert abs(u.var() - 1 / 12) < 0.01
    # a different epoch, node or seed gives a different stream
    assert not np.array_equal(u, olb.uniforms(np.arange(2000), 4, 64, seed=12345))
    assert not np.array_equal(u, olb.uniforms(np.arange(2000), 3, 64, seed=54321))
    assert np.array_equal(u[5:6], olb.uniforms([5], 3, 64, seed=12345))


def test_draws_are_the_fp32_uniform_grid():
    """Each draw is k 2^-24 with k the top 24 bits of the generator word that
    the element's position selects (block j // 4, word j % 4)."""
    nodes = np.array([0, 7, 123456, 2 ** 31 - 1])
    d, epoch, seed = 11, 5, (0xABCDEF << 32) | 0x13579
    u = olb.uniforms(nodes, epoch, d, seed)
    k = u.astype(np.float64) * 2.0 ** 24
    assert np.array_equal(k, np.floor(k)) and k.min() >= 0 and k.max() < 2 ** 24
    for i, node in enumerate(nodes):
        for j in range(d):
            w = olb.philox4x32_10(np.array([[j // 4, node, epoch, 0]], np.uint32),
                                  (seed & 0xFFFFFFFF, seed >> 32))[0, j % 4]
            assert int(k[i, j]) == int(w) >> 8


def _round_up_count(t, B):
    """Over all 2^24 equally likely draws, how many round fp32 t up."""
    grid = np.arange(2 ** 24, dtype=np.float32) * np.float32(2.0 ** -24)
    q = olb.stochastic_round(np.full(grid.size, t, np.float32), grid, B)
    return int(np.sum(q - np.floor(np.float32(t)), dtype=np.int64))


@pytest.mark.parametrize("t", [0.5, 0.75, 1.0, 1.0000001, 2.9999998, 3.3, 127.00781, 200.5, 254.99998])
def test_expected_code_is_exactly_t(t):
    """Sylvie's Low-bit Module is unbiased: with the draw uniform over its
    2^24 values, the code's expectation is exactly the bin position for
    every fp32 t >= 1/2 (its fraction lies on the 2^-24 grid), counted over
    all draws."""
    t = np.float32(t)
    frac = float(t) - np.floor(float(t))
    assert _round_up_count(t, 255) == round(frac * 2 ** 24)


@pytest.mark.parametrize("t", [0.3, 1e-3, 3e-7, 2.0 ** -30])
def test_expected_code_below_one_half(t):
    """Below 1/2 the fraction can be finer than the draw grid: the bias is
    under 2^-24 of a bin."""
    t = np.float32(t)
    count = _round_up_count(t, 1)
    assert abs(count / 2 ** 24 - float(t)) < 2.0 ** -24


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_grid_values_are_exact(bits):
    """Values on the quantization grid (a power-of-two scale) need no
    rounding: codes are the grid indices and the recovery is exact, whatever
    the draw."""
    B = 2 ** bits - 1
    g = np.random.default_rng(bits)
    n, d = 50, 37
    k = g.integers(0, B + 1, (n, d))
    k[:, 0], k[:, 1] = 0, B                       # the row spans the whole grid
    zero = g.integers(-64, 64, n).astype(np.float32) * np.float32(0.25)
    s = np.float32(2.0) ** g.integers(-6, 3, n).astype(np.float32)
    H = (zero[:, None] + k.astype(np.float32) * s[:, None]).astype(np.float32)
    for epoch in range(3):
        q, scale, z = olb.quantize_rows(H, np.arange(n), epoch, 99, bits)
        assert np.array_equal(scale, s) and np.array_equal(z, zero)
        assert np.array_equal(q, k)
        assert np.array_equal(olb.dequantize_rows(q, scale, z), H)


def test_constant_rows_and_one_bit_levels():
    H = np.full((4, 10), 3.5, np.float32)
    q, scale, z = olb.quantize_rows(H, np.arange(4), 0, 1, 1)
    assert np.all(q == 0) and np.all(scale == 0) and np.all(z == 3.5)
    assert np.array_equal(olb.dequantize_rows(q, scale, z), H)
    g = np.random.default_rng(0)
    H = g.standard_normal((100, 33)).astype(np.float32)
    q, scale, z = olb.quantize_rows(H, np.arange(100), 7, 5, 1)
    rec = olb.dequantize_rows(q, scale, z)
    # one bit: every recovered value is the row's minimum or maximum
    lo, hi = H.min(axis=1, keepdims=True), H.max(axis=1, keepdims=True)
    assert np.all((rec == lo) | (np.abs(rec - hi) <= 1e-6 * np.abs(hi) + 1e-6))


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_error_bound(bits):
    """|recovered - h| <= scale (plus fp32 rounding): the code is one of the
    two grid points around t; the bound shrinks as 1 / (2^b - 1)."""
    g = np.random.default_rng(10 + bits)
    H = (g.standard_normal((300, 64)) * g.uniform(0.1, 10, (300, 1))).astype(np.float32)
    q, scale, z = olb.quantize_rows(H, np.arange(300), 1, 2024, bits)
    rec = olb.dequantize_rows(q, scale, z)
    R = H.max(axis=1) - H.min(axis=1)
    err = np.abs(rec.astype(np.float64) - H)
    assert np.all(err <= scale[:, None] * (1 + 1e-5) + 4e-7 * np.abs(H).max(axis=1, keepdims=True))
    assert np.all(scale <= R / (2 ** bits - 1) * (1 + 1e-6))
    assert q.max() <= 2 ** bits - 1


@pytest.mark.parametrize("bits", [1, 2, 4])
def test_unbiased(bits):
    """Sylvie's Low-bit Module is unbiased: over independent draws (epochs)
    the mean recovered vector converges to the original, within the
    binomial standard error s sqrt(f (1 - f) / T) per element."""
    g = np.random.default_rng(bits)
    H = g.standard_normal((3, 40)).astype(np.float32)
    T = 3000
    acc = np.zeros(H.shape)
    for epoch in range(T):
        q, scale, z = olb.quantize_rows(H, np.arange(3), epoch, 777, bits)
        acc += olb.dequantize_rows(q, scale, z)
    mean = acc / T
    q0, scale, z = olb.quantize_rows(H, np.arange(3), 0, 777, bits)
    t = (H - z[:, None]) / scale[:, None]
    f = t - np.floor(t)
    se = scale[:, None] * np.sqrt(f * (1 - f) / T) + 1e-6
    assert np.all(np.abs(mean - H) <= 6 * se + 1e-5)
    # and a deterministic (round-to-nearest) quantizer would fail this test
    near = z[:, None] + np.rint(t) * scale[:, None]
    assert np.any(np.abs(near - H) > 6 * se + 1e-5)


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_pack_layout(bits):
    g = np.random.default_rng(bits)
    d = 29
    q = g.integers(0, 2 ** bits, (20, d)).astype(np.uint8)
    packed = olb.pack_codes(q, bits)
    assert packed.shape == (20, (d * bits + 7) // 8)
    assert np.array_equal(olb.unpack_codes(packed, d, bits), q)
    # element j sits at bit b*j (little-endian): read it back bit by bit
    for j in (0, 1, d - 1):
        val = 0
        for t in range(bits):
            bit = j * bits + t
            val |= ((packed[:, bit // 8] >> (bit % 8)) & 1).astype(np.int64) << t
        assert np.array_equal(val, q[:, j])


def test_push_then_pull_round_trips():
    """DIGEST push then pull: the rows pulled back are the rows pushed."""
    g = np.random.default_rng(3)
    store = g.standard_normal((1000, 16)).astype(np.float32)
    ids = g.choice(np.arange(200, 1200), 300, replace=False)
    src = g.standard_normal((300, 16)).astype(np.float32)
    out = olb.push(store, src, ids, 200)
    assert np.array_equal(out[ids - 200], src)
    untouched = np.setdiff1d(np.arange(1000), ids - 200)
    assert np.array_equal(out[untouched], store[untouched])
    acc = olb.push(store, src, ids, 200, accumulate=True)
    assert np.allclose(acc[ids - 200], store[ids - 200] + src)
