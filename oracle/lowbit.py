"""Oracle low-bit halo messages and representation store updates (test
infrastructure only).

Definitions followed
--------------------
* Quantizer (Sylvie, "Quantizer" paragraph of the system overview): each
  node feature vector h that leaves its partition is quantized to b-bit
  integers with B = 2^b - 1 bins by stochastic rounding (the rounding of
  Courbariaux et al. 2015 that the page names); with it go a scale, the ratio
  of max(h) - min(h) to B, and a zero-point, min(h) ("Communicator").
* Dequantizer (Sylvie, "Dequantizer"): the receiving partition recovers full
  precision values from the integers, the scale and the zero-point.
* Unbiasedness (Sylvie, convergence section, "Unbiased Low-bit Module"): the
  expected recovered vector equals the original one.
* Push and pull (DIGEST, system design: the "push" stores a partition's
  newly computed rows of its own nodes in the representation store, the
  "pull" fetches the out-of-subgraph rows it needs); the backward pass sends
  the halo rows of the input gradient to their owners, which add them to the
  gradient of their own rows (Sylvie, "Backward Propagation").

Readings (the quantization and dequantization equations are missing from
the extracted page)
-----------------------------------------------------------------------------
* With Z = min_j h_j, R = max_j h_j - Z and the scale s = R / B (fp32,
  correctly rounded), element j's bin position is t_j = (h_j - Z) / s (fp32,
  correctly rounded): the distance from the zero-point measured in scales,
  the plain inverse of the recovery Z + q s.  Its code is floor(t_j) plus one
  with probability t_j - floor(t_j) (stochastic rounding), at most B.  A row
  with R = 0 has all codes 0.  The recovered element is Z + q_j s.  Every
  step is an fp32 operation rounded to nearest even, in that order (no fused
  multiply-add), so that the integer decisions are reproducible.
* The uniform draw of element j of the node with id `node`, call `epoch`,
  generator key `seed`: the Philox4x32-10 counter-based generator (Salmon,
  Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
  SC'11) at counter (j // 4, node, epoch, 0) and key (seed low 32 bits, seed
  high 32 bits); output word j % 4, its top 24 bits times 2^-24: the fp32
  uniform on [0, 1), whose 2^24 equally likely values k 2^-24 are all exact
  in fp32.  u < frac rounds up.  Every fp32 t >= 1/2 has a fraction on that
  2^-24 grid, so there the probability of rounding up is exactly the
  fraction and the code's expectation is exactly t (the page's unbiased
  Low-bit Module); below 1/2 the bias is under 2^-24 of a bin.
* Codes are packed little-endian: element j occupies bits [b j, b j + b) of
  the row's code bytes.
"""
from __future__ import annotations

import numpy as np

PHILOX_M = (0xD2511F53, 0xCD9E8D57)
PHILOX_W = (0x9E3779B9, 0xBB67AE85)
BITS = (1, 2, 4, 8)


def philox4x32_10(ctr: np.ndarray, key) -> np.ndarray:
    """Philox4x32 with 10 rounds (Salmon et al., SC'11): counter uint32
    [..., 4], key (k0, k1) -> uint32 [..., 4]."""
    c = np.asarray(ctr, np.uint64) & 0xFFFFFFFF
    c0, c1, c2, c3 = (c[..., i].copy() for i in range(4))
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    m0, m1 = np.uint64(PHILOX_M[0]), np.uint64(PHILOX_M[1])
    mask = np.uint64(0xFFFFFFFF)
    for _ in range(10):
        p0 = m0 * c0            # < 2^64: exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & mask
        hi1, lo1 = p1 >> np.uint64(32), p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + np.uint64(PHILOX_W[0])) & mask
        k1 = (k1 + np.uint64(PHILOX_W[1])) & mask
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def uniforms(nodes, epoch: int, d: int, seed: int) -> np.ndarray:
    """float32 [n, d]: the draw of every element of every listed node."""
    nodes = np.asarray(nodes, np.int64)
    n = nodes.size
    nblk = (d + 3) // 4
    ctr = np.zeros((n, nblk, 4), np.uint64)
    ctr[..., 0] = np.arange(nblk, dtype=np.uint64)[None, :]
    ctr[..., 1] = (nodes.astype(np.uint64) & np.uint64(0xFFFFFFFF))[:, None]
    ctr[..., 2] = np.uint64(epoch & 0xFFFFFFFF)
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)).reshape(n, nblk * 4)[:, :d]
    return ((words >> np.uint32(8)).astype(np.float32) * np.float32(2.0 ** -24)).astype(np.float32)


def stochastic_round(t, u, B):
    """The code of bin position t (fp32) with draw u in [0, 1): floor(t),
    plus one when u < t - floor(t) (the fraction, exact in fp32), at most B."""
    t = np.asarray(t, np.float32)
    fl = np.floor(t).astype(np.float32)
    q = fl + (np.asarray(u, np.float32) < (t - fl).astype(np.float32)).astype(np.float32)
    return np.minimum(q, np.float32(B))


def quantize_rows(H, nodes, epoch: int, seed: int, bits: int):
    """Stochastic b-bit quantization of each row of H (float32 values).

    Returns (codes uint8 [n, d] unpacked, scale float32 [n], zero float32 [n])."""
    if bits not in BITS:
        raise ValueError(f"bits must be one of {BITS}")
    H = np.asarray(H, np.float32)
    n, d = H.shape
    B = np.float32(2 ** bits - 1)
    if n == 0 or d == 0:
        return np.zeros((n, d), np.uint8), np.zeros(n, np.float32), np.zeros(n, np.float32)
    zero = H.min(axis=1)
    rng = (H.max(axis=1) - zero).astype(np.float32)
    scale = (rng / B).astype(np.float32)
    u = uniforms(nodes, epoch, d, seed)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = ((H - zero[:, None]).astype(np.float32) / scale[:, None]).astype(np.float32)
    q = stochastic_round(t, u, B)
    q = np.where(rng[:, None] > 0, q, np.float32(0))
    return q.astype(np.uint8), scale, zero


def dequantize_rows(codes, scale, zero) -> np.ndarray:
    """float32 [n, d]: zero + code * scale, each operation rounded in fp32."""
    q = np.asarray(codes).astype(np.float32)
    prod = (q * np.asarray(scale, np.float32)[:, None]).astype(np.float32)
    return (prod + np.asarray(zero, np.float32)[:, None]).astype(np.float32)


def code_bytes(d: int, bits: int) -> int:
    return (d * bits + 7) // 8


def pack_codes(codes, bits: int) -> np.ndarray:
    """uint8 [n, code_bytes]: element j at bits [b j, b j + b), little-endian."""
    codes = np.asarray(codes, np.uint64)
    n, d = codes.shape
    out = np.zeros((n, code_bytes(d, bits)), np.uint8)
    for j in range(d):
        bit = j * bits
        out[:, bit // 8] |= (codes[:, j] << np.uint64(bit % 8)).astype(np.uint8)
    return out


def unpack_codes(packed, d: int, bits: int) -> np.ndarray:
    packed = np.asarray(packed, np.uint8)
    out = np.zeros((packed.shape[0], d), np.uint8)
    mask = (1 << bits) - 1
    for j in range(d):
        bit = j * bits
        out[:, j] = (packed[:, bit // 8] >> (bit % 8)) & mask
    return out


def push(store, src, ids, base: int, accumulate: bool = False):
    """store[ids[k] - base] = src[k] (or += in float64, for gradients).
    Returns the updated copy."""
    store = np.array(store, copy=True)
    rows = np.asarray(ids, np.int64) - base
    if accumulate:
        store[rows] = store[rows] + src
    else:
        store[rows] = src
    return store
