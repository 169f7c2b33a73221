"""Philox4x32-10 counter-based generator (oracle side) and the sampling draws.

Written from the published definition: Salmon, Moraes, Dror, Shaw, "Parallel
random numbers: as easy as 1, 2, 3" (SC'11).  Ten rounds of the 4x32 Philox
S-box with multipliers 0xD2511F53 / 0xCD9E8D57 and Weyl key increments
0x9E3779B9 / 0xBB67AE85.  Pinned by the published known-answer vectors
(tests/golden/philox4x32_10_kat.txt).

The pages leave the random draws of the accept rule unspecified (LayerSkip blog
§3.3 calls ``random()`` and ``sample()``).  Reading taken: every draw is a
Philox word addressed by (iteration, row, purpose, element):
    key = (seed lo32, seed hi32), counter = (iteration, row, purpose, v // 4),
    word v % 4.
Purposes: 0 = draft sample, 1 = accept uniform, 2 = correction / bonus sample.
A word x becomes the uniform u = (2 * (x >> 9) + 1) * 2^-24 in (0, 1), exact in
float32.
"""
import numpy as np

PURPOSE_DRAFT = 0
PURPOSE_ACCEPT = 1
PURPOSE_SAMPLE = 2

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint32(0x9E3779B9)
_W1 = np.uint32(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  Counter words may be arrays (broadcast)."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint32) for c in (c0, c1, c2, c3))
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    c0, c1, c2, c3 = (np.array(c, dtype=np.uint32) for c in (c0, c1, c2, c3))
    k0 = np.uint32(k0)
    k1 = np.uint32(k1)
    with np.errstate(over="ignore"):
        for _ in range(10):
            p0 = _M0 * c0.astype(np.uint64)
            p1 = _M1 * c2.astype(np.uint64)
            n0 = (p1 >> np.uint64(32)).astype(np.uint32) ^ c1 ^ k0
            n1 = (p1 & _MASK32).astype(np.uint32)
            n2 = (p0 >> np.uint64(32)).astype(np.uint32) ^ c3 ^ k1
            n3 = (p0 & _MASK32).astype(np.uint32)
            c0, c1, c2, c3 = n0, n1, n2, n3
            k0 = np.uint32(k0 + _W0)
            k1 = np.uint32(k1 + _W1)
    return c0, c1, c2, c3


def words(seed, iteration, row, purpose, n):
    """The n Philox words for (iteration, row, purpose), elements 0..n-1."""
    seed = int(seed)
    k0, k1 = seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF
    nblk = (n + 3) // 4
    blk = np.arange(nblk, dtype=np.uint32)
    w = philox4x32_10(np.uint32(iteration), np.uint32(row), np.uint32(purpose), blk, k0, k1)
    return np.stack(w, axis=1).reshape(-1)[:n]


def uniforms(seed, iteration, row, purpose, n):
    """float32 uniforms in (0, 1): u = (2*(x>>9)+1) * 2^-24."""
    x = words(seed, iteration, row, purpose, n)
    return ((x >> np.uint32(9)).astype(np.float32) * np.float32(2.0) + np.float32(1.0)) * np.float32(2.0 ** -24)


def gumbel(seed, iteration, row, purpose, n):
    """float32 Gumbel(0,1) noise g = -log(-log u) for the exponential race."""
    u = uniforms(seed, iteration, row, purpose, n)
    return -np.log(-np.log(u))
