"""A CPU Philox4x32-10 for the tests, written from its published definition
(Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC 2011), independent of the library's device code.

Philox-4x32 with 10 rounds. Each round multiplies counter words 0 and 2 by
two fixed 32-bit multipliers, giving (hi, lo) halves of the 64-bit products.
The new counter is (hi_b ^ c1 ^ k0, lo_b, hi_a ^ c3 ^ k1, lo_a), where a is
the product of word 0 and b that of word 2. Between rounds each key word
advances by its Weyl constant (the golden ratio and sqrt(3) - 1 in 32-bit
fixed point).

normals() maps (seed, stream, element index) to standard normals the way the
library's built-in start documents it: element e uses block e // 4 with
counter (block low word, block high word, stream, 0) and key (seed low word,
seed high word). Words (x0, x1) and (x2, x3) are two Box-Muller pairs with
uniforms u = ((x >> 8) + 1/2) / 2^24, and element e takes normal e % 4:
sqrt(-2 ln u1) cos(2 pi u2) for even, the sine for odd.
"""
import numpy as np

MUL = (0xD2511F53, 0xCD9E8D57)
WEYL = (0x9E3779B9, 0xBB67AE85)
_M32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised over arrays of counters (each word < 2^32); the key is
    scalar. Returns the four output words as uint64 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _M32 for x in (c0, c1, c2, c3)]
    k0 = np.uint64(k0 & 0xFFFFFFFF)
    k1 = np.uint64(k1 & 0xFFFFFFFF)
    for _ in range(10):
        pa = np.uint64(MUL[0]) * c[0]            # < 2^64: exact in uint64
        pb = np.uint64(MUL[1]) * c[2]
        c = [(pb >> np.uint64(32)) ^ c[1] ^ k0, pb & _M32,
             (pa >> np.uint64(32)) ^ c[3] ^ k1, pa & _M32]
        k0 = (k0 + np.uint64(WEYL[0])) & _M32
        k1 = (k1 + np.uint64(WEYL[1])) & _M32
    return c


def normals(seed, stream, count):
    """float64 normals for element indices 0 .. count-1."""
    e = np.arange(count, dtype=np.uint64)
    blk = e >> np.uint64(2)
    x = philox4x32_10(blk & _M32, blk >> np.uint64(32), np.full(count, stream, np.uint64),
                      np.zeros(count, np.uint64), seed & 0xFFFFFFFF, seed >> 32)
    which = (e & np.uint64(3)).astype(np.int64)
    pair = which >> 1
    xa = np.where(pair == 0, x[0], x[2])
    xb = np.where(pair == 0, x[1], x[3])
    u1 = ((xa >> np.uint64(8)).astype(np.float64) + 0.5) / 16777216.0
    u2 = ((xb >> np.uint64(8)).astype(np.float64) + 0.5) / 16777216.0
    rad = np.sqrt(-2.0 * np.log(u1))
    ang = 2.0 * np.pi * u2
    return np.where(which & 1, rad * np.sin(ang), rad * np.cos(ang))
