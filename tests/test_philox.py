"""Pins of the tests' CPU Philox4x32-10 (tests/philox_cpu.py): the known-
answer vectors published with the generator's reference implementation
(Random123), and the moments of the Box-Muller normals built on it. The GPU
test of the library's built-in start compares against this generator."""
import numpy as np
import pytest

from philox_cpu import normals, philox4x32_10

# (counter words, key words, output words), Philox4x32 with 10 rounds
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr, key, out", KAT)
def test_known_answer_vectors(ctr, key, out):
    got = philox4x32_10(*[np.array([w]) for w in ctr], *key)
    assert tuple(int(g[0]) for g in got) == out


def test_vectorised_matches_scalar_calls():
    rng = np.random.default_rng(0)
    words = rng.integers(0, 2 ** 32, size=(4, 16), dtype=np.uint64)
    vec = philox4x32_10(*words, 0x12345678, 0x9abcdef0)
    for j in range(16):
        one = philox4x32_10(*[words[i, j:j + 1] for i in range(4)], 0x12345678, 0x9abcdef0)
        assert [int(o[0]) for o in one] == [int(v[j]) for v in vec]


def test_normals_moments():
    n = 1 << 20
    z = normals(0x0123456789abcdef, 0, n)
    assert np.all(np.isfinite(z))
    se = 1.0 / np.sqrt(n)
    assert abs(z.mean()) < 5 * se
    assert abs(z.var() - 1.0) < 5 * np.sqrt(2.0) * se
    assert abs(np.mean(z ** 3)) < 5 * np.sqrt(15.0) * se          # odd moment: 0
    assert abs(np.mean(z ** 4) - 3.0) < 5 * np.sqrt(96.0) * se    # kurtosis 3
    # the cosine and sine members of a pair are uncorrelated
    assert abs(np.mean(z[0::2] * z[1::2])) < 5 * np.sqrt(2.0) * se
    # streams differ
    z1 = normals(0x0123456789abcdef, 1, 4096)
    assert not np.allclose(z1, z[:4096])
