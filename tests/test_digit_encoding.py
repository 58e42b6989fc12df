"""The fixed-point digit encoding the decode kernels use, checked on the CPU.

The VALU stream splits an integer |n| <= 2^18 (the fixed-point image of a folded
query element or of a softmax weight) into five balanced base-16 digits in
[-8, 7], stored as two's-complement nibbles, and gets all five from one add and
one xor: nibble i of (n + 0x88888) ^ 0x88888.  The matrix-core stream splits the
same range into three balanced base-256 digits, bytes of (n + 32896) ^ 0x8080.
Both must reproduce n exactly over the whole range, and each digit must lie in
its balanced range, or the integer dot products would not be exact.
"""
import numpy as np

LIMIT = 1 << 18


def _signed(field, bits):
    return np.where(field >= (1 << (bits - 1)), field - (1 << bits), field)


def test_five_balanced_hex_digits_from_add_and_xor():
    n = np.arange(-LIMIT, LIMIT + 1, dtype=np.int64)
    x = ((n + 0x88888) & 0xFFFFFFFF) ^ 0x88888
    total = np.zeros_like(n)
    for i in range(5):
        d = _signed((x >> (4 * i)) & 15, 4)
        assert d.min() >= -8 and d.max() <= 7
        total += d << (4 * i)
    assert np.array_equal(total, n)
    # the bits above the five nibbles carry nothing the kernels read
    assert np.all((x >> 20) == 0)


def test_three_balanced_byte_digits():
    n = np.arange(-LIMIT, LIMIT + 1, dtype=np.int64)
    x = ((n + 32896) & 0xFFFFFFFF) ^ 0x8080
    total = np.zeros_like(n)
    for i in range(3):
        d = _signed((x >> (8 * i)) & 255, 8)
        assert d.min() >= -128 and d.max() <= 127
        total += d << (8 * i)
    assert np.array_equal(total, n)


def test_pair_bytes_interleave_two_tokens_per_limb():
    # byte li // 2 of ev (li even) or od (li odd) holds limb li of the first integer
    # in its low nibble and of the second in its high nibble
    rng = np.random.default_rng(7)
    a = rng.integers(-LIMIT, LIMIT + 1, 4096)
    b = rng.integers(-LIMIT, LIMIT + 1, 4096)
    xa = ((a + 0x88888) & 0xFFFFFFFF) ^ 0x88888
    xb = ((b + 0x88888) & 0xFFFFFFFF) ^ 0x88888
    ev = (xa & 0x0F0F0F) | ((xb << 4) & 0xF0F0F0)
    od = ((xa >> 4) & 0x0F0F0F) | (xb & 0xF0F0F0)
    for li in range(5):
        byte = ((od if li & 1 else ev) >> (8 * (li >> 1))) & 0xFF
        assert np.array_equal(byte & 15, (xa >> (4 * li)) & 15)
        assert np.array_equal(byte >> 4, (xb >> (4 * li)) & 15)
