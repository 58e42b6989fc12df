"""Pins of the oracle's group quantizer against what the pages and arithmetic fix.

- Hand-derived worked examples (tests/golden/codec_examples.json): the formulas of
  'Atom: Low-bit Quantization for Efficient and Accurate LLM Serving', section 三
  '核心公式', and the dequantization of 'KV Cache的Int4量化：如何解决Attention Sink导致
  的量化精度崩塌问题', section 2, worked by hand in binary32.
- Invariants that hold for any input: codes in range, the s/2 reconstruction bound,
  exact constant groups, min maps to code 0, exact grid reconstruction, dequant as
  one rounded product.
- Agreement with the independent pure-Python formulation (oracle.brute).
- The symmetric quantizer (codec 1) of the same Atom section: worked examples,
  and invariants (fixed zero point 2^(n-1), s/2 bound inside the signed range,
  clipping only above it, odd symmetry of the codes, exact zero).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_examples.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _f32(s):
    return np.float32(s)


def _bits(x):
    return int(np.asarray(x, np.float32).view(np.uint32))


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["id"])
def test_golden_example(case):
    x = np.array([_f32(v) for v in case["x"]], np.float32)
    s, z, q = oracle.quant_group(x, case["bits"], case.get("codec", 0))
    assert _bits(s) == int(case["scale_bits"], 16), (float(s), case["scale"])
    assert s == _f32(case["scale"])
    assert _bits(z) == _bits(_f32(case["zero"]))  # +0, never -0
    assert list(q) == case["codes"]
    deq = oracle.dequant(q, s, z)
    want = np.array([_f32(v) for v in case["deq"]], np.float32)
    assert np.array_equal(deq.view(np.uint32), want.view(np.uint32)), (deq, want)
    if "deq_bits" in case:
        assert [_bits(d) for d in deq] == [int(b, 16) for b in case["deq_bits"]]


def _random_groups(seed, n_groups, bits):
    rng = np.random.default_rng(seed)
    for i in range(n_groups):
        m = int(rng.choice([2, 3, 16, 32, 64, 128]))
        kind = i % 6
        if kind == 0:
            x = rng.standard_normal(m)
        elif kind == 1:
            x = rng.standard_normal(m) * 10.0 + rng.uniform(-50, 50)
        elif kind == 2:       # one-signed, narrow: zero point far outside the code range
            x = 5.0 + rng.uniform(0, 1, m)
        elif kind == 3:       # few distinct values (ties)
            x = rng.integers(-3, 4, m) * 0.25
        elif kind == 4:       # tiny magnitudes, including binary32 subnormals
            x = rng.standard_normal(m) * 1e-40
        else:                 # heavy tail
            x = rng.standard_t(2, m)
        yield np.asarray(x, np.float32)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_invariants_random_groups(bits):
    qmax = (1 << bits) - 1
    for x in _random_groups(1234 + bits, 600, bits):
        s, z, q = oracle.quant_group(x, bits)
        assert s > 0 and np.isfinite(s)
        assert z == np.rint(z) and not (z == 0 and np.signbit(z))
        # I1: codes in [0, 2^n - 1]
        assert q.min() >= 0 and q.max() <= qmax
        xd = oracle.dequant(q, s, z)
        mn, mx = x.min(), x.max()
        if mn == mx:
            # I3: constant groups reproduce exactly
            assert np.array_equal(xd, x)
            assert np.all(q == 0)
            continue
        # I2: |x' - x| <= s/2 up to a few binary32 roundings (and the rounding of a
        # subnormal s, at most 2^-150, times up to 2^n code steps)
        slack = 2.0 ** -20 * (abs(float(mn)) + abs(float(mx))) + (qmax + 1) * 2.0 ** -149 + 1e-44
        err = np.abs(xd.astype(np.float64) - x.astype(np.float64))
        assert np.all(err <= float(s) / 2 + slack), (x, s, z, q, err.max())
        # I4: the minimum maps to code 0, the maximum to one of the top two codes
        assert np.all(q[x == mn] == 0)
        if abs(float(mn)) / float(s) < 2 ** 22:
            assert np.all(q[x == mx] >= qmax - 1)
        # I6: dequant is a single rounded product of (code - z) and s
        d = (q.astype(np.float32) - z).astype(np.float32)
        assert np.array_equal(xd, (d * s).astype(np.float32))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_exact_grid_reconstruction(bits):
    # I5: values on the grid min + k*s with an exactly representable s come back exactly
    qmax = (1 << bits) - 1
    rng = np.random.default_rng(7 + bits)
    for _ in range(200):
        e = int(rng.integers(-6, 6))
        s = np.float32(2.0 ** e)
        base = np.float32(int(rng.integers(-40, 40))) * s
        k = rng.integers(0, qmax + 1, 32)
        k[0], k[1] = 0, qmax
        x = (base + k.astype(np.float32) * s).astype(np.float32)
        s_, z, q = oracle.quant_group(x, bits)
        assert s_ == s
        assert np.array_equal(oracle.dequant(q, s_, z), x)
        assert np.array_equal(q.astype(np.int64), k)


def test_signed_zero_inputs():
    for x in ([0.0, -0.0, 0.0], [-0.0, -0.0], [-0.0, 1.0], [0.0, -1.0]):
        x = np.array(x, np.float32)
        s, z, q = oracle.quant_group(x, 4)
        assert not np.signbit(z)
        xd = oracle.dequant(q, s, z)
        assert np.allclose(xd, x, atol=float(s) / 2)


def test_underflowing_scale_uses_degenerate_rule():
    # range so small that range / 15 rounds to zero in binary32
    tiny = np.float32(1.4e-45)  # smallest subnormal
    x = np.array([tiny, 2 * tiny, tiny], np.float32)
    s, z, q = oracle.quant_group(x, 4)
    assert s == tiny and z == -1
    assert np.array_equal(oracle.dequant(q, s, z), x)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_matches_pure_python_formulation(bits):
    for x in _random_groups(99 + bits, 300, bits):
        s, z, q = oracle.quant_group(x, bits)
        s2, z2, q2 = brute.quant_group(list(x), bits)
        assert _bits(s) == _bits(s2) and _bits(z) == _bits(z2)
        assert list(q) == q2


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_symmetric_invariants_random_groups(bits):
    qmax = (1 << bits) - 1
    half = 1 << (bits - 1)
    for x in _random_groups(4321 + bits, 600, bits):
        s, z, q = oracle.quant_group(x, bits, 1)
        amax = float(np.abs(x).max())
        assert s > 0 and np.isfinite(s)
        # the zero point is 2^(n-1): stored codes are the signed codes plus 2^(n-1)
        assert z == half
        assert q.min() >= 0 and q.max() <= qmax
        xd = oracle.dequant(q, s, z)
        # dequant is a single rounded product of (code - z) and s
        d = (q.astype(np.float32) - z).astype(np.float32)
        assert np.array_equal(xd, (d * s).astype(np.float32))
        if amax == 0.0:
            assert np.all(q == half) and np.all(xd == 0)
            continue
        # the scale is 2 max|x| / (2^n - 1) within one rounding (or the degenerate rule)
        if float(s) != amax:
            assert abs(float(s) - 2 * amax / qmax) <= 2.0 ** -23 * float(s) + 1e-45
        # |x' - x| <= s/2 inside the signed range; above it the code is clipped to the top
        xs = x.astype(np.float64)
        inside = xs <= (half - 0.5) * float(s) * (1 - 2.0 ** -20)
        slack = 2.0 ** -20 * amax + (qmax + 1) * 2.0 ** -149 + 1e-44
        err = np.abs(xd.astype(np.float64) - xs)
        assert np.all(err[inside] <= float(s) / 2 + slack), (x, s, q)
        assert np.all(q[xs > (half - 0.5) * float(s) * (1 + 2.0 ** -20)] == qmax)
        # a zero input is reproduced exactly
        assert np.all(xd[x == 0] == 0)
        # odd symmetry: x and -x get codes that mirror around z (both inside the range)
        sym = np.concatenate([x, -x])
        s2, z2, q2 = oracle.quant_group(sym, bits, 1)
        m = x.size
        ok = (np.abs(sym[:m].astype(np.float64)) <= (half - 0.5) * float(s2) * (1 - 2.0 ** -20))
        assert np.all((q2[:m].astype(int) + q2[m:].astype(int))[ok] == 2 * half)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_symmetric_matches_pure_python_formulation(bits):
    for x in _random_groups(77 + bits, 300, bits):
        s, z, q = oracle.quant_group(x, bits, 1)
        s2, z2, q2 = brute.quant_group(list(x), bits, 1)
        assert _bits(s) == _bits(s2) and _bits(z) == _bits(z2)
        assert list(q) == q2
