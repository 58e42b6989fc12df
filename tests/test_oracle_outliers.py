"""Pins of the oracle's dense-and-sparse groups (KVQuant).

"LLM系列：KVCache量化1 KIVI…" page, section 3 "KVQuant", item (4): per-vector
dense-and-sparse quantization keeps a small share of numeric outliers (e.g. 1%)
unquantized, in a sparse matrix beside the codes.  Reading: one outlier per
quantization vector, the element of largest magnitude (first among equals); the
others set the scale and zero point; the outlier dequantizes to itself.

Pins:
  - hand-derived examples (tests/golden/outlier_examples.json): the outlier left
    out of the range, a tie in magnitude, a symmetric group, a constant group;
  - invariants on random groups: the outlier is the first element of largest
    magnitude (numpy's argmax), the others round-trip within half a step, the
    scale is the one the other elements alone would get;
  - slices: exactly one outlier per key channel group and per value group, each
    dequantized to its exact value, and agreement with the pure-Python
    formulation (oracle.brute) on codes, scales, zero points, outliers, rows and
    attention.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "outlier_examples.json")


def _cases():
    return json.load(open(GOLDEN))["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["id"])
def test_golden_example(case):
    s, z, q, o = oracle.quant_group_sparse(np.array(case["x"], np.float32), case["bits"], case["codec"])
    assert o == case["outlier"]
    assert np.float32(s) == np.float32(case["scale"])
    assert np.float32(z) == np.float32(case["zero"])
    assert q.tolist() == case["codes"]
    deq = [float(x) if i == o else float(oracle.dequant(np.array([c], np.uint8), s, z)[0])
           for i, (x, c) in enumerate(zip(np.array(case["x"], np.float32), q))]
    assert np.array_equal(np.array(deq, np.float32), np.array(case["dequant"], np.float32))


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("codec", [0, 1])
def test_invariants_random_groups(bits, codec):
    rng = np.random.default_rng(bits * 10 + codec)
    for trial in range(300):
        m = int(rng.integers(2, 40))
        x = (rng.standard_normal(m) * rng.choice([0.01, 1.0, 30.0])).astype(np.float32)
        if trial % 7 == 0:
            x[rng.integers(m)] *= 50.0        # a strong outlier
        if trial % 11 == 0:
            x[:] = np.round(x)                # ties in magnitude
        s, z, q, o = oracle.quant_group_sparse(x, bits, codec)
        assert o == int(np.argmax(np.abs(x)))
        rest = np.delete(x, o)
        s2, z2, _ = oracle.quant_group(rest, bits, codec)
        assert np.float32(s) == np.float32(s2) and np.float32(z) == np.float32(z2)
        assert q.max() <= (1 << bits) - 1
        deq = oracle.dequant(q, s, z)
        err = np.abs(np.delete(deq, o).astype(np.float64) - rest.astype(np.float64))
        if codec == 0:
            assert (err <= 0.5 * float(s) * (1 + 1e-5) + 1e-30).all()
        else:  # inside the signed range [-2^(n-1), 2^(n-1) - 1] steps
            inside = rest.astype(np.float64) <= ((1 << (bits - 1)) - 1) * float(s)
            assert (err[inside] <= 0.5 * float(s) * (1 + 1e-5) + 1e-30).all()


def _slice(bits, codec, S, G, GV, R, n, seed, W=0):
    D = 16
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((n, D)) * 2).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    k[rng.random((n, D)) < 0.02] *= 20.0
    v[rng.random((n, D)) < 0.02] *= 20.0
    cfg = dict(bits=bits, k_group=G, v_group=GV, residual=R, n_sink=S, codec=codec, log_window=W)
    return k, v, cfg, oracle.build_slice(k, v, head_dim=D, outliers=1, **cfg)


@pytest.mark.parametrize("bits,codec,S,G,GV,R,n,W", [(4, 0, 0, 4, 8, 8, 37, 0), (2, 1, 2, 8, 4, 16, 50, 0),
                                                     (8, 0, 1, 4, 16, 12, 41, 4), (2, 0, 0, 2, 2, 4, 23, 0)])
def test_slice_outliers_exact_and_matches_brute(bits, codec, S, G, GV, R, n, W):
    k, v, cfg, st = _slice(bits, codec, S, G, GV, R, n, n + bits, W)
    D = k.shape[1]
    Lq, nS = st["n_quant"], st["n_sink"]
    assert Lq > 0
    K, V = oracle.dequant_slice(st)
    br = brute.build_slice(k.tolist(), v.tolist(), outliers=1, **cfg)
    # one outlier per key channel group and per value group, dequantized exactly
    assert st["ko_idx"].shape == (Lq // G, D) and (st["ko_idx"] >= 0).all() and (st["ko_idx"] < G).all()
    assert st["vo_idx"].shape == (Lq, D // GV) and (st["vo_idx"] >= 0).all() and (st["vo_idx"] < GV).all()
    for g in range(Lq // G):
        for c in range(D):
            t = g * G + st["ko_idx"][g, c]
            assert K[nS + t, c] == st["ko_val"][g, c]
    for t in range(Lq):
        for h in range(D // GV):
            c = h * GV + st["vo_idx"][t, h]
            assert V[nS + t, c] == st["vo_val"][t, h]
    # the brute formulation: codes, metadata, outliers, rows, attention
    np.testing.assert_array_equal(st["k_codes"], np.array(br["k_codes"], np.uint8).reshape(-1, D))
    np.testing.assert_array_equal(st["v_codes"], np.array(br["v_codes"], np.uint8).reshape(-1, D))
    ks = np.array([[m[0] for m in blk] for blk in br["k_meta"]], np.float32)
    np.testing.assert_array_equal(st["k_scale"].view(np.uint32), ks.view(np.uint32))
    ko = np.array([[o for o, _ in blk] for blk in br["k_out"]], np.int32)
    kv = np.array([[x for _, x in blk] for blk in br["k_out"]], np.float32)
    np.testing.assert_array_equal(st["ko_idx"], ko)
    np.testing.assert_array_equal(st["ko_val"].view(np.uint32), kv.view(np.uint32))
    vo = np.array([[o for o, _ in tok] for tok in br["v_out"]], np.int32)
    np.testing.assert_array_equal(st["vo_idx"], vo)
    Kb = np.array(br["sinks_k"] + br["qk"] + br["res_k"], np.float32).reshape(-1, D)
    Vb = np.array(br["sinks_v"] + br["qv"] + br["res_v"], np.float32).reshape(-1, D)
    np.testing.assert_array_equal(K.view(np.uint32), Kb.view(np.uint32))
    np.testing.assert_array_equal(V.view(np.uint32), Vb.view(np.uint32))
    q = np.random.default_rng(1).standard_normal(D).astype(np.float32)
    o1, l1 = oracle.attention(q, K, V, 0.25)
    o2, l2 = brute.attention(q.tolist(), Kb.tolist(), Vb.tolist(), 0.25)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    assert abs(l1 - l2) <= 1e-12


def test_batched_decode_uses_outliers():
    D = 16
    sts = []
    for seed in range(3):
        rng = np.random.default_rng(seed)
        k = (rng.standard_normal((40, D)) * 3).astype(np.float32)
        v = rng.standard_normal((40, D)).astype(np.float32)
        sts.append(oracle.build_slice(k, v, head_dim=D, bits=2, k_group=8, v_group=8, residual=8,
                                      n_sink=0, outliers=1))
    q = np.random.default_rng(9).standard_normal((3, 2, D)).astype(np.float32)
    out, lse = oracle.decode_slices(sts, q, 0.3)
    for i, st in enumerate(sts):
        K, V = oracle.dequant_slice(st)
        for h in range(2):
            o, l = oracle.attention(q[i, h], K, V, 0.3)
            np.testing.assert_allclose(out[i, h], o, rtol=0, atol=1e-12)
            assert abs(lse[i, h] - l) <= 1e-12
