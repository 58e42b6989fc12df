"""Pins of the oracle's head-granular keys (Atom's KV-cache quantization).

"Atom: Low-bit Quantization for Efficient and Accurate LLM Serving" (paper
review), section 三, model-components table, KV-cache row: the KV cache is
quantized to low bits, asymmetrically, at attention-head granularity.  Reading:
each token's key (the head_dim channels of one kv head) is one group of the
asymmetric min-max quantizer (key_axis = 1), as a token's value is with
v_group = head_dim; the cache's residual and flushes are unchanged.

Pins:
  - a hand-derived two-token cache (tests/golden/head_granular_keys.json): codes,
    scales, zero points and dequantized rows of keys and values, and the
    per-channel codes of the same tokens, which differ;
  - invariants on random slices: one scale and zero point per quantized token,
    codes in range, every key row within half a step of its token's scale, the
    row minimum at code 0, constant rows reproduced exactly, and each token's
    key group equal to the quantizer applied to that row alone;
  - agreement with the pure-Python formulation (oracle.brute) on codes, scales,
    zero points, dequantized rows and attention, across code widths, both
    codecs, sinks and log-sparse retention;
  - outliers are refused with per-token keys.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "head_granular_keys.json")


def _cases():
    return json.load(open(GOLDEN))["cases"]


def _f32eq(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["id"])
def test_golden_cache(case):
    k = np.array(case["k"], np.float32)
    v = np.array(case["v"], np.float32)
    kw = dict(head_dim=case["head_dim"], bits=case["bits"], k_group=case["k_group"], v_group=case["v_group"],
              residual=case["residual"], n_sink=case["n_sink"])
    st = oracle.build_slice(k, v, key_axis=1, **kw)
    assert st["n_quant"] == len(case["k"]) and st["n_resid"] == 0
    assert st["k_codes"].tolist() == case["k_codes"]
    assert _f32eq(st["k_scale"].ravel(), case["k_scale"]) and _f32eq(st["k_zero"].ravel(), case["k_zero"])
    assert st["v_codes"].tolist() == case["v_codes"]
    assert _f32eq(st["v_scale"].ravel(), case["v_scale"]) and _f32eq(st["v_zero"].ravel(), case["v_zero"])
    K, V = oracle.dequant_slice(st)
    assert _f32eq(K, case["k_dequant"]) and _f32eq(V, case["v_dequant"])
    # the KIVI axis on the same tokens gives other codes
    st0 = oracle.build_slice(k, v, key_axis=0, **kw)
    assert st0["k_codes"].tolist() == case["per_channel_k_codes"] != case["k_codes"]


def _slice(rng, n, D, **kw):
    k = (rng.standard_normal((n, D)) * rng.choice([0.05, 1.0, 20.0], size=(1, D))).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    return k, v


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("codec", [0, 1])
def test_invariants_random_slices(bits, codec):
    rng = np.random.default_rng(100 + bits * 3 + codec)
    D, G, R = 16, 4, 8
    k, v = _slice(rng, 70, D)
    k[9] = 3.25          # a constant key row (quantized at the first flush)
    st = oracle.build_slice(k, v, head_dim=D, bits=bits, k_group=G, v_group=8, residual=R, n_sink=2,
                            codec=codec, key_axis=1)
    Lq = st["n_quant"]
    assert st["k_scale"].shape == (Lq, 1) and st["k_zero"].shape == (Lq, 1)
    assert st["k_codes"].max() <= (1 << bits) - 1
    K, _ = oracle.dequant_slice(st)
    rows = k[2:2 + Lq]                       # the quantized tokens, in order (after 2 sinks)
    for t in range(Lq):
        s, z, q = oracle.quant_group(rows[t], bits, codec)
        assert _f32eq(st["k_scale"][t, 0], s) and _f32eq(st["k_zero"][t, 0], z)
        assert st["k_codes"][t].tolist() == q.tolist()
        kq = K[2 + t]
        if codec == 0:
            mn, mx = rows[t].min(), rows[t].max()
            slack = 2.0 ** -20 * (abs(float(mn)) + abs(float(mx)))
            assert np.all(np.abs(kq.astype(np.float64) - rows[t]) <= float(s) / 2 + slack)
            assert q[int(np.argmin(rows[t]))] == 0
    if codec == 0:   # the asymmetric degenerate rule reproduces a constant row exactly
        assert np.all(K[2 + 7] == np.float32(3.25))


@pytest.mark.parametrize("bits,codec,S,W,D,GV,n,seed", [
    (4, 0, 0, 0, 8, 8, 37, 0),
    (2, 0, 2, 0, 8, 4, 45, 1),
    (8, 1, 0, 0, 16, 16, 40, 2),
    (2, 1, 1, 4, 8, 8, 61, 3),      # log-sparse retention (R = 12)
    (4, 0, 0, 2, 8, 8, 29, 4),      # log-sparse retention (R = 6)
])
def test_matches_brute(bits, codec, S, W, D, GV, n, seed):
    rng = np.random.default_rng(seed)
    k, v = _slice(rng, n, D)
    G = 2
    R = 3 * W if W else 8
    st = oracle.build_slice(k, v, head_dim=D, bits=bits, k_group=G, v_group=GV, residual=R, n_sink=S,
                            codec=codec, log_window=W, key_axis=1)
    br = brute.build_slice(k, v, bits=bits, k_group=G, v_group=GV, residual=R, n_sink=S, codec=codec,
                           log_window=W, key_axis=1)
    assert st["k_codes"].tolist() == br["k_codes"]
    assert _f32eq(st["k_scale"].ravel(), [m[0][0] for m in br["k_meta"]])
    assert _f32eq(st["k_zero"].ravel(), [m[0][1] for m in br["k_meta"]])
    assert st["v_codes"].tolist() == br["v_codes"]
    K, V = oracle.dequant_slice(st)
    nS, Lq = st["n_sink"], st["n_quant"]
    assert _f32eq(K[nS:nS + Lq], br["qk"]) and _f32eq(V[nS:nS + Lq], br["qv"])
    q = rng.standard_normal(D).astype(np.float32)
    scale = oracle.default_scale(D)
    o1, l1 = oracle.attention(q, K, V, scale)
    rows_k = br["sinks_k"] + br["qk"] + br["res_k"]
    rows_v = br["sinks_v"] + br["qv"] + br["res_v"]
    o2, l2 = brute.attention(q, rows_k, rows_v, scale)
    assert np.abs(o1 - o2).max() < 1e-12 and abs(l1 - l2) < 1e-12
    # the batched decode step reads the per-token key layout
    ob, lb = oracle.decode_slices([st], q[None, None, :], scale)
    assert np.abs(ob[0, 0] - o1).max() < 1e-12 and abs(lb[0, 0] - l1) < 1e-12


def test_per_token_keys_refuse_outliers():
    k = np.zeros((8, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.build_slice(k, k, head_dim=8, bits=4, k_group=2, v_group=8, residual=4, n_sink=0, outliers=1,
                           key_axis=1)
