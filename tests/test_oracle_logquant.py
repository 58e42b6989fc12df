"""Pins of the oracle's log-sparse retention (LogQuant).

"Resumo Técnico: LogQuant", Metodologia item 2: a full-precision reserve of 3W
tokens; when it is full, the older 2W are thinned to every other token
(the density of the earlier windows is halved) and the newest stay.  The
thinned-out tokens are quantized, not evicted (item 3), and the attention
does not depend on where in the cache a token sits (item 4).

Pins:
  - a worked example derived by hand from that description (tests/golden);
  - counting closed forms: no flush before 3W tokens, then one flush per W
    tokens, W tokens quantized per flush, 2W <= r < 3W afterwards;
  - every appended token is held exactly once (sink, quantized or full
    precision), and the newest W are always full precision;
  - the log-sparse shape: the gaps between the kept full-precision positions
    never grow towards the newest token, and are powers of two when W is;
  - agreement with the pure-Python formulation (oracle.brute) on codes,
    scales, zero points, full-precision rows and attention;
  - before the first flush the cache is plain full-precision attention.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "logquant_retention.json")


def _id_tokens(n, D):
    """Token t has every key and value channel equal to t + 1.

    A value group spanning all D channels is then constant, so the quantizer's
    degenerate-group rule reconstructs it exactly: a quantized token's
    dequantized value row names the token.
    """
    x = np.repeat((np.arange(n, dtype=np.float32) + 1.0)[:, None], D, axis=1)
    return x, x.copy()


def _ids(rows):
    return [int(round(float(r[0]))) - 1 for r in rows]


def _layout_ids(st):
    K, V = oracle.dequant_slice(st)
    nS, Lq = st["n_sink"], st["n_quant"]
    return _ids(st["sink_v"]), _ids(V[nS:nS + Lq]), _ids(st["res_v"])


def _cases():
    return json.load(open(GOLDEN))["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "n%d" % c["n"])
def test_golden_worked_example(case):
    cfg = json.load(open(GOLDEN))["config"]
    k, v = _id_tokens(case["n"], cfg["head_dim"])
    st = oracle.build_slice(k, v, **cfg)
    sinks, quant, fp = _layout_ids(st)
    assert sinks == case["sinks"]
    assert quant == case["quantized"]
    assert fp == case["full_precision"]


@pytest.mark.parametrize("S,W,G,n", [(0, 2, 2, 0), (0, 2, 2, 5), (0, 2, 2, 6), (2, 4, 2, 13),
                                     (1, 4, 4, 12), (3, 8, 4, 100), (0, 3, 1, 57)])
def test_counts_closed_form(S, W, G, n):
    k, v = _id_tokens(n, 8)
    st = oracle.build_slice(k, v, head_dim=8, bits=2, k_group=G, v_group=8, residual=3 * W,
                            n_sink=S, log_window=W)
    m = n - min(n, S)
    flushes = 0 if m < 3 * W else (m - 3 * W) // W + 1
    assert st["n_sink"] == min(n, S)
    assert st["flushes"] == flushes
    assert st["n_quant"] == W * flushes
    assert st["n_resid"] == m - W * flushes
    if flushes:
        assert 2 * W <= st["n_resid"] < 3 * W


@pytest.mark.parametrize("W", [1, 2, 3, 4, 6, 8])
def test_every_token_once_newest_kept_and_log_sparse_gaps(W):
    D = 8
    n_max = 40 * W + 7
    k, v = _id_tokens(n_max, D)
    for n in range(0, n_max + 1, max(1, W // 2)):
        st = oracle.build_slice(k[:n], v[:n], head_dim=D, bits=2, k_group=1, v_group=D,
                                residual=3 * W, n_sink=1, log_window=W)
        sinks, quant, fp = _layout_ids(st)
        assert sorted(sinks + quant + fp) == list(range(n))
        newest = list(range(max(1, n - W), n))
        assert fp[len(fp) - len(newest):] == newest
        gaps = np.diff(fp)
        assert (gaps > 0).all()
        assert (gaps[:-1] >= gaps[1:]).all(), (n, fp)
        if W & (W - 1) == 0:
            assert all(g & (g - 1) == 0 for g in gaps.tolist()), (n, fp)


@pytest.mark.parametrize("bits,codec,S,W,G,GV,n", [(2, 0, 0, 4, 2, 8, 37), (4, 1, 2, 4, 4, 4, 41),
                                                   (8, 0, 1, 2, 2, 8, 23), (4, 0, 0, 8, 4, 8, 70)])
def test_matches_brute(bits, codec, S, W, G, GV, n):
    D = 8
    rng = np.random.default_rng(n * 7 + bits)
    k = (rng.standard_normal((n, D)) * 2).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    cfg = dict(bits=bits, k_group=G, v_group=GV, residual=3 * W, n_sink=S, codec=codec, log_window=W)
    st = oracle.build_slice(k, v, head_dim=D, **cfg)
    br = brute.build_slice(k.tolist(), v.tolist(), **cfg)
    assert st["flushes"] == br["flushes"]
    np.testing.assert_array_equal(st["k_codes"], np.array(br["k_codes"], np.uint8).reshape(-1, D))
    np.testing.assert_array_equal(st["v_codes"], np.array(br["v_codes"], np.uint8).reshape(-1, D))
    ks = np.array([[m[0] for m in g] for g in br["k_meta"]], np.float32).reshape(-1, D)
    kz = np.array([[m[1] for m in g] for g in br["k_meta"]], np.float32).reshape(-1, D)
    np.testing.assert_array_equal(st["k_scale"].view(np.uint32), ks.view(np.uint32))
    np.testing.assert_array_equal(st["k_zero"].view(np.uint32), kz.view(np.uint32))
    vs = np.array([[m[0] for m in t] for t in br["v_meta"]], np.float32).reshape(-1, D // GV)
    vz = np.array([[m[1] for m in t] for t in br["v_meta"]], np.float32).reshape(-1, D // GV)
    np.testing.assert_array_equal(st["v_scale"].view(np.uint32), vs.view(np.uint32))
    np.testing.assert_array_equal(st["v_zero"].view(np.uint32), vz.view(np.uint32))
    np.testing.assert_array_equal(st["res_k"], np.array(br["res_k"], np.float32).reshape(-1, D))
    np.testing.assert_array_equal(st["res_v"], np.array(br["res_v"], np.float32).reshape(-1, D))
    K, V = oracle.dequant_slice(st)
    Kb = np.array(br["sinks_k"] + br["qk"] + br["res_k"], np.float32).reshape(-1, D)
    Vb = np.array(br["sinks_v"] + br["qv"] + br["res_v"], np.float32).reshape(-1, D)
    np.testing.assert_array_equal(K, Kb)
    np.testing.assert_array_equal(V, Vb)
    q = rng.standard_normal(D).astype(np.float32)
    o, l = oracle.attention(q, K, V, 0.3)
    ob, lb = brute.attention(q.tolist(), Kb.tolist(), Vb.tolist(), 0.3)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    assert abs(l - lb) <= 1e-12


def test_before_first_flush_is_plain_attention():
    D, W = 16, 4
    rng = np.random.default_rng(3)
    k = rng.standard_normal((3 * W - 1 + 2, D)).astype(np.float32)
    v = rng.standard_normal(k.shape).astype(np.float32)
    st = oracle.build_slice(k, v, head_dim=D, bits=2, k_group=4, v_group=16, residual=3 * W,
                            n_sink=2, log_window=W)
    assert st["n_quant"] == 0 and st["flushes"] == 0
    K, V = oracle.dequant_slice(st)
    np.testing.assert_array_equal(K, k)
    np.testing.assert_array_equal(V, v)


def test_rejects_inconsistent_window():
    k, v = _id_tokens(4, 8)
    for residual, W, G in ((8, 2, 2), (12, 4, 8), (6, -1, 2)):
        with pytest.raises(ValueError):
            oracle.build_slice(k, v, head_dim=8, bits=2, k_group=G, v_group=8, residual=residual,
                               n_sink=0, log_window=W)
