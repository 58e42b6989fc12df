"""Pins of the oracle's cache state machine and attention.

State machine (KIVI notes, 'LLM系列：KVCache量化1 KIVI…', section 1: keys split into a
grouped part and a full-precision residual that is quantized and appended when it
reaches R tokens, then emptied):
  - counting closed forms Lq = R*floor((N-S)/R), r = (N-S) mod R;
  - the flush falls exactly on the append that makes the residual hold R tokens;
  - key groups run per channel over G consecutive tokens, value groups per token over
    G_V consecutive channels (checked against the pure-Python formulation and against
    a direct regrouping of the quantizer).
Attention (Int4 KV-cache post, section 3, softmax(QK^T/sqrt(d_k))V; LogQuant summary,
Metodologia item 4, order independence):
  - closed forms: equal keys or q = 0 give the mean of V'; one token gives v';
  - token permutation leaves the result unchanged;
  - a cache with no quantized tokens equals torch's scaled_dot_product_attention in
    float64;
  - explicit-loop brute force (oracle.brute) to 1e-12.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from oracle import brute


def _cfg(**kw):
    base = dict(head_dim=16, bits=4, k_group=4, v_group=8, residual=8, n_sink=0)
    base.update(kw)
    return base


def _tokens(seed, n, D, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, D)) * scale).astype(np.float32), \
        (rng.standard_normal((n, D)) * scale).astype(np.float32)


@pytest.mark.parametrize("S,R,G,n", [(0, 8, 4, 0), (0, 8, 4, 7), (0, 8, 4, 8), (0, 8, 8, 29),
                                     (3, 8, 4, 2), (3, 8, 4, 3), (3, 8, 2, 40), (5, 16, 4, 100)])
def test_counts_closed_form(S, R, G, n):
    k, v = _tokens(n + 11, n, 16)
    st = oracle.build_slice(k, v, **_cfg(residual=R, k_group=G, n_sink=S))
    nS = min(n, S)
    assert st["n_sink"] == nS
    assert st["n_quant"] == R * ((n - nS) // R)
    assert st["n_resid"] == (n - nS) % R
    assert st["flushes"] == (n - nS) // R
    assert 0 <= st["n_resid"] < R


def test_flush_exactly_at_R():
    cfg = _cfg(residual=8, k_group=4)
    k, v = _tokens(5, 24, 16)
    prev = None
    for n in range(0, 25):
        st = oracle.build_slice(k[:n], v[:n], **cfg)
        if prev is not None:
            flushed = st["flushes"] - prev["flushes"]
            assert flushed == (1 if n % 8 == 0 else 0), n
        prev = st


def test_quantized_part_is_prefix_stable():
    # appending more tokens never changes groups that are already quantized
    cfg = _cfg(residual=8, k_group=4, n_sink=2)
    k, v = _tokens(6, 60, 16)
    a = oracle.build_slice(k[:34], v[:34], **cfg)
    b = oracle.build_slice(k, v, **cfg)
    L = a["n_quant"]
    assert np.array_equal(a["k_codes"], b["k_codes"][:L])
    assert np.array_equal(a["k_scale"], b["k_scale"][:L // 4])
    assert np.array_equal(a["v_codes"], b["v_codes"][:L])
    assert np.array_equal(a["sink_k"], b["sink_k"])


def test_grouping_axes_by_direct_regrouping():
    # key group j, channel c quantizes tokens [S + jG, S + (j+1)G) of channel c;
    # value group h of token t quantizes channels [h G_V, (h+1) G_V) of that token.
    D, G, GV, R, S, bits = 16, 4, 8, 8, 2, 2
    k, v = _tokens(8, 2 + 24 + 5, D, scale=3.0)
    st = oracle.build_slice(k, v, head_dim=D, bits=bits, k_group=G, v_group=GV,
                            residual=R, n_sink=S)
    assert st["n_quant"] == 24 and st["n_resid"] == 5
    for j in range(24 // G):
        for c in range(D):
            s, z, q = oracle.quant_group(k[S + j * G:S + (j + 1) * G, c], bits)
            assert st["k_scale"][j, c] == s and st["k_zero"][j, c] == z
            assert np.array_equal(st["k_codes"][j * G:(j + 1) * G, c], q)
    for t in range(24):
        for h in range(D // GV):
            s, z, q = oracle.quant_group(v[S + t, h * GV:(h + 1) * GV], bits)
            assert st["v_scale"][t, h] == s and st["v_zero"][t, h] == z
            assert np.array_equal(st["v_codes"][t, h * GV:(h + 1) * GV], q)
    assert np.array_equal(st["sink_k"], k[:S])
    assert np.array_equal(st["res_v"], v[S + 24:])


@pytest.mark.parametrize("bits,S,codec", [(2, 0, 0), (4, 3, 0), (2, 1, 1), (4, 0, 1), (8, 2, 0), (8, 0, 1)])
def test_matches_pure_python_cache(bits, S, codec):
    D, G, GV, R = 8, 4, 4, 8
    k, v = _tokens(40 + bits, S + 3 * R + 5, D, scale=2.0)
    st = oracle.build_slice(k, v, head_dim=D, bits=bits, k_group=G, v_group=GV,
                            residual=R, n_sink=S, codec=codec)
    br = brute.build_slice(k.tolist(), v.tolist(), bits=bits, k_group=G, v_group=GV,
                           residual=R, n_sink=S, codec=codec)
    K, V = oracle.dequant_slice(st)
    Kb = np.array(br["sinks_k"] + br["qk"] + br["res_k"], np.float32).reshape(-1, D)
    Vb = np.array(br["sinks_v"] + br["qv"] + br["res_v"], np.float32).reshape(-1, D)
    assert np.array_equal(K.view(np.uint32), Kb.view(np.uint32))
    assert np.array_equal(V.view(np.uint32), Vb.view(np.uint32))
    assert np.array_equal(st["k_codes"], np.array(br["k_codes"], np.uint8).reshape(-1, D))
    assert np.array_equal(st["v_codes"], np.array(br["v_codes"], np.uint8).reshape(-1, D))
    assert st["flushes"] == br["flushes"]


def test_workload_schedules_flush_where_expected():
    # tiny workload: 256-token prefill at R=32 leaves r=0; the 32nd decode append
    # flushes once; the run ends at Lq=288, r=8.
    w = wl.get("tiny")
    st0 = oracle.slice_state(w, 0, 0, 0)
    assert (st0["n_quant"], st0["n_resid"], st0["flushes"]) == (256, 0, 8)
    st31 = oracle.slice_state(w, 0, 0, 31)
    st32 = oracle.slice_state(w, 0, 0, 32)
    assert st31["flushes"] == 8 and st32["flushes"] == 9
    st40 = oracle.slice_state(w, 0, 0, 40)
    assert (st40["n_quant"], st40["n_resid"]) == (288, 8)
    # long-context workload: 4 sinks, Lq = 130816 and r = 252 after prefill,
    # flush at the 4th decode append, ending at Lq = 131072, r = 4.
    w5 = wl.get("long_128k_sink_int2")
    S, R = w5.n_sink, w5.residual
    for n_steps, (Lq, r) in {0: (130816, 252), 3: (130816, 255), 4: (131072, 0),
                             8: (131072, 4)}.items():
        N = w5.prefill + n_steps
        assert R * ((N - S) // R) == Lq and (N - S) % R == r


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def test_attention_closed_form_equal_keys_and_zero_query():
    rng = np.random.default_rng(3)
    T, D = 37, 16
    V = rng.standard_normal((T, D)).astype(np.float32)
    K = np.tile(rng.standard_normal((1, D)).astype(np.float32), (T, 1))
    q = rng.standard_normal(D).astype(np.float32)
    o, lse = oracle.attention(q, K, V, 0.25)
    assert np.allclose(o, V.astype(np.float64).mean(0), atol=1e-14)
    s = 0.25 * float(np.dot(q.astype(np.float64), K[0].astype(np.float64)))
    assert abs(lse - (s + np.log(T))) < 1e-12
    K2 = rng.standard_normal((T, D)).astype(np.float32)
    o2, lse2 = oracle.attention(np.zeros(D, np.float32), K2, V, 0.25)
    assert np.allclose(o2, V.astype(np.float64).mean(0), atol=1e-14)
    assert abs(lse2 - np.log(T)) < 1e-12


def test_attention_single_token():
    rng = np.random.default_rng(4)
    K = rng.standard_normal((1, 8)).astype(np.float32)
    V = rng.standard_normal((1, 8)).astype(np.float32)
    o, _ = oracle.attention(rng.standard_normal(8).astype(np.float32), K, V, 1.0)
    assert np.array_equal(o, V[0].astype(np.float64))


def test_attention_permutation_invariant():
    rng = np.random.default_rng(5)
    T, D = 50, 16
    K = (rng.standard_normal((T, D)) * 3).astype(np.float32)
    V = rng.standard_normal((T, D)).astype(np.float32)
    q = rng.standard_normal(D).astype(np.float32)
    o, l = oracle.attention(q, K, V, 0.3)
    p = rng.permutation(T)
    o2, l2 = oracle.attention(q, K[p], V[p], 0.3)
    assert np.allclose(o, o2, atol=1e-13) and abs(l - l2) < 1e-12


def test_attention_matches_torch_sdpa_float64():
    rng = np.random.default_rng(6)
    for T, D in [(1, 8), (9, 16), (100, 64), (300, 128)]:
        K = rng.standard_normal((T, D)).astype(np.float32)
        V = rng.standard_normal((T, D)).astype(np.float32)
        q = (rng.standard_normal(D) * 2).astype(np.float32)
        o, _ = oracle.attention(q, K, V, 1.0 / np.sqrt(D))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q.astype(np.float64))[None, None, None],
            torch.from_numpy(K.astype(np.float64))[None, None],
            torch.from_numpy(V.astype(np.float64))[None, None])[0, 0, 0].numpy()
        assert np.allclose(o, ref, atol=1e-12, rtol=0)


def test_unquantized_cache_is_plain_attention():
    # fewer than R tokens after the sinks: nothing is quantized, attention is exact SDPA
    D = 32
    k, v = _tokens(12, 3 + 20, D)
    st = oracle.build_slice(k, v, head_dim=D, bits=2, k_group=8, v_group=16, residual=32,
                            n_sink=3)
    assert st["n_quant"] == 0
    K, V = oracle.dequant_slice(st)
    assert np.array_equal(K, k) and np.array_equal(V, v)
    q = np.random.default_rng(1).standard_normal(D).astype(np.float32)
    o, _ = oracle.attention(q, K, V, 1 / np.sqrt(D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None, None, None],
        torch.from_numpy(k.astype(np.float64))[None, None],
        torch.from_numpy(v.astype(np.float64))[None, None])[0, 0, 0].numpy()
    assert np.allclose(o, ref, atol=1e-12)


def test_attention_matches_brute_force_loops():
    rng = np.random.default_rng(7)
    for T, D in [(1, 4), (5, 8), (33, 16)]:
        K = (rng.standard_normal((T, D)) * 4).astype(np.float32)
        V = rng.standard_normal((T, D)).astype(np.float32)
        q = rng.standard_normal(D).astype(np.float32)
        o, l = oracle.attention(q, K, V, 0.5)
        ob, lb = brute.attention(q.tolist(), K.tolist(), V.tolist(), 0.5)
        assert np.allclose(o, ob, atol=1e-12) and abs(l - lb) < 1e-12


def test_decode_slices_matches_single_slice_path():
    w = wl.get("tiny").replace(prefill=70, steps=3)
    st = oracle.slice_state(w, 0, 0, 2)
    q = wl.storage_to_f32(wl.query_slice(w, 0, 0)[1], w.dtype)
    K, V = oracle.dequant_slice(st)
    o1, l1 = oracle.attention(q, K, V, oracle.default_scale(w.head_dim))
    o2, l2 = oracle.decode_slices([st, st], np.stack([q[None], q[None]]),
                                  oracle.default_scale(w.head_dim))
    assert np.array_equal(o2[0, 0], o1) and np.array_equal(o2[1, 0], o1)
    assert l2[0, 0] == l1
