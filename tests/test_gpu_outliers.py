"""GPU tests of dense-and-sparse groups (KVQuant), through the C-ABI.

"LLM系列：KVCache量化1 KIVI…" page, section 3 "KVQuant", item (4): per-vector
dense-and-sparse quantization keeps a small share of numeric outliers at full
precision beside the codes.  One outlier per quantization vector (the element of
largest magnitude, the lowest index among equals) is left out of the vector's
scale and zero point and dequantizes to its exact value.  The GPU must match the
oracle slice by slice: codes, scales, zero points, outlier places and values,
and dequantized rows bit-exact; attention within ATOL.
"""
import numpy as np
import pytest
import torch

import bit_quantized_kv_kvq_amd as kvq
import oracle
import workloads as wl
from tests.gpu_common import (ATOL, assert_export_slice_matches, export_cpu, gpu, log, make_cache,
                              require_gpu)
from workloads.torch_io import to_torch

pytestmark = gpu

DEV = torch.device("cuda:0")


def _w(**kw):
    base = wl.get("C2").replace(name="outliers", batch=2, n_kv_heads=2, n_q_heads=2, prefill=0,
                                steps=0, k_group=32, v_group=32, residual=64, outliers=1)
    return base.replace(**kw)


def _tokens(w, n, seed, scale=1.0):
    x = wl.random_tokens(seed, (w.batch, w.n_kv_heads, n, w.head_dim), "f32", scale)
    rng = np.random.default_rng(seed + 7)
    x[rng.random(x.shape) < 0.01] *= 8.0           # sparse large values (the workloads' outlier scale)
    return wl.to_storage(x, w.dtype)


def _state(w, K, V, b, h, n=None):
    kf = wl.storage_to_f32(K[b, h, :n], w.dtype)
    vf = wl.storage_to_f32(V[b, h, :n], w.dtype)
    return oracle.build_slice(kf, vf, head_dim=w.head_dim, bits=w.bits, k_group=w.k_group, v_group=w.v_group,
                              residual=w.residual, n_sink=w.n_sink, codec=w.codec, log_window=w.log_window,
                              outliers=1)


def _check(w, cache, K, V, q, out, lse, lens=None):
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qf = wl.storage_to_f32(q, w.dtype)
    ex = export_cpu(cache)
    eo = {k: v.cpu().numpy() for k, v in cache.export_outliers().items()}
    Kg, Vg = cache.dequantize()
    torch.cuda.synchronize()
    Kg, Vg = Kg.cpu().numpy(), Vg.cpu().numpy()
    scale = oracle.default_scale(w.head_dim)
    err = 0.0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            st = _state(w, K, V, b, h, lens[b] if lens else None)
            assert_export_slice_matches(ex, st, b, h)
            Lq = st["n_quant"]
            np.testing.assert_array_equal(eo["k_idx"][b, h, :Lq // w.k_group], st["ko_idx"])
            np.testing.assert_array_equal(eo["k_val"][b, h, :Lq // w.k_group].view(np.uint32),
                                          st["ko_val"].view(np.uint32))
            np.testing.assert_array_equal(eo["v_idx"][b, h, :Lq], st["vo_idx"])
            np.testing.assert_array_equal(eo["v_val"][b, h, :Lq].view(np.uint32), st["vo_val"].view(np.uint32))
            Kd, Vd = oracle.dequant_slice(st)
            T = len(Kd)
            np.testing.assert_array_equal(Kg[b, h, :T].view(np.uint32), Kd.view(np.uint32))
            np.testing.assert_array_equal(Vg[b, h, :T].view(np.uint32), Vd.view(np.uint32))
            for j in range(w.gqa):
                hq = h * w.gqa + j
                o, l = oracle.attention(qf[b, hq], Kd, Vd, scale)
                err = max(err, float(np.abs(out[b, hq] - o).max()), abs(float(lse[b, hq]) - l))
    assert err <= ATOL, err
    return err


VARIANTS = [
    dict(),                                                       # 4-bit, 32-token groups
    dict(bits=2, n_sink=3),
    dict(k_group=128, v_group=128, residual=128),                 # two 64-token tiles per group
    dict(k_group=256, v_group=64, residual=256),                  # four tiles per group
    dict(k_group=64, v_group=16, residual=64, dtype="f16"),       # 8 value groups per token
    dict(dtype="f32", head_dim=64, v_group=32, bits=2),
    dict(codec=1),
    dict(residual=96, log_window=32),                             # with log-sparse retention
    dict(n_q_heads=4),                                            # 2 query heads per kv head
    dict(n_q_heads=8, k_group=64, v_group=64, residual=128),      # 4, groups of two 32-token tiles
    dict(n_q_heads=16, bits=2, k_group=128, residual=128),        # 8
    # several query heads per kv head with G, G_V >= 64: the matrix cores
    dict(n_q_heads=4, k_group=64, v_group=64, residual=128),              # g = 2
    dict(n_q_heads=8, k_group=128, v_group=128, residual=128),            # g = 4, two tiles per group
    dict(n_q_heads=8, bits=2, k_group=256, v_group=64, residual=256),     # two value groups, four tiles
    dict(n_q_heads=16, bits=2, k_group=64, v_group=64, residual=64, n_sink=2),  # g = 8
]


@pytest.mark.parametrize("kw", VARIANTS)
@pytest.mark.parametrize("n", [1, 63, 64, 65, 300])
def test_bulk_append_against_oracle(kw, n):
    require_gpu()
    w = _w(**kw)
    log("case %s n=%d" % (kw, n))
    cache = make_cache(w, max_tokens=600)
    K, V = _tokens(w, n, 11, 2.0), _tokens(w, n, 12)
    cache.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    q = wl.random_tokens(5, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
    out, lse = cache.decode(to_torch(q, w.dtype, DEV))
    _check(w, cache, K, V, q, out, lse)


@pytest.mark.parametrize("kw", [VARIANTS[0], VARIANTS[2], VARIANTS[13]])
def test_steps_and_ragged_paged(kw):
    require_gpu()
    w = _w(**kw).replace(batch=3)
    log("case %s" % kw)
    lens = [300, 40, 170]
    steps = 140
    n_all = max(lens) + steps
    K, V = _tokens(w, n_all, 21, 2.0), _tokens(w, n_all, 22)
    cache = make_cache(w, max_tokens=n_all, page_groups=2)
    cache.append_ragged(to_torch(np.ascontiguousarray(K[:, :, :max(lens)]), w.dtype, DEV),
                        to_torch(np.ascontiguousarray(V[:, :, :max(lens)]), w.dtype, DEV), lens)
    # step tokens go after each sequence's own prefill: build per-sequence arrays
    Ks = np.zeros_like(K)
    Vs = np.zeros_like(V)
    for b in range(w.batch):
        Ks[b, :, :lens[b]], Vs[b, :, :lens[b]] = K[b, :, :lens[b]], V[b, :, :lens[b]]
    worst = 0.0
    for s in range(steps):
        k1, v1 = _tokens(w, 1, 1000 + s), _tokens(w, 1, 2000 + s)
        q = wl.random_tokens(3000 + s, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
        out, lse = cache.append_decode(*(to_torch(x, w.dtype, DEV) for x in (k1, v1, q)))
        cur = [n + s + 1 for n in lens]
        for b in range(w.batch):
            Ks[b, :, cur[b] - 1], Vs[b, :, cur[b] - 1] = k1[b, :, 0], v1[b, :, 0]
        if s % 23 == 0 or s == steps - 1:
            worst = max(worst, _check(w, cache, Ks, Vs, q, out, lse, cur))
    log("  max |out - oracle| = %.3g" % worst)


def test_adversarial_groups():
    """Ties in magnitude everywhere, equal magnitudes of opposite sign, constant
    groups, a channel and a token far above the rest, tiny keys.  Magnitudes stay
    within a few tens of the typical entry: the key fold is fixed point relative
    to the largest |q_c s_c| of a group, and the tolerance is absolute."""
    require_gpu()
    w = _w(batch=1, n_kv_heads=4, n_q_heads=4)
    n = 64
    rng = np.random.default_rng(3)
    K = np.zeros((1, 4, n, w.head_dim), np.float32)
    V = np.zeros_like(K)
    K[0, 0] = 2.0                                         # constant: every magnitude ties
    V[0, 0] = -1.5
    K[0, 1] = np.round(rng.standard_normal((n, w.head_dim)) * 2)   # many ties in magnitude
    V[0, 1] = np.round(rng.standard_normal((n, w.head_dim)) * 2)
    K[0, 1, 5] = -(np.abs(K[0, 1]).max() + 3.0)           # equal magnitudes of opposite sign
    K[0, 1, 9] = -K[0, 1, 5]
    V[0, 1, :, 3] = 9.0
    V[0, 1, :, 4] = -9.0
    K[0, 2] = rng.standard_normal((n, w.head_dim)) * 1e-3   # tiny keys
    V[0, 2] = rng.standard_normal((n, w.head_dim))
    K[0, 3] = rng.standard_normal((n, w.head_dim))
    K[0, 3, :, 7] = 6.0                                    # a whole channel at one larger value
    V[0, 3] = rng.standard_normal((n, w.head_dim))
    V[0, 3, 17] = 8.0                                      # a whole token at one larger value
    Ks, Vs = wl.to_storage(K, w.dtype), wl.to_storage(V, w.dtype)
    cache = make_cache(w, max_tokens=n)
    cache.append(to_torch(Ks, w.dtype, DEV), to_torch(Vs, w.dtype, DEV))
    q = wl.random_tokens(8, (1, 4, w.head_dim), w.dtype)
    out, lse = cache.decode(to_torch(q, w.dtype, DEV))
    torch.cuda.synchronize()
    o_cpu, l_cpu = out.cpu().numpy(), lse.cpu().numpy()
    qf = wl.storage_to_f32(q, w.dtype)
    for h in range(4):  # per-head errors, for the log
        Kd, Vd = oracle.dequant_slice(_state(w, Ks, Vs, 0, h))
        eo, el = oracle.attention(qf[0, h], Kd, Vd, oracle.default_scale(w.head_dim))
        log("  head %d: max |out - oracle| = %.3g" % (h, float(np.abs(o_cpu[0, h] - eo).max())))
    _check(w, cache, Ks, Vs, q, out, lse)


@pytest.mark.parametrize("kw", [VARIANTS[0], VARIANTS[2], VARIANTS[9], VARIANTS[12]])
def test_repeat_calls_are_bitwise_deterministic(kw):
    """The outlier terms meet through LDS atomic adds; repeated calls must still agree bit for bit."""
    require_gpu()
    w = _w(**kw)
    cache = make_cache(w, max_tokens=400)
    K, V = _tokens(w, 333, 61, 2.0), _tokens(w, 333, 62)
    cache.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    q = to_torch(wl.random_tokens(63, (w.batch, w.n_q_heads, w.head_dim), w.dtype), w.dtype, DEV)
    o0, l0 = cache.decode(q)
    torch.cuda.synchronize()
    o0, l0 = o0.clone(), l0.clone()
    for _ in range(20):
        o, l = cache.decode(q)
        torch.cuda.synchronize()
        assert torch.equal(o, o0) and torch.equal(l, l0)


def test_outlier_export_needs_outliers():
    require_gpu()
    cache = make_cache(_w(outliers=0), max_tokens=64)
    with pytest.raises(kvq.KVQError) as ei:
        cache.export_outliers()
    assert ei.value.status == kvq.KVQ_ERR_INVALID_ARG
