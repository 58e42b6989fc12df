"""GPU tests of LogQuant's log-sparse retention, through the C-ABI.

"Resumo Técnico: LogQuant", Metodologia item 2: the residual holds R = 3W
full-precision tokens; a flush quantizes the earlier token of each pair among
the oldest 2W and keeps the later ones and the newest W.  The GPU must match the
oracle slice by slice: codes, scales and zero points bit-exact, dequantized rows
(sinks, quantized tokens in the order they were quantized, then the residual)
bit-exact, attention within ATOL, across flushes, on both decode streams.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_common import (ATOL, assert_export_slice_matches, export_cpu, gpu, log, make_cache,
                              require_gpu)
from workloads.torch_io import to_torch

pytestmark = gpu

DEV = torch.device("cuda:0")


def _w(**kw):
    base = wl.get("C2").replace(name="logquant", batch=2, n_kv_heads=2, n_q_heads=2, prefill=0,
                                steps=0, k_group=32, v_group=32, residual=96, log_window=32)
    return base.replace(**kw)


def _tokens(w, n, seed, scale=1.0):
    return wl.random_tokens(seed, (w.batch, w.n_kv_heads, n, w.head_dim), w.dtype, scale)


def _state(w, kf, vf):
    return oracle.build_slice(kf, vf, head_dim=w.head_dim, bits=w.bits, k_group=w.k_group,
                              v_group=w.v_group, residual=w.residual, n_sink=w.n_sink,
                              codec=w.codec, log_window=w.log_window)


def _states(w, K, V, lens=None):
    kf, vf = wl.storage_to_f32(K, w.dtype), wl.storage_to_f32(V, w.dtype)
    return {(b, h): _state(w, kf[b, h, :(lens[b] if lens else None)], vf[b, h, :(lens[b] if lens else None)])
            for b in range(w.batch) for h in range(w.n_kv_heads)}


def _check(w, cache, sts, q, out, lse):
    """Attention within ATOL; export and dequantized rows bit-exact, per slice."""
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qf = wl.storage_to_f32(q, w.dtype)
    scale = oracle.default_scale(w.head_dim)
    ex = export_cpu(cache)
    Kg, Vg = cache.dequantize()
    torch.cuda.synchronize()
    Kg, Vg = Kg.cpu().numpy(), Vg.cpu().numpy()
    err = 0.0
    for (b, h), st in sts.items():
        assert_export_slice_matches(ex, st, b, h)
        Kd, Vd = oracle.dequant_slice(st)
        T = len(Kd)
        np.testing.assert_array_equal(Kg[b, h, :T].view(np.uint32), Kd.view(np.uint32))
        np.testing.assert_array_equal(Vg[b, h, :T].view(np.uint32), Vd.view(np.uint32))
        for j in range(w.gqa):
            hq = h * w.gqa + j
            eo, el = oracle.attention(qf[b, hq], Kd, Vd, scale)
            err = max(err, float(np.abs(out[b, hq] - eo).max()), abs(float(lse[b, hq]) - el))
    assert err <= ATOL, err
    return err


VARIANTS = [
    dict(),                                                                  # VALU stream, W = G = 32
    dict(bits=2, n_sink=3),
    dict(k_group=32, residual=192, log_window=64, n_q_heads=4),              # W = 2G, GQA 2
    dict(n_q_heads=8, bits=2, k_group=64, v_group=64, residual=192, log_window=64),  # matrix cores
    dict(bits=8, k_group=64, v_group=64, residual=192, log_window=64, codec=1),     # 8-bit
    dict(dtype="f32", head_dim=64, v_group=16, n_sink=2),
]


@pytest.mark.parametrize("kw", VARIANTS)
@pytest.mark.parametrize("n", [1, 95, 96, 97, 250, 333])
def test_bulk_append_against_oracle(kw, n):
    require_gpu()
    w = _w(**kw)
    log("case %s n=%d" % (kw, n))
    cache = make_cache(w, max_tokens=400)
    K, V = _tokens(w, n, 11, 2.0), _tokens(w, n, 12)
    cache.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    sts = _states(w, K, V)
    st0 = sts[(0, 0)]
    assert cache.state() == (n, st0["n_sink"], st0["n_quant"], st0["n_resid"])
    q = wl.random_tokens(5, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
    out, lse = cache.decode(to_torch(q, w.dtype, DEV))
    _check(w, cache, sts, q, out, lse)


@pytest.mark.parametrize("kw", [VARIANTS[0], VARIANTS[3]])
def test_steps_across_flushes_with_one_launch_step(kw):
    require_gpu()
    w = _w(**kw)
    log("case %s" % kw)
    n0, steps = 150, 3 * w.log_window + 5
    cache = make_cache(w, max_tokens=n0 + steps)
    K, V = _tokens(w, n0 + steps, 31, 2.0), _tokens(w, n0 + steps, 32)
    cache.append(to_torch(np.ascontiguousarray(K[:, :, :n0]), w.dtype, DEV),
                 to_torch(np.ascontiguousarray(V[:, :, :n0]), w.dtype, DEV))
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.batch, w.n_q_heads), dtype=torch.float32, device=DEV)
    worst = 0.0
    for s in range(steps):
        t = n0 + s
        kt = to_torch(np.ascontiguousarray(K[:, :, t:t + 1]), w.dtype, DEV)
        vt = to_torch(np.ascontiguousarray(V[:, :, t:t + 1]), w.dtype, DEV)
        q = wl.random_tokens(100 + s, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
        cache.append_decode(kt, vt, to_torch(q, w.dtype, DEV), out=out, lse=lse)
        if s % 11 == 0 or s == steps - 1:
            worst = max(worst, _check(w, cache, _states(w, K[:, :, :t + 1], V[:, :, :t + 1]), q, out, lse))
    log("  max |out - oracle| = %.3g" % worst)


def test_chunked_appends_equal_bulk_append():
    require_gpu()
    w = _w(n_sink=2, bits=2)
    n = 7 * 32 + 19
    K, V = _tokens(w, n, 21, 3.0), _tokens(w, n, 22)
    a = make_cache(w, max_tokens=n)
    a.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    b = make_cache(w, max_tokens=n)
    i, j, sizes = 0, 0, [1, 5, 1, 70, 2, 64, 1, 100]
    while i < n:
        m = min(sizes[j % len(sizes)], n - i)
        b.append(to_torch(np.ascontiguousarray(K[:, :, i:i + m]), w.dtype, DEV),
                 to_torch(np.ascontiguousarray(V[:, :, i:i + m]), w.dtype, DEV))
        i, j = i + m, j + 1
    assert a.state() == b.state()
    ea, eb = export_cpu(a), export_cpu(b)
    for k in ea:
        np.testing.assert_array_equal(ea[k], eb[k])
    ka, va = a.dequantize()
    kb, vb = b.dequantize()
    assert torch.equal(ka, kb) and torch.equal(va, vb)


@pytest.mark.parametrize("kw", [VARIANTS[1], VARIANTS[3]])
def test_ragged_lengths_across_flushes(kw):
    require_gpu()
    w = _w(**kw).replace(batch=4)
    log("case %s" % kw)
    lens = [200, 3, 96, 130]
    steps = 70
    n_all = max(lens) + steps
    K, V = _tokens(w, n_all, 41, 2.0), _tokens(w, n_all, 42)
    cache = make_cache(w, max_tokens=n_all)
    cache.append_ragged(to_torch(np.ascontiguousarray(K[:, :, :max(lens)]), w.dtype, DEV),
                        to_torch(np.ascontiguousarray(V[:, :, :max(lens)]), w.dtype, DEV), lens)
    # host copy of every sequence's tokens so far
    Ks = [[K[b, :, :lens[b]]] for b in range(w.batch)]
    Vs = [[V[b, :, :lens[b]]] for b in range(w.batch)]
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.batch, w.n_q_heads), dtype=torch.float32, device=DEV)
    for s in range(steps):
        k1, v1 = _tokens(w, 1, 1000 + s), _tokens(w, 1, 2000 + s)
        q = wl.random_tokens(3000 + s, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
        cache.append_decode(*(to_torch(x, w.dtype, DEV) for x in (k1, v1, q)), out=out, lse=lse)
        for b in range(w.batch):
            Ks[b].append(k1[b])
            Vs[b].append(v1[b])
        if s % 9 == 0 or s == steps - 1:
            cur = [np.concatenate(Ks[b], axis=1) for b in range(w.batch)]
            cvv = [np.concatenate(Vs[b], axis=1) for b in range(w.batch)]
            L = [c.shape[1] for c in cur]
            assert cache.seq_lengths() == L
            Kp = np.zeros((w.batch, w.n_kv_heads, max(L), w.head_dim), K.dtype)
            Vp = np.zeros_like(Kp)
            for b in range(w.batch):
                Kp[b, :, :L[b]], Vp[b, :, :L[b]] = cur[b], cvv[b]
            _check(w, cache, _states(w, Kp, Vp, L), q, out, lse)
