"""GPU tests of head-granular keys (key_axis = KVQ_KEY_PER_TOKEN; "Atom: Low-bit
Quantization for Efficient and Accurate LLM Serving" review, section 三,
model-components table, KV-cache row: asymmetric low-bit KV at attention-head
granularity): each token's key is one group over its head_dim channels.

Against the oracle: codes, per-token key scales and zero points, value metadata
and dequantized rows bit-exact; attention within 1e-3.  Both decode streams (the
VALU stream for one query head per kv head, the matrix cores for several and for
8-bit codes), both codecs, every storage dtype, sinks, the one-launch step, paged
records, log-sparse retention and sequences of different lengths; shapes without
a kernel are refused at creation."""
import numpy as np
import pytest
import torch

import bit_quantized_kv_kvq_amd as kvq
import oracle
import workloads as wl
from tests.gpu_common import ATOL, assert_export_slice_matches, export_cpu, gpu, log, make_cache, require_gpu
from tests.test_gpu_boundary import _attend_and_check, _oracle_states, _tokens
from workloads.torch_io import to_torch

pytestmark = gpu

DEV = torch.device("cuda:0")


def _w(**kw):
    base = wl.get("C2").replace(name="keys", batch=2, n_kv_heads=2, n_q_heads=2, prefill=0, steps=0,
                                k_group=128, v_group=128, residual=128, key_axis=1)
    return base.replace(**kw)


@pytest.mark.parametrize("kw", [
    dict(),                                                   # VALU stream, INT4, two tiles per record
    dict(bits=2),
    dict(k_group=64, residual=128),                           # one tile per record
    dict(v_group=32),                                         # four value groups per token
    dict(v_group=16),                                         # eight value groups (16 key channels per lane)
    dict(dtype="f32", head_dim=64, v_group=64, k_group=64, residual=64),
    dict(dtype="f16", codec=1),                               # symmetric groups
    dict(n_q_heads=8),                                        # matrix cores, g = 4
    dict(n_q_heads=4, bits=2, v_group=64, k_group=64),        # g = 2, two value groups, two waves
    dict(n_q_heads=16, bits=2),                               # g = 8
    dict(bits=8),                                             # 8-bit codes, one query head per kv head
    dict(bits=8, n_q_heads=8, codec=1, head_dim=64, v_group=64, dtype="f32"),
    dict(n_sink=3),
    dict(n_sink=2, n_q_heads=8, bits=2, v_group=64),
])
@pytest.mark.parametrize("n", [1, 127, 128, 129, 700])
def test_per_token_keys_against_oracle(kw, n):
    require_gpu()
    w = _w(**kw)
    log("case %s n=%d" % (kw, n))
    cache = make_cache(w, max_tokens=800)
    K, V = _tokens(w, n, 11, 2.0), _tokens(w, n, 12)
    # a few keys with channel outliers and constant rows
    if n > 5:
        K[:, :, 5] = K[:, :, 5, :1]
    cache.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    sts, err = _attend_and_check(w, cache, K, V)
    ex = export_cpu(cache)
    for (b, h), st in sts.items():
        assert_export_slice_matches(ex, st, b, h)
    Kd, Vd = cache.dequantize()
    torch.cuda.synchronize()
    Kd, Vd = Kd.cpu().numpy(), Vd.cpu().numpy()
    for (b, h), st in sts.items():
        Ko, Vo = oracle.dequant_slice(st)
        np.testing.assert_array_equal(Kd[b, h].view(np.uint32), Ko.view(np.uint32))
        np.testing.assert_array_equal(Vd[b, h].view(np.uint32), Vo.view(np.uint32))


def _kv_steps(w, steps, seed):
    ks = [to_torch(wl.random_tokens(seed + s, (w.batch, w.n_kv_heads, 1, w.head_dim), w.dtype, 2.0), w.dtype, DEV)
          for s in range(steps)]
    vs = [to_torch(wl.random_tokens(seed + 5000 + s, (w.batch, w.n_kv_heads, 1, w.head_dim), w.dtype), w.dtype, DEV)
          for s in range(steps)]
    qs = [to_torch(wl.random_tokens(seed + 9000 + s, (w.batch, w.n_q_heads, w.head_dim), w.dtype), w.dtype, DEV)
          for s in range(steps)]
    return ks, vs, qs


@pytest.mark.parametrize("kw,cache_kw", [
    (dict(), {}),
    (dict(n_q_heads=8, bits=2, v_group=64, k_group=64), {}),
    (dict(k_group=64, residual=192, log_window=64), {}),               # log-sparse retention
    (dict(n_sink=2), dict(page_groups=2)),                             # paged records
])
def test_per_token_keys_one_launch_steps(kw, cache_kw):
    """The one-launch step equals append then decode bit for bit across flushes, and
    matches the oracle built from the same tokens."""
    require_gpu()
    w = _w(**kw)
    prefill, steps = 300, 150
    n = prefill + steps
    log("case %s %s" % (kw, cache_kw))
    K0, V0 = _tokens(w, prefill, 31, 2.0), _tokens(w, prefill, 32)
    a = make_cache(w, max_tokens=n, **cache_kw)
    b = make_cache(w, max_tokens=n)
    for c in (a, b):
        c.append(to_torch(K0, w.dtype, DEV), to_torch(V0, w.dtype, DEV))
    ks, vs, qs = _kv_steps(w, steps, 100)
    for s in range(steps):
        oa, la = a.append_decode(ks[s], vs[s], qs[s])
        b.append(ks[s], vs[s])
        ob, lb = b.decode(qs[s])
        torch.cuda.synchronize()
        assert a.state() == b.state()
        assert torch.equal(oa, ob) and torch.equal(la, lb), s
    kf = np.concatenate([wl.storage_to_f32(K0, w.dtype)] +
                        [wl.storage_to_f32(_host(x, w), w.dtype) for x in ks], 2)
    vf = np.concatenate([wl.storage_to_f32(V0, w.dtype)] +
                        [wl.storage_to_f32(_host(x, w), w.dtype) for x in vs], 2)
    q = wl.storage_to_f32(_host(qs[-1], w), w.dtype)
    o, l = oa.cpu().numpy(), la.cpu().numpy()
    ex = export_cpu(a)
    scale = oracle.default_scale(w.head_dim)
    for bb in range(w.batch):
        for h in range(w.n_kv_heads):
            st = oracle.build_slice(kf[bb, h], vf[bb, h], head_dim=w.head_dim, bits=w.bits, k_group=w.k_group,
                                    v_group=w.v_group, residual=w.residual, n_sink=w.n_sink, codec=w.codec,
                                    log_window=w.log_window, key_axis=1)
            assert_export_slice_matches(ex, st, bb, h)
            Kq, Vq = oracle.dequant_slice(st)
            for j in range(w.gqa):
                hq = h * w.gqa + j
                eo, el = oracle.attention(q[bb, hq], Kq, Vq, scale)
                assert np.abs(o[bb, hq] - eo).max() <= ATOL and abs(float(l[bb, hq]) - el) <= ATOL


def _host(x, w):
    """Storage array of a device tensor (bf16 as its uint16 bits)."""
    t = x.cpu()
    if w.dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def test_per_token_keys_ragged_lengths():
    require_gpu()
    w = _w(batch=4, n_q_heads=8, bits=2, v_group=64, k_group=64)
    lens = [300, 5, 128, 200]
    K, V = _tokens(w, max(lens), 41, 2.0), _tokens(w, max(lens), 42)
    c = make_cache(w, max_tokens=400)
    c.append_ragged(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV), lens)
    q = wl.random_tokens(43, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
    out, lse = c.decode(to_torch(q, w.dtype, DEV))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    kf, vf, qf = (wl.storage_to_f32(x, w.dtype) for x in (K, V, q))
    ex = export_cpu(c)
    for b, n in enumerate(lens):
        for h in range(w.n_kv_heads):
            st = oracle.build_slice(kf[b, h, :n], vf[b, h, :n], head_dim=w.head_dim, bits=w.bits,
                                    k_group=w.k_group, v_group=w.v_group, residual=w.residual, n_sink=0,
                                    key_axis=1)
            assert_export_slice_matches(ex, st, b, h)
            Kq, Vq = oracle.dequant_slice(st)
            for j in range(w.gqa):
                eo, _ = oracle.attention(qf[b, h * w.gqa + j], Kq, Vq, oracle.default_scale(w.head_dim))
                assert np.abs(out[b, h * w.gqa + j] - eo).max() <= ATOL


@pytest.mark.parametrize("kw,status", [
    (dict(k_group=32, residual=64), kvq.KVQ_ERR_UNSUPPORTED),          # records of 32 tokens
    (dict(k_group=256, residual=256), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(outliers=1), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(n_q_heads=8, v_group=32), kvq.KVQ_ERR_UNSUPPORTED),          # several heads, G_V < 64
    (dict(key_axis=2), kvq.KVQ_ERR_INVALID_ARG),
])
def test_per_token_keys_refused_shapes(kw, status):
    require_gpu()
    w = _w(**kw)
    with pytest.raises(kvq.KVQError) as ei:
        make_cache(w, max_tokens=256)
    assert ei.value.status == status
