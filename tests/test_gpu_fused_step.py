"""GPU tests of kvq_append_decode: one call per decode step (append one token per
sequence, then attention) must give exactly the outputs and cache state of
kvq_append followed by kvq_decode_attention, across the sink, residual and flush
phases of a sequence, and match the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_common import ATOL, export_cpu, gpu, log, make_cache, require_gpu
from workloads.torch_io import to_torch

pytestmark = gpu

DEV = torch.device("cuda:0")


def _w(**kw):
    base = wl.get("C2").replace(name="fused", batch=2, n_kv_heads=2, n_q_heads=2, prefill=0,
                                steps=0, k_group=32, v_group=32, residual=64)
    return base.replace(**kw)


@pytest.mark.parametrize("kw,prefill", [
    (dict(n_sink=3), 0),                                        # sinks, residual, two flushes
    (dict(bits=2, n_q_heads=8, k_group=64, residual=128, v_group=64), 300),  # GQA 4, INT2
    (dict(dtype="f32", head_dim=64, v_group=16, n_q_heads=4), 40),           # f32, D64, GQA 2
    (dict(k_group=128, residual=128, v_group=128), 500),        # 64-token tiles
])
def test_fused_step_equals_two_calls(kw, prefill):
    require_gpu()
    w = _w(**kw)
    steps = 150
    n = prefill + steps
    log("case %s prefill %d steps %d" % (kw, prefill, steps))
    K, V = (wl.random_tokens(31, (w.batch, w.n_kv_heads, n, w.head_dim), w.dtype, 2.0),
            wl.random_tokens(32, (w.batch, w.n_kv_heads, n, w.head_dim), w.dtype))
    Q = wl.random_tokens(33, (steps, w.batch, w.n_q_heads, w.head_dim), w.dtype)
    Kd, Vd, Qd = to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV), to_torch(Q, w.dtype, DEV)
    a, b = make_cache(w, max_tokens=n), make_cache(w, max_tokens=n)
    if prefill:
        a.append(Kd[:, :, :prefill].contiguous(), Vd[:, :, :prefill].contiguous())
        b.append(Kd[:, :, :prefill].contiguous(), Vd[:, :, :prefill].contiguous())
    scale = oracle.default_scale(w.head_dim)
    kf, vf = wl.storage_to_f32(K, w.dtype), wl.storage_to_f32(V, w.dtype)
    worst = 0.0
    for s in range(steps):
        t = prefill + s
        kt, vt = Kd[:, :, t:t + 1].contiguous(), Vd[:, :, t:t + 1].contiguous()
        oa, la = a.append_decode(kt, vt, Qd[s])
        b.append(kt, vt)
        ob, lb = b.decode(Qd[s])
        torch.cuda.synchronize()
        assert a.state() == b.state()
        assert torch.equal(oa, ob) and torch.equal(la, lb), s
        if s % 37 == 0 or s == steps - 1:   # against the oracle now and then
            o, l = oa.cpu().numpy(), la.cpu().numpy()
            qf = wl.storage_to_f32(Q[s], w.dtype)
            for bb in range(w.batch):
                for h in range(w.n_kv_heads):
                    st = oracle.build_slice(kf[bb, h, :t + 1], vf[bb, h, :t + 1], head_dim=w.head_dim,
                                            bits=w.bits, k_group=w.k_group, v_group=w.v_group,
                                            residual=w.residual, n_sink=w.n_sink)
                    Kq, Vq = oracle.dequant_slice(st)
                    for j in range(w.gqa):
                        hq = h * w.gqa + j
                        eo, el = oracle.attention(qf[bb, hq], Kq, Vq, scale)
                        worst = max(worst, float(np.abs(o[bb, hq] - eo).max()), abs(float(l[bb, hq]) - el))
    assert worst <= ATOL, worst
    ea, eb = export_cpu(a), export_cpu(b)
    for k in ea:
        np.testing.assert_array_equal(ea[k], eb[k])
    ka, va = a.dequantize()
    kb, vb = b.dequantize()
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    log("  max |out - oracle| = %.3g, final state %s" % (worst, a.state()))


def test_fused_step_validates_before_enqueueing():
    require_gpu()
    import bit_quantized_kv_kvq_amd as kvq
    w = _w()
    c = make_cache(w, max_tokens=65)
    K = to_torch(wl.random_tokens(41, (w.batch, w.n_kv_heads, 65, w.head_dim), w.dtype), w.dtype, DEV)
    q = to_torch(wl.random_tokens(42, (w.batch, w.n_q_heads, w.head_dim), w.dtype), w.dtype, DEV)
    c.append(K[:, :, :64].contiguous(), K[:, :, :64].contiguous())
    before = c.state()
    with pytest.raises(kvq.KVQError) as ei:   # workspace too small
        kvq.kvq_append_decode(c.handle, K[:, :, 64:65].contiguous().data_ptr(),
                              K[:, :, 64:65].contiguous().data_ptr(), q.data_ptr(),
                              torch.empty((w.batch, w.n_q_heads, w.head_dim), device=DEV).data_ptr(),
                              0, c._ws_ptr, 16, torch.cuda.current_stream().cuda_stream)
    assert ei.value.status == kvq.KVQ_ERR_BUFFER_TOO_SMALL
    assert c.state() == before
    c.append_decode(K[:, :, 64:65].contiguous(), K[:, :, 64:65].contiguous(), q)
    with pytest.raises(kvq.KVQError) as ei:   # capacity
        c.append_decode(K[:, :, 64:65].contiguous(), K[:, :, 64:65].contiguous(), q)
    assert ei.value.status == kvq.KVQ_ERR_CAPACITY


def test_fused_step_validates_before_a_flush_step():
    """A step whose token fills the residual takes the two-call path (append, flush,
    decode); a workspace or alignment error must still leave the cache unchanged, so
    that a caller who fixes the arguments and retries appends the token once."""
    require_gpu()
    import bit_quantized_kv_kvq_amd as kvq
    w = _w()
    R = w.residual
    c = make_cache(w, max_tokens=3 * R)
    K = to_torch(wl.random_tokens(43, (w.batch, w.n_kv_heads, 2 * R, w.head_dim), w.dtype), w.dtype, DEV)
    q = to_torch(wl.random_tokens(44, (w.batch, w.n_q_heads, w.head_dim), w.dtype), w.dtype, DEV)
    c.append(K[:, :, :2 * R - 1].contiguous(), K[:, :, :2 * R - 1].contiguous())
    before = c.state()
    assert before[3] == R - 1   # the next token fills the residual
    kt = K[:, :, 2 * R - 1:2 * R].contiguous()
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    with pytest.raises(kvq.KVQError) as ei:   # workspace too small
        kvq.kvq_append_decode(c.handle, kt.data_ptr(), kt.data_ptr(), q.data_ptr(), out.data_ptr(), 0,
                              c._ws_ptr, 16, s)
    assert ei.value.status == kvq.KVQ_ERR_BUFFER_TOO_SMALL
    assert c.state() == before
    with pytest.raises(kvq.KVQError) as ei:   # misaligned output
        kvq.kvq_append_decode(c.handle, kt.data_ptr(), kt.data_ptr(), q.data_ptr(), out.data_ptr() + 2, 0,
                              c._ws_ptr, c.ws_bytes, s)
    assert ei.value.status == kvq.KVQ_ERR_INVALID_ARG
    assert c.state() == before
    o1, _ = c.append_decode(kt, kt, q)   # the retry flushes once
    torch.cuda.synchronize()
    assert c.state() == (before[0] + 1, 0, before[2] + R, 0)


@pytest.mark.parametrize("kw", [dict(n_sink=3), dict(bits=2, n_q_heads=8, k_group=64, residual=128, v_group=64),
                                dict(residual=96, log_window=32), dict(outliers=1)])
def test_fused_step_on_sequences_of_different_lengths(kw):
    """Sequences of different lengths: the one-launch step (each token at its own
    sequence's residual row) equals the two calls bit for bit, and steps in which
    some sequence takes a sink or flushes fall back to them."""
    require_gpu()
    w = _w(**kw).replace(batch=4)
    lens = [150, 2, 64, 97]
    steps = 140
    n = max(lens) + steps
    log("case %s lens %s" % (kw, lens))
    K = wl.random_tokens(41, (w.batch, w.n_kv_heads, max(lens), w.head_dim), w.dtype, 2.0)
    V = wl.random_tokens(42, (w.batch, w.n_kv_heads, max(lens), w.head_dim), w.dtype)
    Kd, Vd = to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV)
    a, b = make_cache(w, max_tokens=n, page_groups=2), make_cache(w, max_tokens=n)
    a.append_ragged(Kd, Vd, lens)
    b.append_ragged(Kd, Vd, lens)
    for s in range(steps):
        k1 = to_torch(wl.random_tokens(1000 + s, (w.batch, w.n_kv_heads, 1, w.head_dim), w.dtype), w.dtype, DEV)
        v1 = to_torch(wl.random_tokens(2000 + s, (w.batch, w.n_kv_heads, 1, w.head_dim), w.dtype), w.dtype, DEV)
        q = to_torch(wl.random_tokens(3000 + s, (w.batch, w.n_q_heads, w.head_dim), w.dtype), w.dtype, DEV)
        oa, la = a.append_decode(k1, v1, q)
        b.append(k1, v1)
        ob, lb = b.decode(q)
        torch.cuda.synchronize()
        assert a.seq_lengths() == b.seq_lengths() and a.state() == b.state()
        assert torch.equal(oa, ob) and torch.equal(la, lb), s
    ea, eb = export_cpu(a), export_cpu(b)
    for name in ea:
        np.testing.assert_array_equal(ea[name], eb[name], err_msg=name)
    ka, va = a.dequantize()
    kb, vb = b.dequantize()
    assert torch.equal(ka, kb) and torch.equal(va, vb)
