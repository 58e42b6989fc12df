"""GPU tests of the boundary's semantics and edge cases, through the C-ABI."""
import numpy as np
import pytest
import torch

import bit_quantized_kv_kvq_amd as kvq
import oracle
import workloads as wl
from tests.gpu_common import (ATOL, assert_export_slice_matches, export_cpu, gpu, log,
                              make_cache, require_gpu)
from workloads.torch_io import TORCH_DTYPES, to_torch

pytestmark = gpu

DEV = torch.device("cuda:0")


def _w(**kw):
    base = wl.get("C2").replace(name="edge", batch=2, n_kv_heads=2, n_q_heads=2, prefill=0,
                                steps=0, k_group=32, v_group=32, residual=64)
    return base.replace(**kw)


def _tokens(w, n, seed, scale=1.0, offset=0.0):
    x = wl.random_tokens(seed, (w.batch, w.n_kv_heads, n, w.head_dim), w.dtype, scale, offset)
    return x


def _oracle_states(w, K, V):
    """Oracle states of every slice for host storage arrays K, V [B, Hkv, n, D]."""
    kf = wl.storage_to_f32(K, w.dtype)
    vf = wl.storage_to_f32(V, w.dtype)
    return {(b, h): oracle.build_slice(kf[b, h], vf[b, h], head_dim=w.head_dim, bits=w.bits,
                                       k_group=w.k_group, v_group=w.v_group,
                                       residual=w.residual, n_sink=w.n_sink, codec=w.codec,
                                       outliers=w.outliers, key_axis=w.key_axis)
            for b in range(w.batch) for h in range(w.n_kv_heads)}


def _attend_and_check(w, cache, K, V, seed=5):
    q = wl.random_tokens(seed, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
    out, lse = cache.decode(to_torch(q, w.dtype, DEV))
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    sts = _oracle_states(w, K, V)
    qf = wl.storage_to_f32(q, w.dtype)
    scale = oracle.default_scale(w.head_dim)
    err = 0.0
    for (b, h), st in sts.items():
        Kd, Vd = oracle.dequant_slice(st)
        for j in range(w.gqa):
            hq = h * w.gqa + j
            eo, el = oracle.attention(qf[b, hq], Kd, Vd, scale)
            err = max(err, float(np.abs(out[b, hq] - eo).max()), abs(float(lse[b, hq]) - el))
    assert err <= ATOL, err
    return sts, err


@pytest.mark.parametrize("kw", [
    dict(),                                             # bf16 MHA INT4
    dict(bits=2),
    dict(dtype="f16"),
    dict(dtype="f32", head_dim=64, v_group=16),
    dict(n_q_heads=4),                                  # GQA 2
    dict(n_q_heads=16, bits=2),                         # GQA 8
    dict(n_q_heads=16, bits=4, head_dim=64),            # GQA 8, D64
    dict(n_q_heads=16, bits=4),                         # GQA 8, D128: 8 channels per lane, 8 tokens per slot
    dict(v_group=16, k_group=64, residual=128),         # 16-channel value groups: 8 tokens per slot
    dict(v_group=16, k_group=64, residual=128, bits=2),
    dict(n_sink=3),
    dict(k_group=64, residual=128, v_group=128),        # 64-token tiles, one per group
    dict(k_group=128, residual=128, v_group=64),        # two tiles per group
    dict(n_q_heads=8, k_group=128, residual=128),       # GQA 4, four tiles per group
    dict(n_q_heads=8, bits=2, k_group=64, residual=128, v_group=64),  # GQA 4, two per group
    dict(codec=1),                                      # symmetric groups
    dict(codec=1, bits=2, n_sink=3, dtype="f32", head_dim=64, v_group=16),
    dict(codec=1, n_q_heads=8, k_group=64, residual=128, v_group=64),  # symmetric, matrix cores
    dict(bits=8, k_group=64, residual=128, v_group=64),                # 8-bit, one head per kv head
    dict(bits=8, n_q_heads=8, k_group=128, residual=128, v_group=128, n_sink=3),  # 8-bit GQA 4
    dict(bits=8, codec=1, head_dim=64, dtype="f32", k_group=64, residual=64, v_group=64),
])
@pytest.mark.parametrize("n", [1, 63, 64, 65, 200])
def test_variants_against_oracle(kw, n):
    require_gpu()
    w = _w(**kw)
    log("case %s n=%d" % (kw, n))
    cache = make_cache(w, max_tokens=256)
    K, V = _tokens(w, n, 11, 2.0), _tokens(w, n, 12)
    cache.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    sts, err = _attend_and_check(w, cache, K, V)
    ex = export_cpu(cache)
    for (b, h), st in sts.items():
        assert_export_slice_matches(ex, st, b, h)


@pytest.mark.parametrize("kw", [
    dict(k_group=256, residual=256, v_group=128),                # 64-token tiles, four per group
    dict(k_group=256, residual=256, n_q_heads=4, bits=2),        # GQA 2, eight 32-token tiles
])
@pytest.mark.parametrize("n", [600, 1100])
def test_long_groups_against_oracle(kw, n):
    require_gpu()
    w = _w(**kw)
    log("case %s n=%d" % (kw, n))
    cache = make_cache(w, max_tokens=1200)
    K, V = _tokens(w, n, 21, 2.0), _tokens(w, n, 22)
    cache.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    sts, err = _attend_and_check(w, cache, K, V)
    ex = export_cpu(cache)
    for (b, h), st in sts.items():
        assert_export_slice_matches(ex, st, b, h)


# 2-bit matrix-core streams with at most four query heads per kv head run two waves
# per SIMD with a ring of two tiles; eight heads keep one wave and a ring of four.
# Each instantiation shape, with the default split plan and with nine key groups per
# split (waves of three and two groups: the ring's tail after the last whole
# iteration).
@pytest.mark.parametrize("kw", [
    dict(n_q_heads=4, bits=2, k_group=64, residual=128, v_group=64),     # g = 2, two value groups
    dict(n_q_heads=8, bits=2, k_group=128, residual=128, v_group=128),   # g = 4, two tiles per group
    dict(n_q_heads=8, bits=2, k_group=256, residual=256, v_group=64),    # g = 4, four tiles per group
    dict(n_q_heads=4, bits=2, head_dim=64, k_group=64, residual=64, v_group=64, dtype="f32"),  # D64
    dict(n_q_heads=16, bits=2, k_group=64, residual=128, v_group=64),    # g = 8, one wave
])
@pytest.mark.parametrize("split_groups", [0, 9])
def test_two_wave_streams_against_oracle(kw, split_groups):
    require_gpu()
    w = _w(**kw)
    n = 40 * w.k_group + w.residual // 2 + 3
    log("case %s split_groups=%d n=%d" % (kw, split_groups, n))
    cache = make_cache(w, max_tokens=n)
    if split_groups:
        cache.set_split_tokens(split_groups * w.k_group)
    K, V = _tokens(w, n, 51, 2.0), _tokens(w, n, 52)
    cache.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    sts, err = _attend_and_check(w, cache, K, V)
    ex = export_cpu(cache)
    for (b, h), st in sts.items():
        assert_export_slice_matches(ex, st, b, h)


def test_bulk_append_equals_one_token_appends():
    require_gpu()
    w = _w(n_sink=2, bits=2)
    n = 3 * 64 + 17
    K, V = _tokens(w, n, 21, 3.0), _tokens(w, n, 22)
    a = make_cache(w, max_tokens=n)
    a.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    b = make_cache(w, max_tokens=n)
    # irregular chunking: 1, 5, 1, 70, ...
    i, sizes = 0, [1, 5, 1, 70, 2, 64, 1]
    j = 0
    while i < n:
        m = min(sizes[j % len(sizes)], n - i)
        b.append(to_torch(np.ascontiguousarray(K[:, :, i:i + m]), w.dtype, DEV),
                 to_torch(np.ascontiguousarray(V[:, :, i:i + m]), w.dtype, DEV))
        i += m
        j += 1
    assert a.state() == b.state()
    ea, eb = export_cpu(a), export_cpu(b)
    for k in ea:
        np.testing.assert_array_equal(ea[k], eb[k])
    ka, va = a.dequantize()
    kb, vb = b.dequantize()
    assert torch.equal(ka, kb) and torch.equal(va, vb)


def test_adversarial_groups_bit_exact():
    require_gpu()
    w = _w(dtype="f32", head_dim=64, v_group=16, k_group=32, residual=32, bits=4)
    n = 32 * 6
    rng = np.random.default_rng(3)
    K = rng.standard_normal((w.batch, w.n_kv_heads, n, 64)).astype(np.float32)
    V = rng.standard_normal((w.batch, w.n_kv_heads, n, 64)).astype(np.float32)
    K[0, 0, 0:32, :] = 0.7              # constant key groups
    K[0, 0, 32:64, 5] = -0.0            # signed zeros
    K[0, 0, 32:64, 6] = np.where(np.arange(32) % 2, 0.0, -0.0)
    K[0, 1, 64:96, :] = (rng.standard_normal((32, 64)) * 1e-40).astype(np.float32)  # subnormals
    K[1, 0, 96:128, :] = 5.0 + rng.uniform(0, 1, (32, 64)).astype(np.float32)       # one-signed
    K[1, 1, 128:160, :] = (rng.integers(-3, 4, (32, 64)) * 0.25).astype(np.float32)  # ties
    K[1, 1, 160:192, 3] = np.float32(1.4e-45) * np.arange(32)  # tiny range, scale underflow
    V[0, 0, :, 0:16] = -2.5             # constant value groups
    V[0, 1, :, 16:32] = 0.0
    V[1, 0, :, 32:48] = (rng.standard_normal((n, 16)) * 1e-42).astype(np.float32)
    V[1, 1, 5, :] = np.float32(1e30)
    V[1, 1, 6, :] = np.float32(-1e30)
    cache = make_cache(w, max_tokens=n)
    cache.append(to_torch(K, "f32", DEV), to_torch(V, "f32", DEV))
    ex = export_cpu(cache)
    for (b, h), st in _oracle_states(w, K, V).items():
        assert_export_slice_matches(ex, st, b, h)
    kd, vd = cache.dequantize()
    kd, vd = kd.cpu().numpy(), vd.cpu().numpy()
    for (b, h), st in _oracle_states(w, K, V).items():
        Ko, Vo = oracle.dequant_slice(st)
        np.testing.assert_array_equal(kd[b, h].view(np.uint32), Ko.view(np.uint32))
        np.testing.assert_array_equal(vd[b, h].view(np.uint32), Vo.view(np.uint32))


def test_state_machine_and_empty_cases():
    require_gpu()
    w = _w(n_sink=4, residual=64, k_group=32)
    cache = make_cache(w, max_tokens=200)
    q = to_torch(wl.random_tokens(1, (w.batch, w.n_q_heads, w.head_dim), w.dtype), w.dtype, DEV)
    # empty cache: attention is an argument error and enqueues nothing
    with pytest.raises(kvq.KVQError) as ei:
        cache.decode(q)
    assert ei.value.status == kvq.KVQ_ERR_INVALID_ARG
    # n_new == 0 is a no-op
    z = torch.empty((w.batch, w.n_kv_heads, 0, w.head_dim), dtype=TORCH_DTYPES[w.dtype], device=DEV)
    cache.append(z, z)
    assert cache.state() == (0, 0, 0, 0)
    K, V = _tokens(w, 200, 31), _tokens(w, 200, 32)
    done = 0
    for m in [2, 2, 3, 60, 1, 64, 68]:   # sinks only, sinks + residual, flushes, ...
        cache.append(to_torch(np.ascontiguousarray(K[:, :, done:done + m]), w.dtype, DEV),
                     to_torch(np.ascontiguousarray(V[:, :, done:done + m]), w.dtype, DEV))
        done += m
        N = done
        nS = min(N, 4)
        assert cache.state() == (N, nS, 64 * ((N - nS) // 64), (N - nS) % 64)
        _attend_and_check(w, cache, K[:, :, :done], V[:, :, :done], seed=done)
    # capacity: one more token is rejected and changes nothing
    one = to_torch(np.ascontiguousarray(K[:, :, :1]), w.dtype, DEV)
    with pytest.raises(kvq.KVQError) as ei:
        cache.append(one, one)
    assert ei.value.status == kvq.KVQ_ERR_CAPACITY
    assert cache.state() == (200, 4, 192, 4)
    _attend_and_check(w, cache, K, V, seed=99)


def test_workspace_and_argument_errors():
    require_gpu()
    w = _w()
    cache = make_cache(w, max_tokens=128)
    K, V = _tokens(w, 70, 41), _tokens(w, 70, 42)
    cache.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    q = to_torch(wl.random_tokens(2, (w.batch, w.n_q_heads, w.head_dim), w.dtype), w.dtype, DEV)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=DEV)
    with pytest.raises(kvq.KVQError) as ei:
        kvq.kvq_decode_attention(cache.handle, q.data_ptr(), out.data_ptr(), 0, cache._ws_ptr,
                                 cache.ws_bytes - 1, torch.cuda.current_stream().cuda_stream)
    assert ei.value.status == kvq.KVQ_ERR_BUFFER_TOO_SMALL
    with pytest.raises(kvq.KVQError) as ei:
        kvq.kvq_decode_attention(cache.handle, q.data_ptr(), out.data_ptr(), 0, cache._ws_ptr + 16,
                                 cache.ws_bytes, torch.cuda.current_stream().cuda_stream)
    assert ei.value.status == kvq.KVQ_ERR_INVALID_ARG
    with pytest.raises(kvq.KVQError) as ei:
        kvq.kvq_append(cache.handle, K.ctypes.data * 0, 0, 1, 0)
    assert ei.value.status == kvq.KVQ_ERR_INVALID_ARG
    with pytest.raises(kvq.KVQError) as ei:
        kvq.kvq_append(cache.handle, 16, 16, -1, 0)
    assert ei.value.status == kvq.KVQ_ERR_INVALID_ARG
    assert cache.state() == (70, 0, 64, 6)
    # lse is optional
    o2, l2 = cache.decode(q, with_lse=False)
    assert l2 is None
    o1, _ = cache.decode(q)
    assert torch.equal(o1, o2)
    _attend_and_check(w, cache, K, V, seed=2)


def test_sm_scale_override():
    require_gpu()
    w = _w()
    K, V = _tokens(w, 100, 51), _tokens(w, 100, 52)
    a = make_cache(w, max_tokens=100, sm_scale=0.3)
    a.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    q = wl.random_tokens(7, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
    out, lse = a.decode(to_torch(q, w.dtype, DEV))
    out = out.cpu().numpy()
    qf = wl.storage_to_f32(q, w.dtype)
    for (b, h), st in _oracle_states(w, K, V).items():
        Kd, Vd = oracle.dequant_slice(st)
        eo, _ = oracle.attention(qf[b, h], Kd, Vd, float(np.float32(0.3)))
        assert np.abs(out[b, h] - eo).max() <= ATOL


def test_two_caches_share_one_stream():
    require_gpu()
    w = _w(bits=2)
    K, V = _tokens(w, 150, 61), _tokens(w, 150, 62)
    a = make_cache(w, max_tokens=150)
    b = make_cache(w.replace(bits=4), max_tokens=150)
    a.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    b.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    _attend_and_check(w, a, K, V)
    _attend_and_check(w.replace(bits=4), b, K, V)


def _hip_runtime():
    """The HIP runtime library torch loaded (for event calls in the tests)."""
    import ctypes
    path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64.so" in l)
    rt = ctypes.CDLL(path)
    rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return rt


def test_timing_events_record_the_decode_kernel():
    import ctypes
    require_gpu()
    w = _w()
    cache = make_cache(w, max_tokens=256)
    K, V = _tokens(w, 151, 81), _tokens(w, 151, 82)
    cache.append(to_torch(K[:, :, :150], w.dtype, DEV), to_torch(V[:, :, :150], w.dtype, DEV))
    q = to_torch(wl.random_tokens(9, (w.batch, w.n_q_heads, w.head_dim), w.dtype), w.dtype, DEV)
    ref, ref_lse = cache.decode(q)
    ref, ref_lse = ref.clone(), ref_lse.clone()
    rt = _hip_runtime()
    ev = [ctypes.c_void_p() for _ in range(2)]
    for e in ev:
        assert rt.hipEventCreate(ctypes.byref(e)) == 0
    try:
        with pytest.raises(kvq.KVQError) as ei:
            cache.set_timing_events(ev[0], None)
        assert ei.value.status == kvq.KVQ_ERR_INVALID_ARG
        cache.set_timing_events(ev[0], ev[1])
        out, lse = cache.decode(q)
        torch.cuda.synchronize()
        ms = ctypes.c_float()
        assert rt.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
        assert 0.0 < ms.value < 1000.0, ms.value
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
        # the fused one-token step records the same way
        kn, vn = (to_torch(x[:, :, 150:151], w.dtype, DEV) for x in (K, V))
        out, lse = cache.append_decode(kn, vn, q)
        torch.cuda.synchronize()
        ms2 = ctypes.c_float()
        assert rt.hipEventElapsedTime(ctypes.byref(ms2), ev[0], ev[1]) == 0
        assert 0.0 < ms2.value < 1000.0, ms2.value
        log("decode kernel %.1f us, fused step kernel %.1f us" % (ms.value * 1e3, ms2.value * 1e3))
        cache.set_timing_events(None, None)
        _attend_and_check(w, cache, K, V, seed=9)
    finally:
        torch.cuda.synchronize()
        for e in ev:
            rt.hipEventDestroy(e)


def test_stream_read_probe():
    require_gpu()
    x = torch.arange(1 << 20, dtype=torch.int32, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    sp = torch.cuda.current_stream().cuda_stream
    for bpc in (1, 4):
        kvq.kvq_stream_read_probe(x.data_ptr(), x.numel() * 4, bpc, sink.data_ptr(), sp)
    kvq.kvq_stream_read_probe(x.data_ptr(), 48, 1, sink.data_ptr(), sp)  # less than one word per thread
    torch.cuda.synchronize()
    for args, why in [((x.data_ptr() + 4, 64, 1), "misaligned"), ((x.data_ptr(), 60, 1), "ragged size"),
                      ((x.data_ptr(), 64, 0), "no workgroups"), ((0, 64, 1), "null")]:
        with pytest.raises(kvq.KVQError) as ei:
            kvq.kvq_stream_read_probe(*args, sink.data_ptr(), sp)
        assert ei.value.status == kvq.KVQ_ERR_INVALID_ARG, why
    assert torch.equal(x, torch.arange(1 << 20, dtype=torch.int32, device=DEV))  # read only


# The cache buffer needs no initialisation and the workspace only zeroed counters.
# Both are filled with 0xFF bytes (NaN as fp32, NaN or -NaN as bf16 / f16) before
# the first append, and attention runs right after a prefill that leaves no
# full-precision token in the slice (a whole number of residuals, no sinks): no
# unwritten byte may reach an output, not even multiplied by a zero weight.
@pytest.mark.parametrize("kw", [
    dict(),                                                      # VALU stream, bf16
    dict(dtype="f32", head_dim=64, v_group=16, bits=2),          # VALU stream, f32
    dict(n_q_heads=8, k_group=64, residual=128, v_group=64),     # matrix cores, g = 4
    dict(bits=8, k_group=64, residual=128, v_group=64),          # 8-bit, matrix cores
    dict(outliers=1),                                            # dense-and-sparse
])
def test_uninitialised_buffers_do_not_reach_outputs(kw):
    require_gpu()
    w = _w(**kw)
    log("case %s" % kw)
    cache = make_cache(w, max_tokens=4 * w.residual)
    cache._buf.fill_(0xFF)
    # past the counters: at most 1 + 16 per slice (a slice counter and, for the
    # two-level split combine, up to 16 group counters)
    ws_off = (w.batch * w.n_kv_heads * 17 * 4 + 255) // 256 * 256
    base = cache._ws_ptr - cache._ws.data_ptr()
    cache._ws[base + ws_off:].fill_(0xFF)
    torch.cuda.synchronize()
    n = 2 * w.residual
    K, V = _tokens(w, n, 71, 2.0), _tokens(w, n, 72)
    cache.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    assert cache.state() == (n, 0, n, 0)
    _attend_and_check(w, cache, K, V, seed=73)
    # one fused step then has a single full-precision token
    K1, V1 = _tokens(w, 1, 74), _tokens(w, 1, 75)
    q = wl.random_tokens(76, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
    out, lse = cache.append_decode(to_torch(K1, w.dtype, DEV), to_torch(V1, w.dtype, DEV), to_torch(q, w.dtype, DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    _attend_and_check(w, cache, np.concatenate([K, K1], 2), np.concatenate([V, V1], 2), seed=77)


# Split combines over many splits: one sequence, one kv head, a split per key
# group.  Up to 16 splits merge in one level; more merge in groups of
# ceil(sqrt(nsplit)) splits, then over the groups (17 splits: groups of 5, 5, 5, 2;
# 256, the most a slice holds: 16 groups of 16).
@pytest.mark.parametrize("kw,groups", [
    (dict(n_q_heads=8, n_kv_heads=1, batch=1, k_group=64, residual=128, v_group=64), 100),   # groups of 10
    (dict(n_q_heads=4, n_kv_heads=1, batch=1, k_group=64, residual=128, v_group=64), 150),   # groups of 13
    (dict(n_q_heads=8, n_kv_heads=1, batch=1, bits=2, k_group=32, residual=64, v_group=32), 120),  # VALU
    (dict(n_q_heads=4, n_kv_heads=1, batch=1, k_group=64, residual=128, v_group=64), 16),    # one level
    (dict(n_q_heads=4, n_kv_heads=1, batch=1, k_group=64, residual=64, v_group=64), 17),     # ragged groups
    (dict(n_q_heads=2, n_kv_heads=1, batch=1, bits=2, k_group=32, residual=64, v_group=32), 256),  # 16 x 16
    (dict(n_q_heads=1, n_kv_heads=1, batch=1, bits=4, k_group=64, residual=64, v_group=64), 256),  # MHA, 16 x 16
])
def test_combine_of_many_splits(kw, groups):
    require_gpu()
    w = _w(**kw)
    n = groups * w.k_group + 5
    log("case %s n=%d" % (kw, n))
    cache = make_cache(w, max_tokens=n)
    K, V = _tokens(w, n, 81, 2.0), _tokens(w, n, 82)
    cache.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    assert cache.state()[2] == groups * w.k_group
    q = to_torch(wl.random_tokens(83, (w.batch, w.n_q_heads, w.head_dim), w.dtype), w.dtype, DEV)
    ref, ref_lse = cache.decode(q)
    ref, ref_lse = ref.clone(), ref_lse.clone()
    cache.set_split_tokens(w.k_group)   # one split per key group
    _attend_and_check(w, cache, K, V, seed=83)
    out, lse = cache.decode(q)
    torch.cuda.synchronize()
    scale = max(1.0, ref.abs().max().item())
    assert (out - ref).abs().max().item() <= 5e-5 * scale
    assert (lse - ref_lse).abs().max().item() <= 5e-5 * max(1.0, ref_lse.abs().max().item())


# Sequences of very different lengths under a split plan made for the longest:
# most splits of the short sequences hold no key group (and the shortest no
# quantized token at all), so their partials are empty; with more than 16 splits
# the combine runs in two levels, and a group of empty partials merges to an empty
# group partial.
@pytest.mark.parametrize("kw", [
    dict(batch=3, n_kv_heads=2, n_q_heads=8, bits=2, k_group=64, residual=128, v_group=64),  # matrix cores
    dict(batch=3, n_kv_heads=2, n_q_heads=2, k_group=32, residual=64, v_group=32),          # VALU stream
])
def test_ragged_lengths_under_many_splits(kw):
    require_gpu()
    w = _w(**kw)
    lens = [3000, 130, 1]
    n_max = max(lens)
    log("case %s lens %s" % (kw, lens))
    cache = make_cache(w, max_tokens=n_max)
    K, V = _tokens(w, n_max, 111, 2.0), _tokens(w, n_max, 112)
    cache.append_ragged(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV), lens)
    cache.set_split_tokens(w.k_group)   # one split per key group of the longest: more than 16
    q = wl.random_tokens(113, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
    out, lse = cache.decode(to_torch(q, w.dtype, DEV))
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    kf, vf, qf = (wl.storage_to_f32(x, w.dtype) for x in (K, V, q))
    scale = oracle.default_scale(w.head_dim)
    err = 0.0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            st = oracle.build_slice(kf[b, h, :lens[b]], vf[b, h, :lens[b]], head_dim=w.head_dim, bits=w.bits,
                                    k_group=w.k_group, v_group=w.v_group, residual=w.residual,
                                    n_sink=w.n_sink, codec=w.codec)
            Kd, Vd = oracle.dequant_slice(st)
            for j in range(w.gqa):
                eo, el = oracle.attention(qf[b, h * w.gqa + j], Kd, Vd, scale)
                err = max(err, float(np.abs(out[b, h * w.gqa + j] - eo).max()),
                          abs(float(lse[b, h * w.gqa + j]) - el))
    assert err <= ATOL, err


# Weighted split plan.  The 2-bit matrix-core streams run two workgroups per CU;
# where the default plan fills every slot once (splits x slices = 2 x CUs, the
# slices dividing the CUs), the splits dispatched first on their CUs take 11/8 of
# the key groups of the others, on a split-major grid.  With T = 2 CUs / slices,
# 4T - 3 key groups (4T - 2 where the residual flushes two groups at a time) plan
# T splits, the first half of 5 groups and the second of 3, the last one empty (or
# of one group); the shorter sequence of the ragged case leaves more splits empty.
# The result must match the oracle and the plain plan of the same split count
# (four groups a split, a fixed split size, which the weighting skips).
@pytest.mark.parametrize("kw", [
    dict(n_q_heads=8, bits=2, k_group=64, residual=128, v_group=64),                       # g = 4
    dict(n_q_heads=4, bits=2, head_dim=64, k_group=64, residual=64, v_group=64, dtype="f32"),  # g = 2, D64
    dict(n_q_heads=8, bits=2, k_group=64, residual=128, v_group=64, key_axis=1),           # per-token keys
    dict(n_q_heads=8, bits=2, k_group=64, residual=128, v_group=64, outliers=1),           # dense-and-sparse
])
@pytest.mark.parametrize("ragged", [False, True])
def test_weighted_split_plan(kw, ragged):
    require_gpu()
    w = _w(**kw)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    bh = w.batch * w.n_kv_heads
    if n_cu % bh:
        pytest.skip("weighted plan needs the slices to divide the %d CUs" % n_cu)
    T = 2 * n_cu // bh
    ng = 4 * T - 3
    n = ng * w.k_group + w.residual // 2 + 7
    lens = [n, n - 37 * w.k_group - 5] if ragged else [n, n]
    log("case %s ragged=%s n=%d lens=%s CUs=%d" % (kw, ragged, n, lens, n_cu))
    cache = make_cache(w, max_tokens=n)
    K, V = _tokens(w, n, 121, 2.0), _tokens(w, n, 122)
    if ragged:
        cache.append_ragged(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV), lens)
    else:
        cache.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
    q = wl.random_tokens(123, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
    qd = to_torch(q, w.dtype, DEV)
    out, lse = cache.decode(qd)
    out, lse = out.clone(), lse.clone()
    cache.set_split_tokens(4 * w.k_group)   # same split count, equal splits
    ref, ref_lse = cache.decode(qd)
    torch.cuda.synchronize()
    scale = max(1.0, ref.abs().max().item())
    assert (out - ref).abs().max().item() <= 5e-5 * scale
    assert (lse - ref_lse).abs().max().item() <= 5e-5 * max(1.0, ref_lse.abs().max().item())
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    kf, vf, qf = (wl.storage_to_f32(x, w.dtype) for x in (K, V, q))
    sc = oracle.default_scale(w.head_dim)
    err = 0.0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            st = oracle.build_slice(kf[b, h, :lens[b]], vf[b, h, :lens[b]], head_dim=w.head_dim, bits=w.bits,
                                    k_group=w.k_group, v_group=w.v_group, residual=w.residual,
                                    n_sink=w.n_sink, codec=w.codec, outliers=w.outliers, key_axis=w.key_axis)
            Kd, Vd = oracle.dequant_slice(st)
            for j in range(w.gqa):
                eo, el = oracle.attention(qf[b, h * w.gqa + j], Kd, Vd, sc)
                err = max(err, float(np.abs(out[b, h * w.gqa + j] - eo).max()),
                          abs(float(lse[b, h * w.gqa + j]) - el))
    assert err <= ATOL, err
