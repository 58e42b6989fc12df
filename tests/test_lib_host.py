"""Host-side checks of libkvq.so that need no GPU: it loads, exports every symbol
that include/kvq.h declares, validates configurations and sizes the cache buffer."""
import ctypes
import os
import re

import pytest

import bit_quantized_kv_kvq_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(kvq.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = kvq.lib()
    for name in _declared():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def _cfg(**kw):
    base = dict(batch=2, n_kv_heads=4, n_q_heads=8, head_dim=128, bits=4, k_group=64,
                v_group=32, residual=128, n_sink=4, dtype=kvq.KVQ_BF16, max_tokens=1000)
    base.update(kw)
    return kvq.make_config(**base)


def _expected_bytes(c):
    """Sinks and residual (K and V), one record per key group of capacity, then the
    int32 length of every sequence."""
    al = lambda x: (x + 255) & ~255
    e = 4 if c.dtype == kvq.KVQ_F32 else 2
    BH = c.batch * c.n_kv_heads
    D, G = c.head_dim, c.k_group
    m = max(0, c.max_tokens - c.n_sink)
    if c.retention == kvq.KVQ_RETAIN_LOG:  # W quantized per flush, the first once 3W are held
        W = c.residual // 3
        Lq_cap = 0 if m < c.residual else W * ((m - c.residual) // W + 1)
    else:
        Lq_cap = c.residual * (m // c.residual)
    row = D * c.bits // 8
    nvg = D // c.v_group
    # with outliers: key outlier values fp32 [D] and (token | code) u16 [D], value outliers
    # fp32 and u16 per (token, value group)
    # key (scale, zero): fp32 [2][D] per channel, or [G][2] per token
    kmeta = 8 * G if c.key_axis else 8 * D
    rec = al(kmeta + 2 * G * row + G * nvg * 8 + (6 * D + 6 * G * nvg if c.outliers else 0))
    if c.page_groups:  # a pool of pages of page_groups key groups of every kv head, and a page table
        max_pages = -(-(Lq_cap // G) // c.page_groups)
        pool = c.pool_pages or c.batch * max_pages
        records, table = pool * c.n_kv_heads * c.page_groups * rec, 4 * c.batch * max_pages
    else:
        records, table = BH * (Lq_cap // G) * rec, 0
    parts = [BH * c.n_sink * D * e] * 2 + [BH * c.residual * D * e] * 2 + [records, 4 * c.batch, table]
    return sum(al(p) for p in parts)


@pytest.mark.parametrize("kw", [{}, dict(bits=2), dict(dtype=kvq.KVQ_F32, head_dim=64, v_group=64),
                                dict(n_sink=0, max_tokens=129), dict(max_tokens=3),
                                dict(n_q_heads=32, n_kv_heads=4), dict(bits=8, v_group=64),
                                dict(bits=8, n_q_heads=4, k_group=128, v_group=128),
                                dict(retention=kvq.KVQ_RETAIN_LOG, residual=192),
                                dict(retention=kvq.KVQ_RETAIN_LOG, residual=192, max_tokens=195),
                                dict(retention=kvq.KVQ_RETAIN_LOG, residual=192, max_tokens=196),
                                dict(retention=kvq.KVQ_RETAIN_LOG, k_group=32, residual=96, n_sink=0),
                                dict(page_groups=4), dict(page_groups=1, max_tokens=5000),
                                dict(page_groups=2, pool_pages=7), dict(page_groups=8, max_tokens=100),
                                dict(page_groups=4, retention=kvq.KVQ_RETAIN_LOG, residual=192),
                                dict(outliers=1, n_q_heads=4), dict(outliers=1, n_q_heads=4, bits=2, head_dim=64),
                                dict(outliers=1), dict(outliers=1, n_q_heads=32),
                                dict(outliers=1, n_q_heads=4, page_groups=2, k_group=32, residual=64),
                                dict(key_axis=1, n_q_heads=4, v_group=64), dict(key_axis=1, n_q_heads=4, k_group=128,
                                                                                v_group=128),
                                dict(key_axis=1, n_q_heads=4, v_group=64, page_groups=2),
                                dict(key_axis=1, n_q_heads=4, v_group=32, bits=2)])
def test_cache_bytes_matches_layout(kw):
    c = _cfg(**kw)
    assert kvq.kvq_cache_bytes(c) == _expected_bytes(c)


@pytest.mark.parametrize("kw,status", [
    (dict(bits=3), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(bits=8), kvq.KVQ_ERR_UNSUPPORTED),                 # 8-bit codes need G_V >= 64
    (dict(bits=8, k_group=32, v_group=64), kvq.KVQ_ERR_UNSUPPORTED),  # and G >= 64
    (dict(bits=16), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(head_dim=96, v_group=32), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(n_q_heads=12, n_kv_heads=4), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(n_q_heads=6, n_kv_heads=4), kvq.KVQ_ERR_INVALID_ARG),
    (dict(residual=100), kvq.KVQ_ERR_INVALID_ARG),
    (dict(v_group=48), kvq.KVQ_ERR_INVALID_ARG),
    (dict(k_group=48, residual=96), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(k_group=96, residual=192), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(k_group=16, residual=64), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(k_group=512, residual=512), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(v_group=8), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(batch=0), kvq.KVQ_ERR_INVALID_ARG),
    (dict(n_sink=-1), kvq.KVQ_ERR_INVALID_ARG),
    (dict(max_tokens=0), kvq.KVQ_ERR_INVALID_ARG),
    (dict(dtype=7), kvq.KVQ_ERR_INVALID_ARG),
    (dict(sm_scale=-1.0), kvq.KVQ_ERR_INVALID_ARG),
    (dict(sm_scale=float("nan")), kvq.KVQ_ERR_INVALID_ARG),
    (dict(page_groups=3), kvq.KVQ_ERR_INVALID_ARG),
    (dict(page_groups=-2), kvq.KVQ_ERR_INVALID_ARG),
    (dict(page_groups=4, pool_pages=-1), kvq.KVQ_ERR_INVALID_ARG),
    (dict(page_groups=4, pool_pages=1 << 22), kvq.KVQ_ERR_UNSUPPORTED),       # pool above 4 GiB
    (dict(outliers=2), kvq.KVQ_ERR_INVALID_ARG),
    (dict(outliers=1, n_q_heads=4, bits=8, v_group=64), kvq.KVQ_ERR_UNSUPPORTED),   # 8-bit codes
    (dict(retention=2), kvq.KVQ_ERR_INVALID_ARG),
    (dict(retention=-1), kvq.KVQ_ERR_INVALID_ARG),
    (dict(retention=kvq.KVQ_RETAIN_LOG), kvq.KVQ_ERR_INVALID_ARG),               # R = 128 is not 3W
    (dict(retention=kvq.KVQ_RETAIN_LOG, residual=256, k_group=128), kvq.KVQ_ERR_INVALID_ARG),  # 3G does not divide R
    (dict(key_axis=2), kvq.KVQ_ERR_INVALID_ARG),
    (dict(key_axis=1, k_group=32), kvq.KVQ_ERR_UNSUPPORTED),        # per-token keys: records of 64 or 128 tokens
    (dict(key_axis=1, k_group=128, residual=256, n_q_heads=4, outliers=1), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(key_axis=1), kvq.KVQ_ERR_UNSUPPORTED),                    # several query heads with G_V = 32
])
def test_invalid_configs_are_rejected(kw, status):
    with pytest.raises(kvq.KVQError) as ei:
        kvq.kvq_cache_bytes(_cfg(**kw))
    assert ei.value.status == status
    assert ei.value.message  # thread-local message is set


def test_codec_field_and_null_pointers():
    c = _cfg()
    for bad in (2, -1, 7):
        c.codec = bad
        with pytest.raises(kvq.KVQError) as ei:
            kvq.kvq_cache_bytes(c)
        assert ei.value.status == kvq.KVQ_ERR_INVALID_ARG
    c.codec = kvq.KVQ_CODEC_SYMMETRIC
    assert kvq.kvq_cache_bytes(c) > 0
    lib = kvq.lib()
    assert lib.kvq_cache_bytes(None, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_cache_state(None, None, None, None, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_append(None, None, None, 1, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_decode_attention(None, None, None, None, None, 0, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_set_timing_events(None, None, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_release_sequence(None, 0, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_pool_free_pages(None, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_export_outliers(None, None, None, None, None, None) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_cache_destroy(None) == kvq.KVQ_OK
    assert kvq.kvq_last_error() == ""


def test_create_rejects_bad_buffer_before_touching_the_device():
    c = _cfg()
    n = kvq.kvq_cache_bytes(c)
    lib = kvq.lib()
    h = ctypes.c_void_p(0)
    assert lib.kvq_cache_create(ctypes.byref(c), None, n, ctypes.byref(h)) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_cache_create(ctypes.byref(c), ctypes.c_void_p(4096 + 8), n,
                                ctypes.byref(h)) == kvq.KVQ_ERR_INVALID_ARG
    assert lib.kvq_cache_create(ctypes.byref(c), ctypes.c_void_p(4096), n - 1,
                                ctypes.byref(h)) == kvq.KVQ_ERR_BUFFER_TOO_SMALL
    assert h.value is None


def test_workload_configs_are_supported():
    import workloads as wl
    for w in wl.WORKLOADS.values():
        c = kvq.make_config(batch=w.batch, n_kv_heads=w.n_kv_heads, n_q_heads=w.n_q_heads,
                            head_dim=w.head_dim, bits=w.bits, k_group=w.k_group,
                            v_group=w.v_group, residual=w.residual, n_sink=w.n_sink,
                            dtype={"f32": 0, "bf16": 1, "f16": 2}[w.dtype],
                            max_tokens=w.max_tokens, codec=w.codec,
                            retention=kvq.KVQ_RETAIN_LOG if w.log_window else kvq.KVQ_RETAIN_WINDOW,
                            page_groups=w.page_groups, outliers=w.outliers, key_axis=w.key_axis)
        assert kvq.kvq_cache_bytes(c) > 0
