"""Low-bit (INT4 / INT2) KV-cache decode attention for MI355X (gfx950).

A thin ctypes binding over libkvq.so (C-ABI declared in include/kvq.h).  Every
step of the path runs in the library's HIP kernels; this module only marshals
arguments: torch supplies device memory and the current stream.  There is no
CPU fallback: if libkvq.so is missing or fails to load, every call raises.

Low-level functions mirror the C entry points one to one (kvq_cache_bytes,
kvq_cache_create, kvq_append, kvq_decode_workspace_bytes, kvq_decode_attention,
kvq_dequantize, kvq_export, kvq_cache_state, kvq_set_split_tokens,
kvq_set_timing_events, kvq_stream_read_probe, kvq_append_ragged, kvq_seq_lengths,
kvq_last_error); ``Cache`` bundles them with torch-allocated buffers.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

# KVQ_LIB names another build of the library (the host-sanitized one of
# `python -m bit_quantized_kv_kvq_amd.build --sanitize`)
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

KVQ_OK = 0
KVQ_ERR_INVALID_ARG = -1
KVQ_ERR_UNSUPPORTED = -2
KVQ_ERR_CAPACITY = -3
KVQ_ERR_BUFFER_TOO_SMALL = -4
KVQ_ERR_DEVICE = -5
STATUS_NAMES = {0: "KVQ_OK", -1: "KVQ_ERR_INVALID_ARG", -2: "KVQ_ERR_UNSUPPORTED",
                -3: "KVQ_ERR_CAPACITY", -4: "KVQ_ERR_BUFFER_TOO_SMALL", -5: "KVQ_ERR_DEVICE"}

KVQ_F32, KVQ_BF16, KVQ_F16 = 0, 1, 2
KVQ_STATIC_SCRATCH_BYTES = 16 << 20
KVQ_CODEC_ASYMMETRIC, KVQ_CODEC_SYMMETRIC = 0, 1
KVQ_RETAIN_WINDOW, KVQ_RETAIN_LOG = 0, 1
KVQ_KEY_PER_CHANNEL, KVQ_KEY_PER_TOKEN = 0, 1

EXPORTED = ["kvq_cache_bytes", "kvq_cache_create", "kvq_cache_destroy", "kvq_append",
            "kvq_decode_workspace_bytes", "kvq_decode_attention", "kvq_decode_attention_static",
            "kvq_append_decode",
            "kvq_dequantize", "kvq_export",
            "kvq_cache_state", "kvq_set_split_tokens", "kvq_set_timing_events", "kvq_stream_read_probe",
            "kvq_append_ragged", "kvq_seq_lengths", "kvq_release_sequence", "kvq_pool_free_pages",
            "kvq_export_outliers", "kvq_last_error"]


class KVQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), message))
        self.status = status
        self.message = message


class Config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("k_group", ctypes.c_int32),
                ("v_group", ctypes.c_int32), ("residual", ctypes.c_int32),
                ("n_sink", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("max_tokens", ctypes.c_int64), ("sm_scale", ctypes.c_float),
                ("codec", ctypes.c_int32), ("retention", ctypes.c_int32),
                ("page_groups", ctypes.c_int32), ("pool_pages", ctypes.c_int64),
                ("outliers", ctypes.c_int32), ("key_axis", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvq.so (built by bit_quantized_kv_kvq_amd.build).  Raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libkvq.so not found at %s: build it with "
                              "`python -m bit_quantized_kv_kvq_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, i64, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        CP = ctypes.POINTER(Config)
        sig = {
            "kvq_cache_bytes": [CP, ctypes.POINTER(ctypes.c_size_t)],
            "kvq_cache_create": [CP, P, ctypes.c_size_t, ctypes.POINTER(P)],
            "kvq_cache_destroy": [P],
            "kvq_append": [P, P, P, i64, P],
            "kvq_decode_workspace_bytes": [P, ctypes.POINTER(ctypes.c_size_t)],
            "kvq_decode_attention": [P, P, P, P, P, ctypes.c_size_t, P],
            "kvq_decode_attention_static": [P, P, P, P, P],
            "kvq_append_decode": [P, P, P, P, P, P, P, ctypes.c_size_t, P],
            "kvq_dequantize": [P, P, P, P],
            "kvq_export": [P, P, P, P, P, P, P, P],
            "kvq_cache_state": [P] + [ctypes.POINTER(i64)] * 4,
            "kvq_set_split_tokens": [P, i64],
            "kvq_set_timing_events": [P, P, P],
            "kvq_stream_read_probe": [P, ctypes.c_size_t, ctypes.c_int32, P, P],
            "kvq_append_ragged": [P, P, P, ctypes.POINTER(ctypes.c_int32), i64, P],
            "kvq_seq_lengths": [P, ctypes.POINTER(i64)],
            "kvq_release_sequence": [P, ctypes.c_int32, P],
            "kvq_pool_free_pages": [P, ctypes.POINTER(i64)],
            "kvq_export_outliers": [P, P, P, P, P, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = st
        L.kvq_last_error.argtypes = []
        L.kvq_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def kvq_last_error() -> str:
    return lib().kvq_last_error().decode()


def _check(status: int):
    if status != KVQ_OK:
        raise KVQError(status, kvq_last_error())


def make_config(*, batch, n_kv_heads, n_q_heads, head_dim, bits, k_group, v_group, residual,
                n_sink=0, dtype=KVQ_BF16, max_tokens, sm_scale=0.0, codec=KVQ_CODEC_ASYMMETRIC,
                retention=KVQ_RETAIN_WINDOW, page_groups=0, pool_pages=0, outliers=0,
                key_axis=KVQ_KEY_PER_CHANNEL) -> Config:
    return Config(batch, n_kv_heads, n_q_heads, head_dim, bits, k_group, v_group, residual,
                  n_sink, dtype, max_tokens, sm_scale, codec, retention, page_groups, pool_pages, outliers,
                  key_axis)


def kvq_cache_bytes(cfg: Config) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().kvq_cache_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def kvq_cache_create(cfg: Config, dev_ptr: int, nbytes: int) -> int:
    h = ctypes.c_void_p(0)
    _check(lib().kvq_cache_create(ctypes.byref(cfg), ctypes.c_void_p(dev_ptr), nbytes,
                                  ctypes.byref(h)))
    return h.value


def kvq_cache_destroy(handle: int):
    _check(lib().kvq_cache_destroy(ctypes.c_void_p(handle)))


def kvq_append(handle: int, k_ptr: int, v_ptr: int, n_new: int, stream: int):
    _check(lib().kvq_append(ctypes.c_void_p(handle), ctypes.c_void_p(k_ptr),
                            ctypes.c_void_p(v_ptr), n_new, ctypes.c_void_p(stream)))


def kvq_decode_workspace_bytes(handle: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().kvq_decode_workspace_bytes(ctypes.c_void_p(handle), ctypes.byref(n)))
    return n.value


def kvq_decode_attention(handle: int, q_ptr: int, out_ptr: int, lse_ptr: int, ws_ptr: int,
                         ws_bytes: int, stream: int):
    _check(lib().kvq_decode_attention(ctypes.c_void_p(handle), ctypes.c_void_p(q_ptr),
                                      ctypes.c_void_p(out_ptr), ctypes.c_void_p(lse_ptr or None),
                                      ctypes.c_void_p(ws_ptr), ws_bytes, ctypes.c_void_p(stream)))


def kvq_decode_attention_static(handle: int, q_ptr: int, out_ptr: int, lse_ptr: int, stream: int):
    _check(lib().kvq_decode_attention_static(ctypes.c_void_p(handle), ctypes.c_void_p(q_ptr),
                                             ctypes.c_void_p(out_ptr), ctypes.c_void_p(lse_ptr or None),
                                             ctypes.c_void_p(stream)))


def kvq_append_decode(handle: int, k_ptr: int, v_ptr: int, q_ptr: int, out_ptr: int, lse_ptr: int,
                      ws_ptr: int, ws_bytes: int, stream: int):
    _check(lib().kvq_append_decode(ctypes.c_void_p(handle), ctypes.c_void_p(k_ptr),
                                   ctypes.c_void_p(v_ptr), ctypes.c_void_p(q_ptr),
                                   ctypes.c_void_p(out_ptr), ctypes.c_void_p(lse_ptr or None),
                                   ctypes.c_void_p(ws_ptr), ws_bytes, ctypes.c_void_p(stream)))


def kvq_dequantize(handle: int, k_ptr: int, v_ptr: int, stream: int):
    _check(lib().kvq_dequantize(ctypes.c_void_p(handle), ctypes.c_void_p(k_ptr),
                                ctypes.c_void_p(v_ptr), ctypes.c_void_p(stream)))


def kvq_export(handle: int, ptrs, stream: int):
    """ptrs: (k_codes, k_scale, k_zero, v_codes, v_scale, v_zero) device pointers or 0."""
    _check(lib().kvq_export(ctypes.c_void_p(handle), *[ctypes.c_void_p(p or None) for p in ptrs],
                            ctypes.c_void_p(stream)))


def kvq_cache_state(handle: int) -> Tuple[int, int, int, int]:
    v = [ctypes.c_int64(0) for _ in range(4)]
    _check(lib().kvq_cache_state(ctypes.c_void_p(handle), *[ctypes.byref(x) for x in v]))
    return tuple(x.value for x in v)


def kvq_set_split_tokens(handle: int, tokens: int):
    _check(lib().kvq_set_split_tokens(ctypes.c_void_p(handle), tokens))


def kvq_append_ragged(handle: int, k: int, v: int, n_new, n_max: int, stream: int):
    """n_new: sequence of B ints (host)."""
    arr = (ctypes.c_int32 * len(n_new))(*[int(x) for x in n_new])
    _check(lib().kvq_append_ragged(ctypes.c_void_p(handle), ctypes.c_void_p(k), ctypes.c_void_p(v), arr,
                                   n_max, ctypes.c_void_p(stream)))


def kvq_seq_lengths(handle: int, batch: int):
    arr = (ctypes.c_int64 * batch)()
    _check(lib().kvq_seq_lengths(ctypes.c_void_p(handle), arr))
    return [int(x) for x in arr]


def kvq_release_sequence(handle: int, b: int, stream: int):
    _check(lib().kvq_release_sequence(ctypes.c_void_p(handle), b, ctypes.c_void_p(stream)))


def kvq_export_outliers(handle: int, k_idx: int, k_val: int, v_idx: int, v_val: int, stream: int):
    _check(lib().kvq_export_outliers(ctypes.c_void_p(handle), ctypes.c_void_p(k_idx), ctypes.c_void_p(k_val),
                                     ctypes.c_void_p(v_idx), ctypes.c_void_p(v_val), ctypes.c_void_p(stream)))


def kvq_pool_free_pages(handle: int) -> int:
    n = ctypes.c_int64(0)
    _check(lib().kvq_pool_free_pages(ctypes.c_void_p(handle), ctypes.byref(n)))
    return n.value


def kvq_stream_read_probe(buf: int, nbytes: int, blocks_per_cu: int, sink: int, stream: int):
    _check(lib().kvq_stream_read_probe(ctypes.c_void_p(buf), nbytes, blocks_per_cu,
                                       ctypes.c_void_p(sink), ctypes.c_void_p(stream)))


def kvq_set_timing_events(handle: int, start_event, stop_event):
    """start_event, stop_event: hipEvent_t handles (int or ctypes.c_void_p), or None, None."""
    _check(lib().kvq_set_timing_events(ctypes.c_void_p(handle), start_event, stop_event))


from .cache import Cache, torch_dtype_code  # noqa: E402  (needs the names above)

__all__ = ["Cache", "Config", "KVQError", "lib", "make_config", "torch_dtype_code"] + EXPORTED
