"""CPU oracle for low-bit KV-cache decode attention (test infrastructure only).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never does, and the oracle never imports the product: the two share
only the seeded input generators in ``workloads``.

The arithmetic lives in ``kvq_oracle.c`` (fp32 codec in the written operation
order, binary64 attention); this module builds it with gcc and wraps it with
ctypes.  ``oracle.brute`` holds a second, pure-Python/numpy formulation for
tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
          "-fopenmp", "-fPIC", "-shared", "-Wall", "-Werror"]


def build(force: bool = False) -> str:
    """Compile the oracle library with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def load(path: str):
    """Load an oracle build with its ctypes prototypes."""
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    L.orc_quant_group.argtypes = [P, i64, i64, i32, i32, P, P, P, i64]
    L.orc_quant_group.restype = None
    L.orc_quant_group_skip.argtypes = [P, i64, i64, i32, i32, i64, P, P, P, i64]
    L.orc_quant_group_skip.restype = None
    L.orc_outlier_index.argtypes = [P, i64, i64]
    L.orc_outlier_index.restype = i64
    L.orc_dequant.argtypes = [ctypes.c_uint8, ctypes.c_float, ctypes.c_float]
    L.orc_dequant.restype = ctypes.c_float
    L.orc_build_slice.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, P, P, i64] + [P] * 14 + [P]
    L.orc_build_slice.restype = i32
    L.orc_dequant_slice.argtypes = [i32, i32, i32, i32, i64, i64, i64] + [P] * 10 + [i32] + [P] * 6
    L.orc_dequant_slice.restype = None
    L.orc_attention.argtypes = [P, P, P, i64, i32, dbl, P, P]
    L.orc_attention.restype = None
    L.orc_decode_slices.argtypes = [i64, i32, i32, i32, i32, i32, i64, i64, i64, dbl] + [P] * 10 + [i32] + [P] * 7
    L.orc_decode_slices.restype = None
    L.orc_num_threads.argtypes = []
    L.orc_num_threads.restype = i32
    L.orc_set_num_threads.argtypes = [i32]
    L.orc_set_num_threads.restype = None
    return L


def build_sanitized() -> str:
    """The oracle under gcc's AddressSanitizer and UndefinedBehaviorSanitizer
    (libkvq_oracle_san.so beside the source).  A process loads it through
    KVQ_ORACLE_LIB with gcc's libasan and libubsan preloaded, e.g.

        LD_PRELOAD=$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so) \
        ASAN_OPTIONS=detect_leaks=0 KVQ_ORACLE_LIB=oracle/libkvq_oracle_san.so \
        python -m pytest tests/test_oracle_*.py
    """
    out = os.path.join(_HERE, "libkvq_oracle_san.so")
    flags = [f for f in CFLAGS if f != "-O2"] + ["-O1", "-g", "-fno-omit-frame-pointer",
                                                 "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    subprocess.check_call(["gcc", *flags, _SRC, "-o", out, "-lm"])
    return out


def lib():
    global _lib
    if _lib is None:
        _lib = load(os.environ.get("KVQ_ORACLE_LIB") or build())
    return _lib


def compile_source(src: str, out: str) -> str:
    """Compile an oracle source file with the oracle's flags (used for mutant checks)."""
    subprocess.check_call(["gcc", *CFLAGS, src, "-o", out, "-lm"])
    return out


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------------------
# codec
# ---------------------------------------------------------------------------

def quant_group(x, bits: int, codec: int = 0):
    """Quantize one group (codec 0 asymmetric min-max, 1 symmetric).
    Returns (scale: np.float32, zero: np.float32, codes: uint8[m])."""
    x = _f32(x).ravel()
    m = x.size
    s = np.zeros(1, np.float32)
    z = np.zeros(1, np.float32)
    q = np.zeros(m, np.uint8)
    lib().orc_quant_group(_p(x), m, 1, bits, codec, _p(s), _p(z), _p(q), 1)
    return s[0], z[0], q


def quant_group_sparse(x, bits: int, codec: int = 0):
    """Dense-and-sparse group: (scale, zero, codes, outlier index); the outlier
    (largest magnitude, first among equals) is left out of the scale and zero."""
    x = _f32(x).ravel()
    m = x.size
    o = int(lib().orc_outlier_index(_p(x), m, 1))
    s = np.zeros(1, np.float32)
    z = np.zeros(1, np.float32)
    q = np.zeros(m, np.uint8)
    lib().orc_quant_group_skip(_p(x), m, 1, bits, codec, o, _p(s), _p(z), _p(q), 1)
    return s[0], z[0], q, o


def dequant(q, s, z) -> np.ndarray:
    """x' = (q - z) * s elementwise, one fp32 subtraction then one fp32 product."""
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty(q.shape, np.float32)
    f = lib().orc_dequant
    s = np.broadcast_to(np.asarray(s, np.float32), q.shape)
    z = np.broadcast_to(np.asarray(z, np.float32), q.shape)
    for idx in np.ndindex(q.shape):
        out[idx] = f(int(q[idx]), float(s[idx]), float(z[idx]))
    return out


# ---------------------------------------------------------------------------
# one slice of the cache
# ---------------------------------------------------------------------------

def quantized_count(m: int, residual: int, log_window: int = 0) -> int:
    """Quantized tokens of a slice holding m tokens past its sinks.

    Whole-residual flushes quantize residual tokens each time the residual fills;
    the log-sparse retention quantizes W of them once 3W are held, then W more
    after every further W tokens.
    """
    if log_window == 0:
        return residual * (m // residual)
    return 0 if m < residual else log_window * ((m - residual) // log_window + 1)


def build_slice(k_tok, v_tok, *, head_dim: int, bits: int, k_group: int, v_group: int,
                residual: int, n_sink: int, codec: int = 0, log_window: int = 0,
                outliers: int = 0, key_axis: int = 0) -> Dict[str, np.ndarray]:
    """Append the tokens of one (sequence, kv-head) one at a time; return the state.

    k_tok, v_tok: fp32 [n, D] (already rounded to the storage dtype).  codec: 0
    asymmetric min-max groups, 1 symmetric groups.  log_window W > 0: LogQuant's
    log-sparse retention with a full-precision part of residual = 3W tokens
    ("Resumo Técnico: LogQuant", Metodologia item 2); 0: the whole residual is
    quantized when it reaches residual tokens.  outliers = 1: KVQuant's per-vector
    dense-and-sparse quantization, one full-precision outlier per key channel
    group and per value group (ko_idx/ko_val [Lq/G, D], vo_idx/vo_val [Lq, D/GV]).
    """
    k_tok = _f32(k_tok)
    v_tok = _f32(v_tok)
    n, D = k_tok.shape
    assert D == head_dim and v_tok.shape == k_tok.shape
    S, R, G, GV = n_sink, residual, k_group, v_group
    nS = min(n, S)
    Lq = quantized_count(n - nS, R, log_window)
    nvg = D // GV
    kmeta = (Lq, 1) if key_axis else (Lq // G, D)
    st = dict(
        sink_k=np.zeros((S, D), np.float32), sink_v=np.zeros((S, D), np.float32),
        k_codes=np.zeros((Lq, D), np.uint8), k_scale=np.zeros(kmeta, np.float32),
        k_zero=np.zeros(kmeta, np.float32),
        v_codes=np.zeros((Lq, D), np.uint8), v_scale=np.zeros((Lq, nvg), np.float32),
        v_zero=np.zeros((Lq, nvg), np.float32),
        res_k=np.zeros((R, D), np.float32), res_v=np.zeros((R, D), np.float32),
        ko_idx=np.full((Lq // G, D), -1, np.int32), ko_val=np.zeros((Lq // G, D), np.float32),
        vo_idx=np.full((Lq, nvg), -1, np.int32), vo_val=np.zeros((Lq, nvg), np.float32))
    counts = np.zeros(4, np.int64)
    rc = lib().orc_build_slice(D, bits, codec, G, GV, R, S, log_window, outliers, key_axis, _p(k_tok), _p(v_tok), n,
                               _p(st["sink_k"]), _p(st["sink_v"]),
                               _p(st["k_codes"]), _p(st["k_scale"]), _p(st["k_zero"]),
                               _p(st["v_codes"]), _p(st["v_scale"]), _p(st["v_zero"]),
                               _p(st["res_k"]), _p(st["res_v"]),
                               _p(st["ko_idx"]), _p(st["ko_val"]), _p(st["vo_idx"]), _p(st["vo_val"]),
                               _p(counts))
    if rc != 0:
        raise ValueError("invalid oracle configuration")
    nS_, Lq_, r_, fl = (int(c) for c in counts)
    assert nS_ == nS and Lq_ == Lq
    st["sink_k"] = st["sink_k"][:nS_]
    st["sink_v"] = st["sink_v"][:nS_]
    st["res_k"] = st["res_k"][:r_]
    st["res_v"] = st["res_v"][:r_]
    st.update(n_sink=nS_, n_quant=Lq_, n_resid=r_, flushes=fl, head_dim=D, bits=bits,
              k_group=G, v_group=GV, residual=R, S=S, codec=codec, log_window=log_window,
              outliers=outliers, key_axis=key_axis)
    return st


def dequant_slice(st) -> tuple:
    """fp32 K', V' [nS+Lq+r, D] of a slice state in storage order (sinks, quantized, residual)."""
    D, G, GV = st["head_dim"], st["k_group"], st["v_group"]
    nS, Lq, r = st["n_sink"], st["n_quant"], st["n_resid"]
    T = nS + Lq + r
    ko = np.zeros((T, D), np.float32)
    vo = np.zeros((T, D), np.float32)
    arrs = [np.ascontiguousarray(st[k]) for k in
            ("sink_k", "sink_v", "k_codes", "k_scale", "k_zero", "v_codes", "v_scale",
             "v_zero", "res_k", "res_v")]
    sparse = [np.ascontiguousarray(st[k]) for k in ("ko_idx", "ko_val", "vo_idx", "vo_val")]
    lib().orc_dequant_slice(D, G, GV, int(st.get("key_axis", 0)), nS, Lq, r, *[_p(a) for a in arrs],
                            int(st.get("outliers", 0)),
                            *[_p(a) for a in sparse], _p(ko), _p(vo))
    return ko, vo


def attention(q, K, V, scale: float):
    """Binary64 softmax(scale q K^T) V for one query row; returns (out[D], lse)."""
    q = _f32(q).ravel()
    K = _f32(K)
    V = _f32(V)
    T, D = K.shape if K.size else (0, q.size)
    out = np.zeros(D, np.float64)
    lse = np.zeros(1, np.float64)
    lib().orc_attention(_p(q), _p(K), _p(V), T, D, float(scale), _p(out), _p(lse))
    return out, lse[0]


def default_scale(head_dim: int) -> float:
    return 1.0 / np.sqrt(np.float64(head_dim))


def decode_slices(states, q, scale: float):
    """One decode step for several slices that share (nS, Lq, r).

    states: list of slice states; q: fp32 [n, g, D].  Returns binary64
    (out [n, g, D], lse [n, g]).  Runs the slices on OpenMP threads.
    """
    n = len(states)
    st0 = states[0]
    D, G, GV = st0["head_dim"], st0["k_group"], st0["v_group"]
    nS, Lq, r = st0["n_sink"], st0["n_quant"], st0["n_resid"]
    q = _f32(q)
    g = q.shape[1]

    def stack(key):
        return np.ascontiguousarray(np.stack([s[key] for s in states]))

    arrs = [stack(k) for k in ("sink_k", "sink_v", "k_codes", "k_scale", "k_zero",
                                "v_codes", "v_scale", "v_zero", "res_k", "res_v")]
    sparse = [stack(k) for k in ("ko_idx", "ko_val", "vo_idx", "vo_val")]
    out = np.zeros((n, g, D), np.float64)
    lse = np.zeros((n, g), np.float64)
    lib().orc_decode_slices(n, g, D, G, GV, int(st0.get("key_axis", 0)), nS, Lq, r, float(scale),
                            *[_p(a) for a in arrs],
                            int(st0.get("outliers", 0)), *[_p(a) for a in sparse],
                            _p(q), _p(out), _p(lse))
    return out, lse


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel regions (for timing it on fewer cores)."""
    lib().orc_set_num_threads(int(n))


# ---------------------------------------------------------------------------
# whole-workload helpers (one slice at a time)
# ---------------------------------------------------------------------------

def slice_tokens_f32(w, b: int, kvh: int, n_steps: int):
    """fp32 (storage-rounded) tokens of a slice: prefill followed by n_steps step tokens."""
    import workloads as wl
    kp, vp = wl.prefill_slice(w, b, kvh)
    n0 = wl.prefill_lengths(w)[b]
    kp, vp = kp[:n0], vp[:n0]
    k = wl.storage_to_f32(kp, w.dtype)
    v = wl.storage_to_f32(vp, w.dtype)
    if n_steps:
        ks, vs = wl.step_slice(w, b, kvh)
        k = np.concatenate([k, wl.storage_to_f32(ks[:n_steps], w.dtype)])
        v = np.concatenate([v, wl.storage_to_f32(vs[:n_steps], w.dtype)])
    return k, v


def slice_state(w, b: int, kvh: int, n_steps: int):
    """Oracle cache state of slice (b, kvh) after the prefill and n_steps appends."""
    k, v = slice_tokens_f32(w, b, kvh, n_steps)
    return build_slice(k, v, head_dim=w.head_dim, bits=w.bits, k_group=w.k_group,
                       v_group=w.v_group, residual=w.residual, n_sink=w.n_sink, codec=w.codec,
                       log_window=w.log_window, outliers=w.outliers, key_axis=w.key_axis)


def expected_outputs(w, b: int, kvh: int, n_steps: int, qi: int, scale: float | None = None):
    """Binary64 outputs of query index qi for every query head of kv-head kvh.

    Returns (out [g, D], lse [g]) for the state after the prefill and n_steps appends.
    """
    import workloads as wl
    st = slice_state(w, b, kvh, n_steps)
    K, V = dequant_slice(st)
    scale = default_scale(w.head_dim) if scale is None else scale
    g = w.gqa
    out = np.zeros((g, w.head_dim))
    lse = np.zeros(g)
    for j in range(g):
        hq = kvh * g + j
        q = wl.storage_to_f32(wl.query_slice(w, b, hq)[qi], w.dtype)
        out[j], lse[j] = attention(q, K, V, scale)
    return out, lse
