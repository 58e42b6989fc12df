"""Seeded synthetic inputs for low-bit KV-cache decode attention.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle.  It holds shapes, schedules and random draws only: no quantization,
no attention, nothing of the method's arithmetic.  Every draw comes from a
numpy PCG64 stream keyed by (config seed, purpose, indices), so any single
(batch, kv-head) slice can be regenerated on its own without generating the
rest of the batch.

Workload shapes follow the decode settings the pages study: a Llama-7B-shaped
MHA decode, the KIVI 2-bit setting, long-context GQA, and a long-context cache
with full-precision attention-sink tokens (KIVI notes, section 1; Atom review,
runtime-breakdown figure; LogQuant summary, problem statement).  No page gives
a dataset item or trained weights; the value distributions below (Gaussian
keys/values with per-channel key outliers, channel offsets, large-norm sink
tokens) stand in for the real activations those pages measure.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Iterator, Tuple

import numpy as np

# purposes used as the second word of every seed key
_P_OUTLIER = 1
_P_OFFSET = 2
_P_PREFILL_K = 3
_P_PREFILL_V = 4
_P_STEP_KV = 5
_P_QUERY = 6


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, codec parameters and decode schedule of one synthetic workload."""

    name: str
    description: str
    batch: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    dtype: str            # "f32" | "bf16" | "f16": K/V/q storage type
    bits: int             # 2 or 4
    k_group: int          # G: tokens per per-channel key group
    v_group: int          # G_V: channels per per-token value group
    residual: int         # R: full-precision residual capacity
    n_sink: int           # S: leading tokens kept at full precision
    prefill: int          # tokens appended in bulk before decoding
    steps: int            # decode steps (append one token, then attend)
    attend_after_prefill: bool  # one extra attention call right after prefill
    seed: int
    k_outlier_channels: int = 0     # channels per kv-head scaled as outliers
    k_outlier_scale: float = 1.0
    k_offset_range: float = 0.0     # per-(kv-head, channel) key mean ~ U(-a, a)
    sink_scale: float = 1.0         # K and V scale of the first n_sink tokens
    codec: int = 0                  # 0 asymmetric min-max groups, 1 symmetric groups
    prefill_min_frac: float = 1.0   # sequence b prefills prefill * (1 - (1 - f) b / (B - 1)) tokens
    log_window: int = 0             # W > 0: log-sparse full-precision retention, residual = 3W
    page_groups: int = 0            # P > 0: quantized records in pages of P key groups
    prefill_chunk: int = 0          # prefill in rounds of this many tokens per sequence (0: at once)
    outliers: int = 0               # 1: one full-precision outlier per quantization vector
    key_axis: int = 0               # 0: keys per channel over G tokens; 1: per token over D channels

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_tokens(self) -> int:
        return self.prefill + self.steps

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        name="tiny",
        description="tiny single-head decode: B1 H1 D64, 256 cached tokens, fp32, "
                    "INT4 G32 / G_V64, R32, 40 appended tokens (one flush)",
        batch=1, n_kv_heads=1, n_q_heads=1, head_dim=64, dtype="f32",
        bits=4, k_group=32, v_group=64, residual=32, n_sink=0,
        prefill=256, steps=40, attend_after_prefill=True, seed=1001,
        k_outlier_channels=2, k_outlier_scale=10.0),
    "llama7b_mha_int4": Workload(
        name="llama7b_mha_int4",
        description="Llama-7B-shaped MHA decode: B8 H32 D128, context 4096, bf16, "
                    "INT4 G128 / G_V128, R128, 64 decode steps",
        batch=8, n_kv_heads=32, n_q_heads=32, head_dim=128, dtype="bf16",
        bits=4, k_group=128, v_group=128, residual=128, n_sink=0,
        prefill=4096, steps=64, attend_after_prefill=False, seed=1002,
        k_outlier_channels=4, k_outlier_scale=8.0),
    "kivi2_long_batch": Workload(
        name="kivi2_long_batch",
        description="KIVI-style 2-bit long-batch decode: B32 H32 D128, context 8192, "
                    "bf16, INT2 G32 / G_V32, R128, 32 decode steps",
        batch=32, n_kv_heads=32, n_q_heads=32, head_dim=128, dtype="bf16",
        bits=2, k_group=32, v_group=32, residual=128, n_sink=0,
        prefill=8192, steps=32, attend_after_prefill=False, seed=1003,
        k_outlier_channels=4, k_outlier_scale=10.0),
    "gqa_32k_int4": Workload(
        name="gqa_32k_int4",
        description="GQA decode: B16, 32 query heads on 8 KV heads, D128, context "
                    "32768, bf16, INT4 G128 / G_V128, R128, 16 decode steps",
        batch=16, n_kv_heads=8, n_q_heads=32, head_dim=128, dtype="bf16",
        bits=4, k_group=128, v_group=128, residual=128, n_sink=0,
        prefill=32768, steps=16, attend_after_prefill=False, seed=1004,
        k_offset_range=3.0),
    "long_128k_sink_int2": Workload(
        name="long_128k_sink_int2",
        description="long-context mixed precision: B1, 32 query / 8 KV heads, D128, "
                    "context 131072, bf16, 4 sink tokens (x20 norm) and a 256-token "
                    "residual kept bf16, INT2 G64 / G_V64, 8 decode steps",
        batch=1, n_kv_heads=8, n_q_heads=32, head_dim=128, dtype="bf16",
        bits=2, k_group=64, v_group=64, residual=256, n_sink=4,
        prefill=131072, steps=8, attend_after_prefill=False, seed=1005,
        sink_scale=20.0),
    "llama7b_mha_int4_sym": Workload(
        name="llama7b_mha_int4_sym",
        description="the Llama-7B-shaped MHA decode with symmetric INT4 groups: B8 H32 D128, "
                    "context 4096, bf16, G128 / G_V128, R128, 64 decode steps",
        batch=8, n_kv_heads=32, n_q_heads=32, head_dim=128, dtype="bf16",
        bits=4, k_group=128, v_group=128, residual=128, n_sink=0,
        prefill=4096, steps=64, attend_after_prefill=False, seed=1002,
        k_outlier_channels=4, k_outlier_scale=8.0, codec=1),
    "llama7b_mha_int4_ragged": Workload(
        name="llama7b_mha_int4_ragged",
        description="the Llama-7B-shaped MHA decode on sequences of different lengths: B8 H32 "
                    "D128, contexts 4096 down to 2048 (evenly spaced), bf16, INT4 G128 / G_V128, "
                    "R128, 64 decode steps",
        batch=8, n_kv_heads=32, n_q_heads=32, head_dim=128, dtype="bf16",
        bits=4, k_group=128, v_group=128, residual=128, n_sink=0,
        prefill=4096, steps=64, attend_after_prefill=False, seed=1002,
        k_outlier_channels=4, k_outlier_scale=8.0, prefill_min_frac=0.5),
    "llama7b_mha_int8": Workload(
        name="llama7b_mha_int8",
        description="the Llama-7B-shaped MHA decode with INT8 groups (a layer kept at 8 bits "
                    "in per-layer mixed precision): B8 H32 D128, context 4096, bf16, "
                    "G128 / G_V128, R128, 64 decode steps",
        batch=8, n_kv_heads=32, n_q_heads=32, head_dim=128, dtype="bf16",
        bits=8, k_group=128, v_group=128, residual=128, n_sink=0,
        prefill=4096, steps=64, attend_after_prefill=False, seed=1002,
        k_outlier_channels=4, k_outlier_scale=8.0),
    "llama7b_mha_int4_paged": Workload(
        name="llama7b_mha_int4_paged",
        description="the ragged Llama-7B-shaped MHA decode on paged records: B8 H32 D128, contexts "
                    "4096 down to 2048, bf16, INT4 G128 / G_V128, R128, pages of 4 key groups (512 "
                    "tokens) from a pool sized to the sequences, prefilled in 512-token rounds so "
                    "that the sequences' pages interleave, 64 decode steps",
        batch=8, n_kv_heads=32, n_q_heads=32, head_dim=128, dtype="bf16",
        bits=4, k_group=128, v_group=128, residual=128, n_sink=0,
        prefill=4096, steps=64, attend_after_prefill=False, seed=1002,
        k_outlier_channels=4, k_outlier_scale=8.0, prefill_min_frac=0.5,
        page_groups=4, prefill_chunk=512),
    "llama7b_mha_int4_outliers": Workload(
        name="llama7b_mha_int4_outliers",
        description="the Llama-7B-shaped MHA decode with dense-and-sparse groups (one full-precision "
                    "outlier per key channel group and per value group): B8 H32 D128, context 4096, "
                    "bf16, INT4 G128 / G_V128, R128, 64 decode steps",
        batch=8, n_kv_heads=32, n_q_heads=32, head_dim=128, dtype="bf16",
        bits=4, k_group=128, v_group=128, residual=128, n_sink=0,
        prefill=4096, steps=64, attend_after_prefill=False, seed=1002,
        k_outlier_channels=4, k_outlier_scale=8.0, outliers=1),
    "gqa_32k_int4_outliers": Workload(
        name="gqa_32k_int4_outliers",
        description="the GQA decode with dense-and-sparse groups (one full-precision outlier per key "
                    "channel group and per value group): B16, 32 query heads on 8 KV heads, D128, "
                    "context 32768, bf16, INT4 G128 / G_V128, R128, 16 decode steps",
        batch=16, n_kv_heads=8, n_q_heads=32, head_dim=128, dtype="bf16",
        bits=4, k_group=128, v_group=128, residual=128, n_sink=0,
        prefill=32768, steps=16, attend_after_prefill=False, seed=1004,
        k_offset_range=3.0, outliers=1),
    "llama7b_mha_int4_headgran": Workload(
        name="llama7b_mha_int4_headgran",
        description="the Llama-7B-shaped MHA decode with head-granular groups (Atom's KV-cache "
                    "quantization: each token's key and value one asymmetric group over the head's "
                    "128 channels): B8 H32 D128, context 4096, bf16, INT4, records of 128 tokens, "
                    "R128, 64 decode steps",
        batch=8, n_kv_heads=32, n_q_heads=32, head_dim=128, dtype="bf16",
        bits=4, k_group=128, v_group=128, residual=128, n_sink=0,
        prefill=4096, steps=64, attend_after_prefill=False, seed=1002,
        k_outlier_channels=4, k_outlier_scale=8.0, key_axis=1),
    "logquant_gqa_int2": Workload(
        name="logquant_gqa_int2",
        description="Llama-3.1-8B-shaped GQA decode with LogQuant's log-sparse retention: B8, "
                    "32 query / 8 KV heads, D128, context 32768, bf16, INT2 G64 / G_V64, "
                    "full-precision reserve 3W = 192 tokens (W = 64), 64 decode steps",
        batch=8, n_kv_heads=8, n_q_heads=32, head_dim=128, dtype="bf16",
        bits=2, k_group=64, v_group=64, residual=192, n_sink=0,
        prefill=32768, steps=64, attend_after_prefill=False, seed=1006,
        k_outlier_channels=4, k_outlier_scale=8.0, log_window=64),
}

# short aliases in the order the workloads are listed
ALIASES = {"C1": "tiny", "C2": "llama7b_mha_int4", "C3": "kivi2_long_batch",
           "C4": "gqa_32k_int4", "C5": "long_128k_sink_int2"}


def get(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


def prefill_lengths(w: Workload) -> list:
    """Prefill tokens of each sequence: w.prefill for all, or evenly spaced from
    w.prefill down to w.prefill * w.prefill_min_frac.  Sequence b's prefill is the
    first prefill_lengths(w)[b] rows of its prefill draw."""
    if w.prefill_min_frac == 1.0 or w.batch == 1:
        return [w.prefill] * w.batch
    return [int(round(w.prefill * (1.0 - (1.0 - w.prefill_min_frac) * b / (w.batch - 1))))
            for b in range(w.batch)]


def prefill_rounds(w: Workload) -> list:
    """The prefill as rounds of (first token, tokens of each sequence): one round of
    prefill_lengths(w), or, with prefill_chunk, rounds of up to prefill_chunk
    tokens per sequence (a serving engine taking prompts a chunk at a time)."""
    lens = prefill_lengths(w)
    if not w.prefill_chunk:
        return [(0, lens)]
    return [(t0, [max(0, min(w.prefill_chunk, n - t0)) for n in lens])
            for t0 in range(0, max(lens), w.prefill_chunk)]


# --------------------------------------------------------------------------
# rounding of fp32 draws to the storage dtype (input preparation only)
# --------------------------------------------------------------------------

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest even.  Finite input."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # no uint32 overflow for finite inputs: the largest finite pattern is 0xff7fffff
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values -> storage array (f32: float32, bf16: uint16 bits, f16: float16)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16_bits(x)
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
    raise ValueError(dtype)


def storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a storage array to fp32."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(a)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float32)
    raise ValueError(dtype)


def storage_np_dtype(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16, "f16": np.float16}[dtype]


def elem_bytes(dtype: str) -> int:
    return {"f32": 4, "bf16": 2, "f16": 2}[dtype]


# --------------------------------------------------------------------------
# per-slice structure and draws
# --------------------------------------------------------------------------

def _rng(w: Workload, *key: int) -> np.random.Generator:
    return np.random.default_rng([w.seed, *key])


def outlier_channels(w: Workload, kvh: int) -> np.ndarray:
    """Key outlier channels of one kv-head (shared by every sequence)."""
    if w.k_outlier_channels == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(w, _P_OUTLIER, kvh).choice(w.head_dim, w.k_outlier_channels,
                                                   replace=False))


def channel_offsets(w: Workload, kvh: int) -> np.ndarray:
    """Per-channel key mean offsets of one kv-head (shared by every sequence)."""
    if w.k_offset_range == 0.0:
        return np.zeros(w.head_dim, dtype=np.float32)
    a = w.k_offset_range
    return _rng(w, _P_OFFSET, kvh).uniform(-a, a, w.head_dim).astype(np.float32)


def _shape_keys(w: Workload, kvh: int, k: np.ndarray) -> np.ndarray:
    ch = outlier_channels(w, kvh)
    if ch.size:
        k[:, ch] *= np.float32(w.k_outlier_scale)
    if w.k_offset_range:
        k += channel_offsets(w, kvh)[None, :]
    return k


def prefill_slice_f32(w: Workload, b: int, kvh: int, n: int | None = None
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """fp32 draws (before storage rounding) of the prefill tokens of one slice.

    Returns K, V of shape [n, D].  Token positions 0..n_sink-1 carry the sink
    scale on both K and V.
    """
    n = w.prefill if n is None else n
    D = w.head_dim
    k = _rng(w, _P_PREFILL_K, b, kvh).standard_normal((n, D), dtype=np.float32)
    v = _rng(w, _P_PREFILL_V, b, kvh).standard_normal((n, D), dtype=np.float32)
    k = _shape_keys(w, kvh, k)
    s = min(w.n_sink, n)
    if s and w.sink_scale != 1.0:
        k[:s] *= np.float32(w.sink_scale)
        v[:s] *= np.float32(w.sink_scale)
    return k, v


def step_slice_f32(w: Workload, b: int, kvh: int) -> Tuple[np.ndarray, np.ndarray]:
    """fp32 draws of the tokens appended at decode steps 0..steps-1: [steps, D] each."""
    D = w.head_dim
    g = _rng(w, _P_STEP_KV, b, kvh)
    kv = g.standard_normal((w.steps, 2, D), dtype=np.float32)
    k = _shape_keys(w, kvh, np.ascontiguousarray(kv[:, 0]))
    v = np.ascontiguousarray(kv[:, 1])
    return k, v


def n_queries(w: Workload) -> int:
    return w.steps + (1 if w.attend_after_prefill else 0)


def query_f32(w: Workload, b: int, hq: int) -> np.ndarray:
    """fp32 draws of every query of one (sequence, query head): [n_queries, D]."""
    return _rng(w, _P_QUERY, b, hq).standard_normal((n_queries(w), w.head_dim),
                                                     dtype=np.float32)


# storage-rounded views (what both the HIP path and the oracle consume)

def prefill_slice(w: Workload, b: int, kvh: int, n: int | None = None):
    k, v = prefill_slice_f32(w, b, kvh, n)
    return to_storage(k, w.dtype), to_storage(v, w.dtype)


def step_slice(w: Workload, b: int, kvh: int):
    k, v = step_slice_f32(w, b, kvh)
    return to_storage(k, w.dtype), to_storage(v, w.dtype)


def query_slice(w: Workload, b: int, hq: int):
    return to_storage(query_f32(w, b, hq), w.dtype)


def _each_slice(fn, pairs) -> None:
    """fn(pair) for every pair, on a pool of threads (numpy's generators release the
    GIL); every slice has its own generator, so the values do not depend on the
    order.  At most 16 threads."""
    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(fn, pairs))


def prefill_batch(w: Workload, n: int | None = None):
    """Storage arrays K, V [B, Hkv, n, D] of the whole prefill (slice by slice)."""
    n = w.prefill if n is None else n
    dt = storage_np_dtype(w.dtype)
    K = np.empty((w.batch, w.n_kv_heads, n, w.head_dim), dtype=dt)
    V = np.empty_like(K)

    def fill(p):
        K[p[0], p[1]], V[p[0], p[1]] = prefill_slice(w, p[0], p[1], n)

    _each_slice(fill, [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)])
    return K, V


def steps_batch(w: Workload):
    """Storage arrays K, V [steps, B, Hkv, D] of the decode-step tokens."""
    dt = storage_np_dtype(w.dtype)
    K = np.empty((w.steps, w.batch, w.n_kv_heads, w.head_dim), dtype=dt)
    V = np.empty_like(K)

    def fill(p):
        K[:, p[0], p[1]], V[:, p[0], p[1]] = step_slice(w, p[0], p[1])

    _each_slice(fill, [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)])
    return K, V


def queries_batch(w: Workload):
    """Storage array Q [n_queries, B, Hq, D]."""
    dt = storage_np_dtype(w.dtype)
    Q = np.empty((n_queries(w), w.batch, w.n_q_heads, w.head_dim), dtype=dt)

    def fill(p):
        Q[:, p[0], p[1]] = query_slice(w, p[0], p[1])

    _each_slice(fill, [(b, h) for b in range(w.batch) for h in range(w.n_q_heads)])
    return Q


def schedule(w: Workload) -> Iterator[Tuple[str, int]]:
    """The decode schedule after the bulk prefill: ("attend", qi) / ("append", step)."""
    qi = 0
    if w.attend_after_prefill:
        yield ("attend", qi)
        qi += 1
    for s in range(w.steps):
        yield ("append", s)
        yield ("attend", qi)
        qi += 1


def random_tokens(seed: int, shape, dtype: str, scale: float = 1.0, offset: float = 0.0):
    """Generic seeded N(offset, scale^2) draws rounded to the storage dtype (tests)."""
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    x = x * np.float32(scale) + np.float32(offset)
    return to_storage(x, dtype)
