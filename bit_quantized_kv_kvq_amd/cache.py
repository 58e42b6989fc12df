"""torch-facing wrapper: one low-bit KV cache with torch-owned device buffers.

torch allocates the cache buffer, the decode workspace and the outputs, and
supplies the current HIP stream; the library's kernels do all of the work.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import torch

import bit_quantized_kv_kvq_amd as _k


def torch_dtype_code(dt: torch.dtype) -> int:
    return {torch.float32: _k.KVQ_F32, torch.bfloat16: _k.KVQ_BF16,
            torch.float16: _k.KVQ_F16}[dt]


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


class Cache:
    """A KIVI-style low-bit KV cache for `batch` sequences of uniform length.

    Keys are quantized per channel over groups of `k_group` tokens, values per
    token over groups of `v_group` channels, with `bits`-bit asymmetric min-max
    codes; the newest tokens stay in a full-precision residual of `residual`
    tokens and the first `n_sink` tokens stay full precision for good.
    `retention` = KVQ_RETAIN_LOG selects LogQuant's log-sparse retention
    (residual = 3W): a flush quantizes every other token of the oldest 2W.
    `page_groups` > 0 keeps the quantized records in pages of that many key
    groups from a pool of `pool_pages` pages (0: one per sequence at capacity).
    `outliers` = 1 keeps one full-precision outlier per quantization vector
    (KVQuant's dense-and-sparse groups).  `key_axis` = KVQ_KEY_PER_TOKEN groups
    each token's key over its head_dim channels (Atom's head granularity).
    """

    def __init__(self, *, batch: int, n_kv_heads: int, n_q_heads: int, head_dim: int, bits: int,
                 k_group: int, v_group: int, residual: int, max_tokens: int, n_sink: int = 0,
                 dtype: torch.dtype = torch.bfloat16, sm_scale: float = 0.0,
                 device: Optional[torch.device] = None, codec: int = 0, retention: int = 0,
                 page_groups: int = 0, pool_pages: int = 0, outliers: int = 0, key_axis: int = 0):
        _k.lib()
        self.device = torch.device(device or "cuda")
        self.dtype = dtype
        self.cfg = _k.make_config(batch=batch, n_kv_heads=n_kv_heads, n_q_heads=n_q_heads,
                                  head_dim=head_dim, bits=bits, k_group=k_group, v_group=v_group,
                                  residual=residual, n_sink=n_sink, dtype=torch_dtype_code(dtype),
                                  max_tokens=max_tokens, sm_scale=sm_scale, codec=codec,
                                  retention=retention, page_groups=page_groups, pool_pages=pool_pages,
                                  outliers=outliers, key_axis=key_axis)
        self.nbytes = _k.kvq_cache_bytes(self.cfg)
        # over-allocate by 256 bytes so the handle's buffer is 256-byte aligned
        self._buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=self.device)
        ptr = self._buf.data_ptr()
        self._base = ptr + (-ptr) % 256
        self.handle = None
        with torch.cuda.device(self.device):
            self.handle = _k.kvq_cache_create(self.cfg, self._base, self.nbytes)
        self.ws_bytes = _k.kvq_decode_workspace_bytes(self.handle)
        # counters must start at zero; every decode call leaves them at zero
        self._ws = torch.zeros(self.ws_bytes + 256, dtype=torch.uint8, device=self.device)
        wp = self._ws.data_ptr()
        self._ws_ptr = wp + (-wp) % 256

    # -- properties --------------------------------------------------------
    @property
    def batch(self):
        return self.cfg.batch

    @property
    def n_kv_heads(self):
        return self.cfg.n_kv_heads

    @property
    def n_q_heads(self):
        return self.cfg.n_q_heads

    @property
    def head_dim(self):
        return self.cfg.head_dim

    def state(self) -> Tuple[int, int, int, int]:
        """(n_tokens, n_sink, n_quant, n_resid) per sequence."""
        return _k.kvq_cache_state(self.handle)

    # -- calls -------------------------------------------------------------
    def _check_tokens(self, x: torch.Tensor, name: str):
        c = self.cfg
        if x.dtype != self.dtype or x.device != self.device or not x.is_contiguous():
            raise ValueError("%s must be a contiguous %s tensor on %s" % (name, self.dtype, self.device))
        if x.dim() != 4 or x.shape[0] != c.batch or x.shape[1] != c.n_kv_heads or x.shape[3] != c.head_dim:
            raise ValueError("%s must have shape [B, Hkv, n, D], got %s" % (name, tuple(x.shape)))

    def append(self, k: torch.Tensor, v: torch.Tensor):
        """Append n tokens: k, v [B, Hkv, n, D] in the cache dtype."""
        self._check_tokens(k, "k")
        self._check_tokens(v, "v")
        if k.shape != v.shape:
            raise ValueError("k and v shapes differ")
        _k.kvq_append(self.handle, k.data_ptr(), v.data_ptr(), k.shape[2], _stream())

    def append_ragged(self, k: torch.Tensor, v: torch.Tensor, n_new):
        """Append n_new[b] tokens to sequence b: k, v [B, Hkv, n_max, D] in the cache
        dtype (rows past n_new[b] are not read); n_new: B ints in [0, n_max]."""
        self._check_tokens(k, "k")
        self._check_tokens(v, "v")
        if k.shape != v.shape:
            raise ValueError("k and v shapes differ")
        if len(n_new) != self.cfg.batch:
            raise ValueError("n_new needs one count per sequence")
        _k.kvq_append_ragged(self.handle, k.data_ptr(), v.data_ptr(), list(n_new), k.shape[2], _stream())

    def seq_lengths(self):
        """Tokens held by each sequence (host-side)."""
        return _k.kvq_seq_lengths(self.handle, self.cfg.batch)

    def release_sequence(self, b: int):
        """Empty sequence b and return its pages to the pool."""
        _k.kvq_release_sequence(self.handle, b, _stream())

    def free_pages(self) -> int:
        """Free pages of the pool (paged records)."""
        return _k.kvq_pool_free_pages(self.handle)

    def decode(self, q: torch.Tensor, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, with_lse: bool = True):
        """Attention of q [B, Hq, D] over the cache -> (out fp32 [B, Hq, D], lse fp32 [B, Hq])."""
        c = self.cfg
        if q.dtype != self.dtype or q.device != self.device or not q.is_contiguous() or \
                tuple(q.shape) != (c.batch, c.n_q_heads, c.head_dim):
            raise ValueError("q must be a contiguous [B, Hq, D] %s tensor" % self.dtype)
        if out is None:
            out = torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32,
                              device=self.device)
        if lse is None and with_lse:
            lse = torch.empty((c.batch, c.n_q_heads), dtype=torch.float32, device=self.device)
        _k.kvq_decode_attention(self.handle, q.data_ptr(), out.data_ptr(),
                                lse.data_ptr() if lse is not None else 0, self._ws_ptr,
                                self.ws_bytes, _stream())
        return out, lse

    def append_decode(self, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      with_lse: bool = True):
        """One decode step: append one token per sequence (k, v [B, Hkv, 1, D]), then
        attention of q [B, Hq, D] over the cache, in one library call."""
        c = self.cfg
        self._check_tokens(k, "k")
        self._check_tokens(v, "v")
        if k.shape[2] != 1 or v.shape[2] != 1:
            raise ValueError("append_decode appends exactly one token per sequence")
        if q.dtype != self.dtype or q.device != self.device or not q.is_contiguous() or \
                tuple(q.shape) != (c.batch, c.n_q_heads, c.head_dim):
            raise ValueError("q must be a contiguous [B, Hq, D] %s tensor" % self.dtype)
        if out is None:
            out = torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32,
                              device=self.device)
        if lse is None and with_lse:
            lse = torch.empty((c.batch, c.n_q_heads), dtype=torch.float32, device=self.device)
        _k.kvq_append_decode(self.handle, k.data_ptr(), v.data_ptr(), q.data_ptr(), out.data_ptr(),
                             lse.data_ptr() if lse is not None else 0, self._ws_ptr, self.ws_bytes,
                             _stream())
        return out, lse

    def dequantize(self) -> Tuple[torch.Tensor, torch.Tensor]:
        """fp32 K', V' [B, Hkv, n_tokens, D] in storage order (sinks, quantized, residual)."""
        c = self.cfg
        T = self.state()[0]
        # zero-filled: rows past a shorter sequence's own length are not written
        k = torch.zeros((c.batch, c.n_kv_heads, T, c.head_dim), dtype=torch.float32,
                        device=self.device)
        v = torch.zeros_like(k)
        _k.kvq_dequantize(self.handle, k.data_ptr(), v.data_ptr(), _stream())
        return k, v

    def export(self) -> Dict[str, torch.Tensor]:
        """Canonical unpacked codes and fp32 scales / zero points of the quantized part."""
        c = self.cfg
        Lq = self.state()[2]
        dev = self.device
        out = dict(
            k_codes=torch.zeros((c.batch, c.n_kv_heads, Lq, c.head_dim), dtype=torch.uint8, device=dev),
            k_scale=torch.zeros((c.batch, c.n_kv_heads, Lq, 1) if c.key_axis else
                                (c.batch, c.n_kv_heads, Lq // c.k_group, c.head_dim),
                                dtype=torch.float32, device=dev),
            v_codes=torch.zeros((c.batch, c.n_kv_heads, Lq, c.head_dim), dtype=torch.uint8, device=dev),
            v_scale=torch.zeros((c.batch, c.n_kv_heads, Lq, c.head_dim // c.v_group),
                                dtype=torch.float32, device=dev))
        out["k_zero"] = torch.zeros_like(out["k_scale"])
        out["v_zero"] = torch.zeros_like(out["v_scale"])
        ptrs = [out[n].data_ptr() if out[n].numel() else 0
                for n in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero")]
        _k.kvq_export(self.handle, ptrs, _stream())
        return out

    def export_outliers(self) -> Dict[str, torch.Tensor]:
        """Outliers of dense-and-sparse records: k_idx / k_val [B, Hkv, Lq / G, D] (token
        within the key group, exact value), v_idx / v_val [B, Hkv, Lq, D / G_V] (channel
        within the value group, exact value)."""
        c = self.cfg
        Lq = self.state()[2]
        dev = self.device
        nk = (c.batch, c.n_kv_heads, Lq // c.k_group, c.head_dim)
        nv = (c.batch, c.n_kv_heads, Lq, c.head_dim // c.v_group)
        out = dict(k_idx=torch.zeros(nk, dtype=torch.uint8, device=dev),
                   k_val=torch.zeros(nk, dtype=torch.float32, device=dev),
                   v_idx=torch.zeros(nv, dtype=torch.uint8, device=dev),
                   v_val=torch.zeros(nv, dtype=torch.float32, device=dev))
        ptrs = [out[n].data_ptr() if out[n].numel() else 0 for n in ("k_idx", "k_val", "v_idx", "v_val")]
        _k.kvq_export_outliers(self.handle, *ptrs, _stream())
        return out

    def set_split_tokens(self, n: int):
        _k.kvq_set_split_tokens(self.handle, n)

    def set_timing_events(self, start_event, stop_event):
        """Record hipEvent_t handles at the start and end of every later decode kernel
        of this cache (None, None stops)."""
        _k.kvq_set_timing_events(self.handle, start_event, stop_event)

    def close(self):
        if self.handle is not None:
            _k.kvq_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
