"""GPU tests of paged quantized records, through the C-ABI.

Records live in pages of P key groups taken from a pool as sequences grow and
located through a page table (the page-table management of a serving KV cache
in "Atom: Low-bit Quantization for Efficient and Accurate LLM Serving",
runtime-breakdown figure and baselines).  Storage is all that changes, so a
paged cache must give bitwise the outputs, exports and dequantized rows of a
contiguous cache fed the same tokens, and match the oracle slice by slice.
"""
import numpy as np
import pytest
import torch

import bit_quantized_kv_kvq_amd as kvq
import oracle
import workloads as wl
from tests.gpu_common import ATOL, export_cpu, gpu, log, make_cache, require_gpu
from workloads.torch_io import to_torch

pytestmark = gpu

DEV = torch.device("cuda:0")


def _w(**kw):
    base = wl.get("C2").replace(name="paged", batch=4, n_kv_heads=2, n_q_heads=2, prefill=0,
                                steps=0, k_group=32, v_group=32, residual=64)
    return base.replace(**kw)


def _tokens(w, n, seed, scale=1.0):
    return wl.random_tokens(seed, (w.batch, w.n_kv_heads, n, w.head_dim), w.dtype, scale)


class Twin:
    """A paged and a contiguous cache fed the same calls, and a host copy of every
    sequence's tokens for the oracle."""

    def __init__(self, w, max_tokens, page_groups, pool_pages=0):
        self.w = w
        self.paged = make_cache(w, max_tokens=max_tokens, page_groups=page_groups, pool_pages=pool_pages)
        self.flat = make_cache(w, max_tokens=max_tokens)
        empty = _tokens(w, 0, 0)
        self.k = [[empty[b, h] for h in range(w.n_kv_heads)] for b in range(w.batch)]
        self.v = [[empty[b, h] for h in range(w.n_kv_heads)] for b in range(w.batch)]

    def append_ragged(self, n_new, seed):
        w = self.w
        n_max = max(max(n_new), 1)
        K, V = _tokens(w, n_max, seed, 2.0), _tokens(w, n_max, seed + 1)
        kt, vt = to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV)
        for c in (self.paged, self.flat):
            c.append_ragged(kt, vt, n_new)
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                self.k[b][h] = np.concatenate([self.k[b][h], K[b, h, :n_new[b]]])
                self.v[b][h] = np.concatenate([self.v[b][h], V[b, h, :n_new[b]]])

    def step(self, seed):
        """One token to every sequence, then attention; returns (q, out, lse) of the paged
        cache after checking that the contiguous one gives the same bits."""
        w = self.w
        k1, v1 = _tokens(w, 1, seed), _tokens(w, 1, seed + 1)
        q = wl.random_tokens(seed + 2, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
        args = [to_torch(x, w.dtype, DEV) for x in (k1, v1, q)]
        o1, l1 = self.paged.append_decode(*args)
        o2, l2 = self.flat.append_decode(*args)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                self.k[b][h] = np.concatenate([self.k[b][h], k1[b, h]])
                self.v[b][h] = np.concatenate([self.v[b][h], v1[b, h]])
        return q, o1, l1

    def release(self, b):
        for c in (self.paged, self.flat):
            c.release_sequence(b)
        for h in range(self.w.n_kv_heads):
            self.k[b][h] = self.k[b][h][:0]
            self.v[b][h] = self.v[b][h][:0]

    def state(self, b, h):
        w = self.w
        return oracle.build_slice(wl.storage_to_f32(self.k[b][h], w.dtype), wl.storage_to_f32(self.v[b][h], w.dtype),
                                  head_dim=w.head_dim, bits=w.bits, k_group=w.k_group, v_group=w.v_group,
                                  residual=w.residual, n_sink=w.n_sink, codec=w.codec,
                                  log_window=w.log_window)

    def check(self, q, out, lse):
        """Exports and dequantized rows of the two caches equal; the paged one against the oracle."""
        w = self.w
        ep, ef = export_cpu(self.paged), export_cpu(self.flat)
        for name in ep:
            np.testing.assert_array_equal(ep[name], ef[name], err_msg=name)
        Kp, Vp = self.paged.dequantize()
        Kf, Vf = self.flat.dequantize()
        torch.cuda.synchronize()
        assert torch.equal(Kp, Kf) and torch.equal(Vp, Vf)
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
        qf = wl.storage_to_f32(q, w.dtype)
        scale = oracle.default_scale(w.head_dim)
        err = 0.0
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                st = self.state(b, h)
                Lq = st["n_quant"]
                np.testing.assert_array_equal(ep["k_codes"][b, h, :Lq], st["k_codes"])
                np.testing.assert_array_equal(ep["v_codes"][b, h, :Lq], st["v_codes"])
                Kd, Vd = oracle.dequant_slice(st)
                for j in range(w.gqa):
                    hq = h * w.gqa + j
                    eo, el = oracle.attention(qf[b, hq], Kd, Vd, scale)
                    err = max(err, float(np.abs(out[b, hq] - eo).max()), abs(float(lse[b, hq]) - el))
        assert err <= ATOL, err
        return err


VARIANTS = [
    (dict(), 1),                                                                    # VALU stream, a page per group
    (dict(bits=2, n_sink=3), 2),
    (dict(n_q_heads=8, bits=2, k_group=64, v_group=64, residual=128), 1),           # matrix cores
    (dict(bits=8, k_group=64, v_group=64, residual=64, codec=1), 2),                # 8-bit
    (dict(residual=96, log_window=32), 2),                                          # log-sparse retention
]


@pytest.mark.parametrize("kw,P", VARIANTS)
def test_paged_equals_contiguous_and_oracle(kw, P):
    require_gpu()
    w = _w(**kw)
    log("case %s P=%d" % (kw, P))
    tw = Twin(w, max_tokens=700, page_groups=P)
    # prefill in rounds of chunks, so that the sequences' pages interleave in the pool
    seed = 100
    for rnd in range(4):
        n_new = [(37 * (b + rnd) + 29) % 120 + 10 for b in range(w.batch)]
        tw.append_ragged(n_new, seed)
        seed += 2
    q, out, lse = tw.step(seed)
    tw.check(q, out, lse)
    # release a sequence: its pages go back to the pool and are taken by the others
    free0 = tw.paged.free_pages()
    tw.release(1)
    assert tw.paged.free_pages() > free0
    tw.append_ragged([90, 0, 150, 60], seed + 10)
    tw.append_ragged([0, 200, 0, 0], seed + 20)   # the released sequence takes a new prompt
    worst = 0.0
    for s in range(40):
        q, out, lse = tw.step(seed + 30 + 3 * s)
        if s % 13 == 0 or s == 39:
            worst = max(worst, tw.check(q, out, lse))
    log("  max |out - oracle| = %.3g, free pages %d" % (worst, tw.paged.free_pages()))


def test_splits_spanning_many_pages():
    require_gpu()
    w = _w(batch=2)
    # one group per page, 80 groups per sequence, splits as long as allowed (63 pages)
    tw = Twin(w, max_tokens=2700, page_groups=1)
    for c in (tw.paged, tw.flat):
        c.set_split_tokens(63 * w.k_group)
    tw.append_ragged([1300, 700], 7)
    tw.append_ragged([1300, 1900], 9)
    q, out, lse = tw.step(11)
    tw.check(q, out, lse)


def test_pool_exhaustion_changes_nothing():
    require_gpu()
    w = _w()
    # pages of 2 groups (64 tokens); 6 pages in the pool
    cache = make_cache(w, max_tokens=700, page_groups=2, pool_pages=6)
    K, V = _tokens(w, 300, 3), _tokens(w, 300, 4)
    kt, vt = to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV)
    cache.append_ragged(kt, vt, [130, 0, 70, 0])   # quantized 128 and 64 tokens: 2 + 1 pages
    assert cache.free_pages() == 3
    lens, free = cache.seq_lengths(), cache.free_pages()
    with pytest.raises(kvq.KVQError) as ei:
        cache.append_ragged(kt, vt, [0, 300, 0, 0])  # needs 4 pages
    assert ei.value.status == kvq.KVQ_ERR_CAPACITY
    assert cache.seq_lengths() == lens and cache.free_pages() == free
    cache.release_sequence(0)
    assert cache.free_pages() == 5 and cache.seq_lengths() == [0, 0, 70, 0]
    cache.append_ragged(kt, vt, [1, 300, 60, 1])   # 4 pages, and a second one for sequence 2
    assert cache.free_pages() == 0
    with pytest.raises(kvq.KVQError) as ei:
        cache.append_ragged(kt, vt, [0, 0, 64, 0])
    assert ei.value.status == kvq.KVQ_ERR_CAPACITY
    q = to_torch(wl.random_tokens(5, (w.batch, w.n_q_heads, w.head_dim), w.dtype), w.dtype, DEV)
    out, lse = cache.decode(q)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    with pytest.raises(kvq.KVQError):
        cache.release_sequence(4)
