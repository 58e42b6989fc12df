"""GPU tests of caches whose sequences differ in length, through the C-ABI.

Each sequence follows the cache state machine from its own length (KIVI notes,
section 1): the oracle builds every (sequence, kv head) slice from that slice's
own tokens, and the GPU must match it slice by slice: codes, scales and zero
points bit-exact, attention within ATOL, at every step.
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
    base = wl.get("C2").replace(name="ragged", batch=4, n_kv_heads=2, n_q_heads=2, prefill=0,
                                steps=0, k_group=32, v_group=32, residual=64)
    return base.replace(**kw)


class Mirror:
    """Host copy of every slice's tokens (storage dtype), for the oracle."""

    def __init__(self, w):
        self.w = w
        self.k = [[[] for _ in range(w.n_kv_heads)] for _ in range(w.batch)]
        self.v = [[[] for _ in range(w.n_kv_heads)] for _ in range(w.batch)]

    def add(self, K, V, n_new):
        for b in range(self.w.batch):
            for h in range(self.w.n_kv_heads):
                self.k[b][h].extend(list(K[b, h, :n_new[b]]))
                self.v[b][h].extend(list(V[b, h, :n_new[b]]))

    def lengths(self):
        return [len(self.k[b][0]) for b in range(self.w.batch)]

    def state(self, b, h):
        w = self.w
        D = w.head_dim
        kf = wl.storage_to_f32(np.array(self.k[b][h]).reshape(-1, D), w.dtype)
        vf = wl.storage_to_f32(np.array(self.v[b][h]).reshape(-1, D), w.dtype)
        return oracle.build_slice(kf, vf, head_dim=D, bits=w.bits, k_group=w.k_group,
                                  v_group=w.v_group, residual=w.residual, n_sink=w.n_sink,
                                  codec=w.codec)


def _tokens(w, n, seed, scale=1.0):
    return wl.random_tokens(seed, (w.batch, w.n_kv_heads, n, w.head_dim), w.dtype, scale)


def _check_attention(w, mirror, out, lse, q):
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    qf = wl.storage_to_f32(q, w.dtype)
    scale = oracle.default_scale(w.head_dim)
    err = 0.0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            Kd, Vd = oracle.dequant_slice(mirror.state(b, h))
            for j in range(w.gqa):
                hq = h * w.gqa + j
                eo, el = oracle.attention(qf[b, hq], Kd, Vd, scale)
                err = max(err, float(np.abs(out[b, hq] - eo).max()), abs(float(lse[b, hq]) - el))
    assert err <= ATOL, err
    return err


def _check_export_and_dequant(w, cache, mirror):
    ex = export_cpu(cache)
    K, V = cache.dequantize()
    torch.cuda.synchronize()
    K, V = K.cpu().numpy(), V.cpu().numpy()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            st = mirror.state(b, h)
            Lq, T = st["n_quant"], st["n_sink"] + st["n_quant"] + st["n_resid"]
            np.testing.assert_array_equal(ex["k_codes"][b, h, :Lq], st["k_codes"])
            np.testing.assert_array_equal(ex["v_codes"][b, h, :Lq], st["v_codes"])
            for name in ("k_scale", "k_zero"):
                got = np.ascontiguousarray(ex[name][b, h, :Lq // w.k_group]).view(np.uint32)
                np.testing.assert_array_equal(got, np.ascontiguousarray(st[name]).view(np.uint32), err_msg=name)
            for name in ("v_scale", "v_zero"):
                got = np.ascontiguousarray(ex[name][b, h, :Lq]).view(np.uint32)
                np.testing.assert_array_equal(got, np.ascontiguousarray(st[name]).view(np.uint32), err_msg=name)
            # rows past this slice's own tokens are left as the caller's zeros
            assert not ex["k_codes"][b, h, Lq:].any() and not K[b, h, T:].any()
            Ko, Vo = oracle.dequant_slice(st)
            np.testing.assert_array_equal(K[b, h, :T].view(np.uint32), Ko.view(np.uint32))
            np.testing.assert_array_equal(V[b, h, :T].view(np.uint32), Vo.view(np.uint32))


@pytest.mark.parametrize("kw", [
    dict(),                                                            # VALU stream
    dict(n_sink=3, bits=2),                                            # a sequence shorter than S
    dict(n_q_heads=8, k_group=64, v_group=64, residual=128),           # matrix-core stream, g = 4
    dict(bits=8, k_group=64, v_group=64, residual=64, codec=1),        # 8-bit, symmetric
])
def test_ragged_prefill_then_steps(kw):
    require_gpu()
    w = _w(**kw)
    log("case %s" % kw)
    cache = make_cache(w, max_tokens=320)
    mirror = Mirror(w)
    lens = [150, 2, 64, 97]
    K, V = _tokens(w, 150, 31, 2.0), _tokens(w, 150, 32)
    cache.append_ragged(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV), lens)
    mirror.add(K, V, lens)
    assert cache.seq_lengths() == lens
    assert cache.state()[0] == 150
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=DEV)
    lse = torch.empty((w.batch, w.n_q_heads), dtype=torch.float32, device=DEV)
    worst = 0.0
    for step in range(70):
        # every residual fills at a different step: sequences flush one at a time
        k1, v1 = _tokens(w, 1, 1000 + step), _tokens(w, 1, 2000 + step)
        q = wl.random_tokens(3000 + step, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
        kt, vt, qt = (to_torch(x, w.dtype, DEV) for x in (k1, v1, q))
        if step % 3 == 2:
            cache.append_decode(kt, vt, qt, out=out, lse=lse)
        else:
            cache.append(kt, vt)
            cache.decode(qt, out=out, lse=lse)
        mirror.add(k1, v1, [1] * w.batch)
        if step % 7 == 0 or step >= 60:
            torch.cuda.synchronize()
            worst = max(worst, _check_attention(w, mirror, out, lse, q))
    assert cache.seq_lengths() == mirror.lengths()
    _check_export_and_dequant(w, cache, mirror)
    log("  max |out - oracle| = %.3g, lengths %s" % (worst, cache.seq_lengths()))


def test_ragged_bulk_appends_and_return_to_uniform():
    require_gpu()
    w = _w(n_sink=2)
    cache = make_cache(w, max_tokens=400)
    mirror = Mirror(w)
    seed = 40
    for n_new in ([10, 0, 5, 20], None, [23, 33, 28, 13]):
        if n_new is None:  # several tokens to every sequence: sequence by sequence
            K, V = _tokens(w, 7, seed, 2.0), _tokens(w, 7, seed + 1)
            cache.append(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV))
            mirror.add(K, V, [7] * w.batch)
        else:
            n_max = max(n_new) + 3
            K, V = _tokens(w, n_max, seed, 2.0), _tokens(w, n_max, seed + 1)
            cache.append_ragged(to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV), n_new)
            mirror.add(K, V, n_new)
        seed += 2
        assert cache.seq_lengths() == mirror.lengths()
    # all sequences now hold 40 tokens: the uniform layout again
    assert cache.seq_lengths() == [40] * w.batch
    assert cache.state() == (40, 2, 0, 38)
    q = wl.random_tokens(77, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
    out, lse = cache.decode(to_torch(q, w.dtype, DEV))
    torch.cuda.synchronize()
    _check_attention(w, mirror, out, lse, q)
    for step in range(30):  # the one-launch step on the uniform layout
        k1, v1 = _tokens(w, 1, 500 + step), _tokens(w, 1, 600 + step)
        q = wl.random_tokens(700 + step, (w.batch, w.n_q_heads, w.head_dim), w.dtype)
        out, lse = cache.append_decode(*(to_torch(x, w.dtype, DEV) for x in (k1, v1, q)))
        mirror.add(k1, v1, [1] * w.batch)
    torch.cuda.synchronize()
    _check_attention(w, mirror, out, lse, q)
    _check_export_and_dequant(w, cache, mirror)


def test_ragged_validation_leaves_state_unchanged():
    require_gpu()
    w = _w()
    cache = make_cache(w, max_tokens=100)
    K, V = _tokens(w, 8, 51), _tokens(w, 8, 52)
    kt, vt = to_torch(K, w.dtype, DEV), to_torch(V, w.dtype, DEV)
    cache.append_ragged(kt, vt, [8, 0, 3, 5])
    q = to_torch(wl.random_tokens(5, (w.batch, w.n_q_heads, w.head_dim), w.dtype), w.dtype, DEV)
    with pytest.raises(kvq.KVQError) as ei:      # sequence 1 is empty
        cache.decode(q)
    assert ei.value.status == kvq.KVQ_ERR_INVALID_ARG
    for bad, status in (([9, 0, 0, 0], kvq.KVQ_ERR_INVALID_ARG), ([-1, 0, 0, 0], kvq.KVQ_ERR_INVALID_ARG)):
        with pytest.raises(kvq.KVQError) as ei:
            cache.append_ragged(kt, vt, bad)
        assert ei.value.status == status
    big_k = to_torch(_tokens(w, 96, 53), w.dtype, DEV)
    with pytest.raises(kvq.KVQError) as ei:      # 8 + 93 > 100
        cache.append_ragged(big_k, big_k, [93, 0, 0, 0])
    assert ei.value.status == kvq.KVQ_ERR_CAPACITY
    assert cache.seq_lengths() == [8, 0, 3, 5]
    cache.append_ragged(kt, vt, [0, 1, 0, 0])
    out, lse = cache.decode(q)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
