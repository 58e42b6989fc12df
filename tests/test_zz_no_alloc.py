"""GPU test of kvq_decode_attention_static, the decode for callers that cannot
allocate: its output must equal kvq_decode_attention's, bit for bit (same kernels,
same split plan, the workspace taken from the library's static scratch), on two
calls in a row, the second on a smaller cache; a cache whose decode needs more
than the static scratch is refused before anything is enqueued."""
import pytest
import torch

import bit_quantized_kv_kvq_amd as kvq
import workloads as wl
from tests.gpu_common import gpu, log, make_cache, require_gpu
from workloads.torch_io import to_torch

pytestmark = gpu

DEV = torch.device("cuda:0")


def _filled(w, n, seed):
    c = make_cache(w, max_tokens=n + 4)
    K = to_torch(wl.random_tokens(seed, (w.batch, w.n_kv_heads, n, w.head_dim), w.dtype, 2.0), w.dtype, DEV)
    V = to_torch(wl.random_tokens(seed + 1, (w.batch, w.n_kv_heads, n, w.head_dim), w.dtype), w.dtype, DEV)
    c.append(K, V)
    q = to_torch(wl.random_tokens(seed + 2, (w.batch, w.n_q_heads, w.head_dim), w.dtype), w.dtype, DEV)
    return c, q


def _static(c, q):
    out = torch.full((c.batch, c.n_q_heads, c.head_dim), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((c.batch, c.n_q_heads), float("nan"), dtype=torch.float32, device=DEV)
    kvq.kvq_decode_attention_static(c.handle, q.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    return out, lse


def test_static_scratch_decode_equals_workspace_decode():
    require_gpu()
    base = wl.get("C2")
    cases = [   # a larger cache, then a smaller one (fewer slices, shorter, several splits)
        (base.replace(batch=4, n_kv_heads=8, n_q_heads=8), 3000, 11),
        (base.replace(batch=1, n_kv_heads=2, n_q_heads=8, bits=2, k_group=64, v_group=64), 1500, 21),
    ]
    for w, n, seed in cases:
        log("case %s n=%d" % (w, n))
        c, q = _filled(w, n, seed)
        assert c.ws_bytes <= kvq.KVQ_STATIC_SCRATCH_BYTES
        ref, ref_lse = c.decode(q)
        for _ in range(2):   # repeated calls: the counters are left at zero
            out, lse = _static(c, q)
            torch.cuda.synchronize()
            assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
        c.close()


def test_static_scratch_refuses_a_larger_workspace():
    require_gpu()
    # 4096 slices with one split each need more than 16 MiB of partials
    w = wl.get("C2").replace(batch=128, n_kv_heads=32, n_q_heads=32)
    c, q = _filled(w, 8, 31)
    assert c.ws_bytes > kvq.KVQ_STATIC_SCRATCH_BYTES
    with pytest.raises(kvq.KVQError) as ei:
        _static(c, q)
    assert ei.value.status == kvq.KVQ_ERR_BUFFER_TOO_SMALL
    out, lse = c.decode(q)   # the workspace call still serves it
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
