"""Host logic of bench.py, checked against the oracle on the CPU.

The bench predicts each cache's state from the schedule (slice_counts), sizes
page pools from it, and converts times to GB/s with the algorithmic bytes of the
state.  These must agree with the cache state the oracle builds token by token,
for both flush rules (KIVI notes, section 1; "Resumo Técnico: LogQuant",
Metodologia item 2), and the bytes must count every field the decode reads.
"""
import numpy as np
import pytest

import bench
import oracle
import workloads as wl


@pytest.mark.parametrize("S,R,W", [(0, 8, 0), (3, 8, 0), (0, 12, 4), (2, 6, 2)])
def test_slice_counts_follow_the_oracle(S, R, W):
    w = wl.get("tiny").replace(n_sink=S, residual=R, log_window=W, k_group=2, v_group=8, head_dim=8)
    rng = np.random.default_rng(S * 31 + R)
    k = rng.standard_normal((90, 8)).astype(np.float32)
    for n in range(0, 90, 7):
        st = oracle.build_slice(k[:n], k[:n], head_dim=8, bits=4, k_group=2, v_group=8, residual=R,
                                n_sink=S, log_window=W)
        assert bench.slice_counts(w, n) == (st["n_sink"], st["n_quant"], st["n_resid"])


def test_algorithmic_bytes_count_every_field():
    w = wl.get("llama7b_mha_int4")
    D, G, e = w.head_dim, w.k_group, 2
    Lq, r = 4096, 64
    per_slice = Lq * 2 * D * 4 // 8 + (Lq // G) * 2 * D * 4 + Lq * 2 * 4 + r * 2 * D * e
    q_out = w.batch * w.n_q_heads * D * (e + 4)
    assert bench.algorithmic_bytes(w, 0, Lq, r) == w.batch * w.n_kv_heads * per_slice + q_out
    wo = w.replace(outliers=1)
    extra = (Lq // G) * D * 6 + Lq * 6            # one (value, place, code) per key and value vector
    assert bench.algorithmic_bytes(wo, 0, Lq, r) == w.batch * w.n_kv_heads * (per_slice + extra) + q_out
    # ragged: a sequence's share of the bytes is that of a batch of one
    lens = [4096, 2048]
    wr = w.replace(batch=2)
    assert bench.algorithmic_bytes_seqs(wr, lens) == sum(
        bench.algorithmic_bytes(w.replace(batch=1), *bench.slice_counts(w, n)) for n in lens)


def test_prefill_rounds_cover_each_prefill_once():
    w = wl.get("llama7b_mha_int4_paged")
    lens = wl.prefill_lengths(w)
    got = [0] * w.batch
    for t0, n_new in wl.prefill_rounds(w):
        for b, n in enumerate(n_new):
            assert n == 0 or t0 == got[b]          # each round continues where the last stopped
            got[b] += n
    assert got == lens
