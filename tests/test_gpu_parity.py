"""GPU parity of the HIP path against the CPU oracle, through the C-ABI.

Small versions of every workload (all slices, every attention call, sizes that
span several tiles and splits with a ragged residual tail and at least one flush)
and the full-size workloads in the launch configuration the benchmark times
(sampled slices checked one by one).  Codes, scales and zero points must be
bit-exact; attention outputs and log-sum-exp within 1e-3 absolute.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_common import (ATOL, WorkloadRun, assert_export_slice_matches, check_outputs,
                              check_outputs_many, export_cpu, gpu, log, make_cache, oracle_states_iter,
                              require_gpu, sample_pairs)

pytestmark = gpu

SMALL = {
    "tiny": wl.get("tiny"),
    "llama7b_small": wl.get("C2").replace(name="llama7b_small", batch=2, n_kv_heads=3,
                                          n_q_heads=3, prefill=1000, steps=30),
    "kivi2_small": wl.get("C3").replace(name="kivi2_small", batch=2, n_kv_heads=3, n_q_heads=3,
                                        prefill=700, steps=40),
    "gqa_small": wl.get("C4").replace(name="gqa_small", batch=2, n_kv_heads=2, n_q_heads=8,
                                      prefill=1200, steps=20),
    "sink_small": wl.get("C5").replace(name="sink_small", batch=1, n_kv_heads=2, n_q_heads=8,
                                       prefill=1000, steps=40),
    "sym_small": wl.get("llama7b_mha_int4_sym").replace(name="sym_small", batch=2, n_kv_heads=3,
                                                        n_q_heads=3, prefill=1000, steps=30),
    "int8_small": wl.get("llama7b_mha_int8").replace(name="int8_small", batch=2, n_kv_heads=3,
                                                     n_q_heads=6, prefill=1000, steps=30),
    "outliers_small": wl.get("llama7b_mha_int4_outliers").replace(name="outliers_small", batch=2, n_kv_heads=3,
                                                                  n_q_heads=3, prefill=1000, steps=30),
    "logquant_small": wl.get("logquant_gqa_int2").replace(name="logquant_small", batch=2, n_kv_heads=2,
                                                          n_q_heads=8, prefill=1000, steps=100),
    "headgran_small": wl.get("llama7b_mha_int4_headgran").replace(name="headgran_small", batch=2, n_kv_heads=3,
                                                                  n_q_heads=3, prefill=1000, steps=30),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_workload_all_slices_every_step(name):
    require_gpu()
    w = SMALL[name]
    log("case %s: %s" % (name, w))
    run = WorkloadRun(w)
    # after the bulk prefill: every slice bit-exact
    ex = export_cpu(run.cache)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            assert_export_slice_matches(ex, oracle.slice_state(w, b, h, 0), b, h)
    worst = [0.0]
    flush_checked = []
    last_Lq = [run.cache.state()[2]]

    def on_attend(n_steps, qi, out, lse):
        torch.cuda.synchronize()
        o, l = out.cpu().numpy(), lse.cpu().numpy()
        n_tok, nS, Lq, r = run.cache.state()
        N = w.prefill + n_steps
        assert nS == min(N, w.n_sink)
        assert Lq == oracle.quantized_count(N - nS, w.residual, w.log_window) and r == N - nS - Lq
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                worst[0] = max(worst[0], check_outputs(w, o, l, b, h, n_steps, qi))
        flushed, last_Lq[0] = Lq != last_Lq[0], Lq
        if n_steps > 0 and flushed and n_steps not in flush_checked:
            flush_checked.append(n_steps)
            exf = export_cpu(run.cache)
            for b in range(w.batch):
                for h in range(w.n_kv_heads):
                    assert_export_slice_matches(exf, oracle.slice_state(w, b, h, n_steps), b, h)

    run.run(on_attend)
    ex = export_cpu(run.cache)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            assert_export_slice_matches(ex, oracle.slice_state(w, b, h, w.steps), b, h)
    log("case %s: max |out - oracle| = %.3g, flushes checked at steps %s" % (name, worst[0], flush_checked))


@pytest.mark.parametrize("name", ["llama7b_small", "sink_small", "tiny"])
def test_dequantize_bit_exact(name):
    require_gpu()
    w = SMALL[name]
    run = WorkloadRun(w)
    for s in range(min(w.steps, 7)):
        run.append_step(s)
    K, V = run.cache.dequantize()
    torch.cuda.synchronize()
    K, V = K.cpu().numpy(), V.cpu().numpy()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            Ko, Vo = oracle.dequant_slice(oracle.slice_state(w, b, h, run.n_steps))
            np.testing.assert_array_equal(K[b, h].view(np.uint32), Ko.view(np.uint32))
            np.testing.assert_array_equal(V[b, h].view(np.uint32), Vo.view(np.uint32))


@pytest.mark.parametrize("name", ["llama7b_small", "gqa_small", "sink_small", "kivi2_small"])
def test_split_count_invariance(name):
    require_gpu()
    w = SMALL[name]
    run = WorkloadRun(w)
    run.append_step(0)
    q = run.Q[0].contiguous()
    ref, ref_lse = run.cache.decode(q)
    ref, ref_lse = ref.clone(), ref_lse.clone()
    for tokens in [w.k_group, 2 * w.k_group, 3 * w.k_group, 5 * w.k_group, 1 << 30]:
        run.cache.set_split_tokens(tokens)
        out, lse = run.cache.decode(q)
        torch.cuda.synchronize()
        d = (out - ref).abs().max().item()
        dl = (lse - ref_lse).abs().max().item()
        # The fixed-point image of the softmax weights (2^-19 of the largest weight
        # since the last rescale, which may sit up to 2^8 above the running max)
        # depends on how tokens are split, so split plans agree to a few 1e-5 of
        # the output scale; each is within 1e-3 of the binary64 oracle.
        scale = max(1.0, ref.abs().max().item())
        assert d <= 5e-5 * scale and dl <= 5e-5 * max(1.0, ref_lse.abs().max().item()), (tokens, d, dl)
    run.cache.set_split_tokens(0)
    out, _ = run.cache.decode(q)
    assert torch.equal(out, ref)


def test_repeat_calls_are_bitwise_deterministic():
    require_gpu()
    w = SMALL["gqa_small"]
    run = WorkloadRun(w)
    run.append_step(0)
    q = run.Q[0].contiguous()
    a, la = run.cache.decode(q)
    a, la = a.clone(), la.clone()
    for _ in range(5):
        b, lb = run.cache.decode(q)
        assert torch.equal(a, b) and torch.equal(la, lb)


# ---------------------------------------------------------------------------
# full-size workloads in the launch configuration the benchmark times
# ---------------------------------------------------------------------------

# Every workload at its full size, prefilled and then stepped exactly as bench.py
# steps it: one kvq_append_decode call per decode step (the one-launch step with
# the automatic split plan: one split per slice on the Llama-7B-shaped and KIVI
# workloads, the single-split branch of the kernel; the library falls back to
# append + decode on sink and flush steps).  After the prefill, every slice's
# export of the Llama-7B-shaped, KIVI 2-bit, GQA and long-context workloads is
# compared bit for bit (a sample of slices for the others); at the first and last decode steps and at every step
# that flushed, the four corner slices and eight seeded others are compared with
# the oracle element by element.
FULL = ["tiny", "llama7b_mha_int4", "kivi2_long_batch", "gqa_32k_int4", "long_128k_sink_int2",
        "llama7b_mha_int4_sym", "llama7b_mha_int8", "llama7b_mha_int4_ragged", "logquant_gqa_int2",
        "llama7b_mha_int4_paged", "llama7b_mha_int4_outliers", "gqa_32k_int4_outliers",
        "llama7b_mha_int4_headgran"]
EXPORT_ALL = {"llama7b_mha_int4", "kivi2_long_batch", "gqa_32k_int4", "long_128k_sink_int2"}


@pytest.mark.parametrize("name", FULL)
def test_full_size_bench_path(name):
    require_gpu()
    w = wl.get(name)
    pairs = sample_pairs(w)
    log("full-size case %s: %s; sampled slices %s" % (name, w.description, pairs))
    run = WorkloadRun(w)
    log("  prefill uploaded and quantized")
    ex = export_cpu(run.cache)
    every = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    n_exp = 0
    for (b, h), st in oracle_states_iter(w, every if name in EXPORT_ALL else pairs, 0):
        assert_export_slice_matches(ex, st, b, h)
        n_exp += 1
    del ex
    log("  exports after the prefill bit-exact on %d slices" % n_exp)
    last_q = wl.n_queries(w) - 1
    checked, worst = [], [0.0]
    last_Lq = [run.cache.state()[2]]

    def on_attend(n_steps, qi, out, lse):
        Lq = run.cache.state()[2]
        flushed, last_Lq[0] = Lq != last_Lq[0], Lq
        if not (qi in (0, last_q) or flushed):
            return
        torch.cuda.synchronize()
        o, l = out.cpu().numpy(), lse.cpu().numpy()
        worst[0] = max(worst[0], check_outputs_many(w, o, l, pairs, n_steps, qi))
        checked.append(qi)

    run.run(on_attend, fused=True)
    ex = export_cpu(run.cache)
    for (b, h), st in oracle_states_iter(w, pairs, w.steps):
        assert_export_slice_matches(ex, st, b, h)
    log("  %s: queries %s checked on %d slices, max err %.3g" % (name, checked, len(pairs), worst[0]))
