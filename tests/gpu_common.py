"""Shared helpers of the GPU tests: drive a workload through the C-ABI on cuda:0 and
compare with the CPU oracle.

Bars (the target of this path): codes, scales and zero points bit-exact; attention
outputs within ATOL = 1e-3 absolute of the binary64 oracle, for every output of
every attention call checked.
"""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from workloads.torch_io import TORCH_DTYPES, to_torch

ATOL = 1e-3

gpu = pytest.mark.gpu


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def make_cache(w: wl.Workload, max_tokens: int | None = None, **over):
    from bit_quantized_kv_kvq_amd import Cache
    kw = dict(batch=w.batch, n_kv_heads=w.n_kv_heads, n_q_heads=w.n_q_heads,
              head_dim=w.head_dim, bits=w.bits, k_group=w.k_group, v_group=w.v_group,
              residual=w.residual, n_sink=w.n_sink, dtype=TORCH_DTYPES[w.dtype],
              max_tokens=max_tokens or w.max_tokens, device=torch.device("cuda:0"), codec=w.codec,
              retention=1 if w.log_window else 0, page_groups=w.page_groups, outliers=w.outliers,
              key_axis=w.key_axis)
    kw.update(over)
    return Cache(**kw)


def prefill(cache, w: wl.Workload, Kd, Vd):
    """The workload's prefill (device K, V [B, Hkv, prefill, D]) in its rounds."""
    rounds = wl.prefill_rounds(w)
    t0, n_new = rounds[0]
    if len(rounds) == 1 and len(set(n_new)) == 1:
        cache.append(Kd, Vd)
        return
    for t0, n_new in rounds:
        n = max(n_new)
        cache.append_ragged(Kd[:, :, t0:t0 + n].contiguous(), Vd[:, :, t0:t0 + n].contiguous(), n_new)


class WorkloadRun:
    """Uploads a workload and steps through its schedule on the GPU."""

    def __init__(self, w: wl.Workload, cache=None):
        self.w = w
        self.dev = torch.device("cuda:0")
        self.cache = cache or make_cache(w)
        Kp, Vp = wl.prefill_batch(w)
        prefill(self.cache, w, to_torch(Kp, w.dtype, self.dev), to_torch(Vp, w.dtype, self.dev))
        del Kp, Vp
        Ks, Vs = wl.steps_batch(w)
        self.Ks = to_torch(Ks, w.dtype, self.dev)
        self.Vs = to_torch(Vs, w.dtype, self.dev)
        self.Q = to_torch(wl.queries_batch(w), w.dtype, self.dev)
        self.n_steps = 0

    def append_step(self, s: int):
        self.cache.append(self.Ks[s][:, :, None].contiguous(), self.Vs[s][:, :, None].contiguous())
        self.n_steps = s + 1

    def attend(self, qi: int):
        out, lse = self.cache.decode(self.Q[qi].contiguous())
        return out, lse

    def run(self, on_attend, fused: bool = False):
        """on_attend(n_steps, qi, out, lse) after every attention call of the schedule.

        fused: every append that an attention call follows is made with it in one
        kvq_append_decode call, as the benchmark steps (the library itself takes
        the two-call path on steps where a token becomes a sink or fills a residual).
        """
        sched = list(wl.schedule(self.w))
        i = 0
        while i < len(sched):
            op, idx = sched[i]
            if op == "append" and fused and i + 1 < len(sched) and sched[i + 1][0] == "attend":
                qi = sched[i + 1][1]
                out, lse = self.cache.append_decode(self.Ks[idx][:, :, None].contiguous(),
                                                    self.Vs[idx][:, :, None].contiguous(),
                                                    self.Q[qi].contiguous())
                self.n_steps = idx + 1
                on_attend(self.n_steps, qi, out, lse)
                i += 2
                continue
            if op == "append":
                self.append_step(idx)
            else:
                out, lse = self.attend(idx)
                on_attend(self.n_steps, idx, out, lse)
            i += 1


def export_cpu(cache):
    torch.cuda.synchronize()
    ex = cache.export()
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in ex.items()}


def assert_export_slice_matches(ex, st, b: int, kvh: int):
    """Bit-exact codes, scales and zero points of slice (b, kvh) vs an oracle state
    (the export holds the longest sequence's rows; a shorter slice uses the first)."""
    Lq = st["n_quant"]
    G = st["k_group"]
    assert ex["k_codes"].shape[2] >= Lq
    np.testing.assert_array_equal(ex["k_codes"][b, kvh, :Lq], st["k_codes"])
    np.testing.assert_array_equal(ex["v_codes"][b, kvh, :Lq], st["v_codes"])
    krows = Lq if st.get("key_axis", 0) else Lq // G   # per-token keys: one (scale, zero) per token
    for name, rows in (("k_scale", krows), ("k_zero", krows), ("v_scale", Lq), ("v_zero", Lq)):
        got = np.ascontiguousarray(ex[name][b, kvh, :rows]).view(np.uint32)
        want = np.ascontiguousarray(st[name]).view(np.uint32)
        np.testing.assert_array_equal(got, want, err_msg=name)


def _pool_size() -> int:
    # at most 16 workers: the GPU machine's CPU share, whatever os.cpu_count() reports
    return max(1, min(16, os.cpu_count() or 1))


def oracle_states_iter(w, pairs, n_steps: int):
    """(pair, oracle state) for each (b, kvh) pair, built on a thread pool (the
    draws and the oracle's C code release the GIL), in the order of pairs."""
    with ThreadPoolExecutor(_pool_size()) as ex:
        yield from zip(pairs, ex.map(lambda p: oracle.slice_state(w, p[0], p[1], n_steps), pairs))


def expected_outputs_many(w, pairs, n_steps: int, qi: int):
    """{(b, kvh): (out [g, D], lse [g])} of the binary64 oracle, on a thread pool."""
    with ThreadPoolExecutor(_pool_size()) as ex:
        res = ex.map(lambda p: oracle.expected_outputs(w, p[0], p[1], n_steps, qi), pairs)
        return dict(zip(pairs, res))


def sample_pairs(w, n_random: int = 8, seed: int = 0):
    """The four corner (sequence, kv head) slices and n_random seeded others."""
    B, H = w.batch, w.n_kv_heads
    pairs = sorted({(0, 0), (0, H - 1), (B - 1, 0), (B - 1, H - 1)})
    rest = [(b, h) for b in range(B) for h in range(H) if (b, h) not in pairs]
    rng = np.random.default_rng([w.seed, 77, seed])
    pick = rng.choice(len(rest), size=min(n_random, len(rest)), replace=False) if rest else []
    return pairs + sorted(rest[int(i)] for i in pick)


def check_outputs_many(w, out_cpu, lse_cpu, pairs, n_steps: int, qi: int):
    """check_outputs for several slices, with the oracle run on a thread pool."""
    exp = expected_outputs_many(w, pairs, n_steps, qi)
    g = w.gqa
    worst = 0.0
    for (b, kvh), (eo, el) in exp.items():
        got = out_cpu[b, kvh * g:(kvh + 1) * g].astype(np.float64)
        err = float(np.abs(got - eo).max())
        lerr = float(np.abs(lse_cpu[b, kvh * g:(kvh + 1) * g].astype(np.float64) - el).max())
        assert err <= ATOL, (w.name, b, kvh, n_steps, qi, err)
        assert lerr <= ATOL, (w.name, b, kvh, n_steps, qi, lerr)
        worst = max(worst, err, lerr)
    return worst


def check_outputs(w, out_cpu, lse_cpu, b: int, kvh: int, n_steps: int, qi: int):
    """Max abs error of out/lse of every query head of (b, kvh) vs the oracle."""
    eo, el = oracle.expected_outputs(w, b, kvh, n_steps, qi)
    g = w.gqa
    got = out_cpu[b, kvh * g:(kvh + 1) * g].astype(np.float64)
    err = float(np.abs(got - eo).max())
    lerr = float(np.abs(lse_cpu[b, kvh * g:(kvh + 1) * g].astype(np.float64) - el).max())
    assert err <= ATOL, (w.name, b, kvh, n_steps, qi, err)
    assert lerr <= ATOL, (w.name, b, kvh, n_steps, qi, lerr)
    return err
