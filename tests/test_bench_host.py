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
    wk = w.replace(key_axis=1)                    # head-granular keys: one (scale, zero) per token
    per_tok = Lq * 2 * D * 4 // 8 + Lq * 2 * 4 + Lq * 2 * 4 + r * 2 * D * e
    assert bench.algorithmic_bytes(wk, 0, Lq, r) == w.batch * w.n_kv_heads * per_tok + q_out
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


@pytest.mark.parametrize("steps", [1, 5, 15, 16, 20, 31, 64, 127, 256, 1000])
def test_event_stride_times_enough_launches(steps):
    """At least 16 timed launches whatever --steps is (every launch below that), and
    never more than one in eight of a long region."""
    stride = bench.event_stride(steps)
    timed = len(range(0, steps, stride))
    assert timed >= min(16, steps)
    assert 1 <= stride <= 8


def test_step_plan_fuses_only_steps_without_sinks_or_flushes():
    w = wl.get("long_128k_sink_int2").replace(prefill=300)   # S4, R256: 44 residual tokens
    L = 2
    plan = bench.step_plan(w, L, 2 * 300)
    for s, (fused, nbytes) in enumerate(plan):
        n_before = w.prefill + s // L
        nS, Lq, r = bench.slice_counts(w, n_before)
        assert fused == (nS >= w.n_sink and r + 1 < w.residual)
        assert nbytes == bench.algorithmic_bytes_seqs(w, [n_before + 1])
    assert not all(f for f, _ in plan) and any(f for f, _ in plan)


def test_write_traffic_averages_the_timed_dispatches(tmp_path, monkeypatch):
    """The traffic summary scales the decode kernel's counters by the probes' and
    averages the last `steps` decode dispatches only (the timed ones)."""
    import csv
    import json
    w = wl.get("llama7b_mha_int4")
    steps, warmup = 4, 3
    monkeypatch.setattr(bench, "traffic_path", lambda w_: str(tmp_path / "t.json"))

    def write(path, rows):
        with open(path, "w", newline="") as f:
            wr = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            wr.writeheader()
            for r in rows:
                wr.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))

    dec = [(i, "kvq::dec::decode_kernel<4>", "FETCH_SIZE", 1000.0 if i < warmup else 100.0 * i)
           for i in range(warmup + steps)]
    decw = [(i, "kvq::dec::decode_kernel<4>", "WRITE_SIZE", 7.0) for i in range(warmup + steps)]
    probe = [(100 + i, "kvq::stream_read_kernel", "FETCH_SIZE", 2 ** 21 / 2.0) for i in range(3)] + \
            [(200 + i, "elementwise_kernel", "FETCH_SIZE", 2 ** 20 / 2.2) for i in range(3)]
    copyw = [(300 + i, "elementwise_kernel", "WRITE_SIZE", 2 ** 20) for i in range(3)]
    for name, rows in (("f", dec), ("w", decw), ("p", probe), ("c", copyw)):
        write(tmp_path / name, rows)
    bench.write_traffic(w, steps, warmup, 2, *(str(tmp_path / n) for n in "fwpc"))
    t = json.load(open(tmp_path / "t.json"))
    run = t["runs"][0]
    timed = [100.0 * i for i in range(warmup, warmup + steps)]
    assert run["fetch_kib_per_dispatch"] == sum(timed) / steps
    assert abs(t["read_probe_fetch_scale"] - 2.0) < 1e-12 and abs(t["copy_probe_fetch_scale"] - 2.2) < 1e-12
    assert run["hbm_bytes_per_launch"] == int(sum(timed) / steps * 1024 * 2.0 + 7.0 * 1024)
    plan = bench.step_plan(w, 2, warmup + steps)[warmup:]
    assert run["algorithmic_bytes_per_launch"] == int(sum(b for _, b in plan) / steps)
    assert bench.traffic_from_profile(w, steps, warmup, 2) == run["hbm_bytes_per_launch"]
    assert bench.traffic_from_profile(w, steps + 1, warmup, 2) is None
