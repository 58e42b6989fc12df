"""Benchmark of quantized decode attention over a low-bit KV cache on one MI355X.

One step = one pass of the whole hot path over one batch: append one token per
sequence (residual copy; a flush when the residual fills) and decode attention
of one query per (sequence, query head) over sinks + quantized tokens +
residual, made with the library's one-call step (kvq_append_decode) except on
sink and flush steps, which take kvq_append + kvq_decode_attention.  Inputs are
resident in HBM before timing starts.

To measure HBM rather than the 256 MB MALL, the benchmark keeps L independent
caches of the same workload ("layers") whose combined size is at least three
times the MALL, and step s works on layer s mod L (as consecutive layers of a
model would): every step streams its layer's cache from HBM.

Prints one JSON line.  `value` is the effective KV bandwidth of the step:
algorithmic bytes of decode attention (packed codes, scales and zero points,
full-precision sinks and residual, q in and fp32 out) per step divided by the
wall time per step.  `roofline.achieved` uses the decode kernel's own duration:
on every EVENT_STRIDE-th timed step the launch records two HIP events at the
kernel's start and end (kvq_set_timing_events, hipExtLaunchKernel on the stream
the kernel runs on).  `decode_call_us` is the duration between events recorded
on the stream around the call, dispatch gaps included.  `stream_read_ceiling`
is the bandwidth of a plain streaming read of 2 GiB (the library's probe) on the
same device: an achievable ceiling beside the 8 TB/s peak, not the denominator.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as wl  # noqa: E402

METRIC = "effective KV GB/s (and % HBM peak) of quantized decode attention; tokens/s"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 * 2 ** 20
MAX_EVENT_STRIDE = 8
MIN_TIMED_LAUNCHES = 16
# the largest single-GPU workload (B32 H32 D128, context 8192, INT2: about 1.1 GB per call)
DEFAULT_WORKLOAD = "kivi2_long_batch"
DECODE_SOURCES = ["decode_impl.h", "decode_dispatch.h", "decode.hip", "kvq_internal.h",
                  "decode_b4_d128.hip", "decode_b2_d128.hip", "decode_b4_d64.hip", "decode_b2_d64.hip",
                  "decode_mf_b4_d128.hip", "decode_mf_b2_d128.hip", "decode_mf_b4_d64.hip", "decode_mf_b2_d64.hip",
                  "decode_mf_b8_d128.hip", "decode_mf_b8_d64.hip",
                  "decode_sp_b4_d128.hip", "decode_sp_b2_d128.hip", "decode_sp_b4_d64.hip", "decode_sp_b2_d64.hip",
                  "decode_mfsp_b4_d128.hip", "decode_mfsp_b2_d128.hip",
                  "decode_kt_b4_d128.hip", "decode_kt_b2_d128.hip", "decode_kt_b8_d128.hip",
                  "decode_kt_b4_d64.hip", "decode_kt_b2_d64.hip", "decode_kt_b8_d64.hip"]


def algorithmic_bytes(w: wl.Workload, n_sink: int, n_quant: int, n_resid: int) -> int:
    """Bytes the method itself must move for one decode-attention call."""
    D, e = w.head_dim, wl.elem_bytes(w.dtype)
    kmeta = n_quant * 2 * 4 if w.key_axis else (n_quant // w.k_group) * 2 * D * 4  # per token, or per channel
    per_slice = (n_quant * 2 * D * w.bits // 8                 # K and V codes
                 + kmeta                                         # K scale + zero
                 + n_quant * (D // w.v_group) * 2 * 4            # V scale + zero
                 + (n_sink + n_resid) * 2 * D * e)               # full-precision tokens
    if w.outliers:  # one per key channel group and per value group: fp32 value, place and code
        per_slice += (n_quant // w.k_group) * D * 6 + n_quant * (D // w.v_group) * 6
    return w.batch * w.n_kv_heads * per_slice + w.batch * w.n_q_heads * D * (e + 4)


def slice_counts(w: wl.Workload, n: int):
    """(sinks, quantized, residual) tokens of a sequence of n tokens: a flush when
    the residual holds R tokens quantizes all R, or W = R / 3 under log-sparse
    retention."""
    nS = min(n, w.n_sink)
    m, R, Q = n - nS, w.residual, w.log_window or w.residual
    Lq = 0 if m < R else ((m - R) // Q + 1) * Q
    return nS, Lq, m - Lq


def algorithmic_bytes_seqs(w: wl.Workload, lens) -> int:
    """algorithmic_bytes for sequences of the given lengths (one per sequence)."""
    per_seq = [algorithmic_bytes(w.replace(batch=1), *slice_counts(w, n)) for n in lens]
    return sum(per_seq)


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "bit_quantized_kv_kvq_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def n_layers(w: wl.Workload, layers: int = 0) -> int:
    """Caches rotated per step: enough that their combined decode traffic is three
    times the 256 MB MALL (layers = 0), or the given count."""
    if layers:
        return layers
    b0 = algorithmic_bytes_seqs(w, wl.prefill_lengths(w))
    return min(64, max(2, math.ceil(3 * MALL_BYTES / b0)))


def default_steps(w: wl.Workload, L: int) -> int:
    """Timed steps by default: every layer appends as many tokens as separate two
    flushes (R, or W under log-sparse retention), so the region holds each layer's
    residual flush once (its amortised share of the steps)."""
    return L * (w.log_window or w.residual)


def event_stride(steps: int) -> int:
    """Kernel events on every stride-th timed step: at most every 8th (timing every
    step lengthens the steps a little), and at least MIN_TIMED_LAUNCHES launches,
    or every launch when the region has fewer steps."""
    return max(1, min(MAX_EVENT_STRIDE, steps // MIN_TIMED_LAUNCHES))


def step_plan(w: wl.Workload, L: int, total_steps: int):
    """For each step s (warm-up steps first): whether the step is one fused launch
    (every sequence's token joins its residual without filling it) and the
    algorithmic bytes of its decode call (the cache state after the append)."""
    lens0 = wl.prefill_lengths(w)
    plan = []
    for s in range(total_steps):
        fused = True
        for n0 in lens0:
            nb = n0 + s // L          # this sequence's tokens before the append
            fused &= nb >= w.n_sink and slice_counts(w, nb)[2] + 1 < w.residual
        plan.append((fused, algorithmic_bytes_seqs(w, [n0 + s // L + 1 for n0 in lens0])))
    return plan


def traffic_path(w: wl.Workload) -> str:
    return os.path.join(ROOT, "profiles", "decode_traffic_%s.json" % w.name)


def traffic_from_profile(w: wl.Workload, steps: int, warmup: int, layers: int):
    """HBM bytes per timed decode launch, from the committed counter summary of a
    run of this exact schedule (workload, steps, warm-up, layers) on the current
    decode kernel source; else None."""
    path = traffic_path(w)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("decode_source_hash") != decode_source_hash():
        return None
    for r in t.get("runs", []):
        if (r["steps"], r["warmup"], r["layers"]) == (steps, warmup, layers):
            return r["hbm_bytes_per_launch"]
    return None


COPY_PROBE_BYTES = 1 << 30
READ_PROBE_BYTES = 1 << 31


def copy_probe(torch, dev, kvq):
    """Kernels of known traffic, ten dispatches each, so that rocprofv3's FETCH_SIZE /
    WRITE_SIZE per dispatch can be scaled to bytes: a plain device copy (1 GiB read,
    1 GiB written) and the library's streaming read (2 GiB read once, nothing
    written but one word)."""
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(10):
        torch.mul(src, 1.0, out=dst)
    del src, dst
    x = torch.ones(READ_PROBE_BYTES // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    sp = torch.cuda.current_stream().cuda_stream
    for _ in range(10):
        kvq.kvq_stream_read_probe(x.data_ptr(), READ_PROBE_BYTES, 4, sink.data_ptr(), sp)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": COPY_PROBE_BYTES, "copy_probe_bytes_written": COPY_PROBE_BYTES,
                      "read_probe_bytes_read": READ_PROBE_BYTES, "dispatches": 10}))


def stream_read_ceiling(torch, dev, kvq) -> dict:
    """Bandwidth of a plain streaming read of 2 GiB (kvq_stream_read_probe): the best,
    over 1 to 16 workgroups per CU, of the median of 7 timed reads."""
    nbytes = READ_PROBE_BYTES
    x = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    sp = torch.cuda.current_stream().cuda_stream
    best = None
    for bpc in (1, 2, 4, 8, 16):
        times = []
        for rep in range(9):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            kvq.kvq_stream_read_probe(x.data_ptr(), nbytes, bpc, sink.data_ptr(), sp)
            b.record()
            b.synchronize()
            if rep >= 2:
                times.append(a.elapsed_time(b))
        times.sort()
        ms = times[len(times) // 2]
        if best is None or ms < best[0]:
            best = (ms, bpc)
    del x
    return {"gbs": round(nbytes / (best[0] * 1e-3) / 1e9, 1),
            "kernel": "kvq_stream_read_probe over 2 GiB, %d workgroups per CU" % best[1],
            "ms": round(best[0], 4)}


def _counter_rows(path: str, name_part: str, counter: str) -> list:
    """Values of one counter for the dispatches of kernels whose name contains
    name_part, in dispatch order."""
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    rows.sort()
    return [v for _, v in rows]


def write_traffic(w: wl.Workload, steps: int, warmup: int, layers: int, dec_fetch: str, dec_write: str,
                  probe_fetch: str, copy_write: str):
    """Adds one schedule's HBM bytes per timed decode launch to the workload's
    traffic summary: the decode kernel's FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch; the mean over the last `steps` decode dispatches, i.e. the timed
    ones) scaled by what the same counters read for kernels of known traffic
    (FETCH_SIZE: the library's 2 GiB streaming read; WRITE_SIZE: the 1 GiB copy)."""
    L = n_layers(w, layers)
    f_dec = _counter_rows(dec_fetch, "decode_kernel", "FETCH_SIZE")[-steps:]
    w_dec = _counter_rows(dec_write, "decode_kernel", "WRITE_SIZE")[-steps:]
    assert len(f_dec) == steps and len(w_dec) == steps, (len(f_dec), len(w_dec), steps)
    f_rd = _counter_rows(probe_fetch, "stream_read_kernel", "FETCH_SIZE")
    f_cp = _counter_rows(probe_fetch, "elementwise", "FETCH_SIZE")
    w_cp = _counter_rows(copy_write, "elementwise", "WRITE_SIZE")
    mean = lambda v: sum(v) / len(v)
    k_fetch = READ_PROBE_BYTES / (mean(f_rd) * 1024.0)
    k_fetch_copy = COPY_PROBE_BYTES / (mean(f_cp) * 1024.0)
    k_write = COPY_PROBE_BYTES / (mean(w_cp) * 1024.0)
    plan = step_plan(w, L, warmup + steps)[warmup:]
    alg = sum(b for _, b in plan) / len(plan)
    run = {"steps": steps, "warmup": warmup, "layers": L,
           "fetch_kib_per_dispatch": mean(f_dec), "write_kib_per_dispatch": mean(w_dec),
           "hbm_bytes_per_launch": int(mean(f_dec) * 1024.0 * k_fetch + mean(w_dec) * 1024.0 * k_write),
           "algorithmic_bytes_per_launch": int(alg)}
    run["traffic_over_algorithmic"] = round(run["hbm_bytes_per_launch"] / alg, 4)
    path = traffic_path(w)
    old = {}
    if os.path.exists(path):
        with open(path) as f:
            old = json.load(f)
    runs = [r for r in old.get("runs", []) if old.get("decode_source_hash") == decode_source_hash()
            and (r["steps"], r["warmup"], r["layers"]) != (steps, warmup, L)]
    out = {"workload": w.name, "decode_source_hash": decode_source_hash(),
           "read_probe_fetch_kib": mean(f_rd), "read_probe_fetch_scale": k_fetch,
           "copy_probe_fetch_kib": mean(f_cp), "copy_probe_fetch_scale": k_fetch_copy,
           "copy_probe_write_kib": mean(w_cp), "write_scale": k_write,
           "runs": runs + [run]}
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


class HipEvents:
    """Timing events of the HIP runtime this process already uses (the one torch
    loaded), created without the system-scope fence that default events add
    (its cache write-back and invalidate would lengthen the timed kernels)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64.so" in l)
        self.lib = ctypes.CDLL(path)
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.lib.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e

    def record(self, e, stream):
        if self.lib.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, events):
        for e in events:
            self.lib.hipEventDestroy(e)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed(fn, budget_s: float):
    """Runs fn() repeatedly for about budget_s seconds (at least once); returns
    (seconds per run, runs)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return (time.perf_counter() - t0) / reps, reps


def cpu_baseline(w: wl.Workload, budget_s: float):
    """The oracle, as it is, on the host's cores, over a bounded sample of the
    workload's (sequence, kv-head) slices.  Three phases:
      - decode step: dequantize + binary64 attention of the sampled slices after
        the prefill (OpenMP across slices); `value` is its effective GB/s over the
        same algorithmic bytes as the GPU line;
      - prefill quantization: the oracle's cache build (one-token appends and the
        residual flushes) over the sampled slices' prefill tokens;
      - append and flush: the build of one residual's worth of tokens (R appends
        and one flush; the sinks first when the workload keeps them).
    The small workloads (tiny, Llama-7B-shaped) also time the decode step on one
    thread.  Slices run on a thread pool of the oracle's thread count (the C
    oracle releases the GIL); each phase gets a share of budget_s."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    threads = oracle.num_threads()
    n_slices_total = w.batch * w.n_kv_heads
    slices = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    g = w.gqa
    scale = oracle.default_scale(w.head_dim)
    # sample: as many slices as fit the decode share of the budget, measured on a probe
    probe = slices[:1]
    states = [oracle.slice_state(w, b, h, 0) for b, h in probe]
    qs = np.stack([np.stack([wl.storage_to_f32(wl.query_slice(w, b, h * g + j)[0], w.dtype)
                             for j in range(g)]) for b, h in probe])
    t0 = time.perf_counter()
    oracle.decode_slices(states, qs, scale)
    t_probe = max(time.perf_counter() - t0, 1e-4)
    n = int(min(n_slices_total, max(threads, 0.5 * budget_s / t_probe * threads)))
    sample = slices[:max(1, n)]
    lens = wl.prefill_lengths(w)
    # one batched oracle call per sequence (its slices share one length)
    groups = []
    for b in sorted({b for b, _ in sample}):
        hs = [h for bb, h in sample if bb == b]
        groups.append(([oracle.slice_state(w, b, h, 0) for h in hs],
                       np.stack([np.stack([wl.storage_to_f32(wl.query_slice(w, b, h * g + j)[0], w.dtype)
                                           for j in range(g)]) for h in hs])))

    def decode_step():
        for st_, q_ in groups:
            oracle.decode_slices(st_, q_, scale)

    dt, reps = _timed(decode_step, 0.5 * budget_s)
    # algorithmic bytes of the sampled slices (a sequence's bytes split evenly over its kv heads)
    full = algorithmic_bytes_seqs(w, lens)
    sampled = sum(algorithmic_bytes_seqs(w, [lens[b]]) / w.n_kv_heads for b, _ in sample)
    frac = sampled / full
    res = {"value": round(sampled / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "cpu_model": _cpu_model(),
           "sample": "decode step (dequantize + binary64 attention) of %d of %d (sequence, kv-head) "
                     "slices after the %d-token prefill, repeated %d times in %.1f s; %.4f s per "
                     "sampled step" % (len(sample), n_slices_total, w.prefill, reps, dt * reps, dt),
           "seconds_per_step_estimate": round(dt / frac, 4)}

    # prefill quantization and append/flush: the oracle's slice build from fp32 tokens
    def build(args):
        k, v = args
        return oracle.build_slice(k, v, head_dim=w.head_dim, bits=w.bits, k_group=w.k_group,
                                  v_group=w.v_group, residual=w.residual, n_sink=w.n_sink, codec=w.codec,
                                  log_window=w.log_window, outliers=w.outliers, key_axis=w.key_axis)

    toks = [oracle.slice_tokens_f32(w, b, h, 0) for b, h in sample[:threads]]
    with ThreadPoolExecutor(threads) as ex:
        dtp, rp = _timed(lambda: list(ex.map(build, toks)), 0.25 * budget_s)
        n_in = sum(k.shape[0] for k, _ in toks)
        e = wl.elem_bytes(w.dtype)
        res["prefill_quantize"] = {
            "slice_tokens_per_s": round(n_in / dtp, 1),
            "input_gb_per_s": round(n_in * 2 * w.head_dim * e / dtp / 1e9, 4),
            "sample": "%d slices x %d tokens, %d runs" % (len(toks), toks[0][0].shape[0], rp)}
        m = w.n_sink + w.residual
        short = [(k[:m], v[:m]) for k, v in toks]
        dta, ra = _timed(lambda: list(ex.map(build, short)), 0.1 * budget_s)
        res["append_flush"] = {
            "us_per_token": round(dta / (len(short) * m) * threads * 1e6, 3),
            "sample": "%d slices x (%d appends incl. one flush of %d tokens), %d runs, %d threads; "
                      "per token per thread" % (len(short), m, w.residual, ra, threads)}
    if w.name in ("tiny", "llama7b_mha_int4"):
        oracle.set_num_threads(1)
        try:
            dt1, r1 = _timed(decode_step, 0.15 * budget_s)
        finally:
            oracle.set_num_threads(threads)
        res["decode_step_1_thread"] = {"value": round(sampled / dt1 / 1e9, 4), "unit": "GB/s",
                                       "seconds_per_sampled_step": round(dt1, 5), "runs": r1}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: layers x residual, one flush per layer)")
    # enough warm-up steps for the GPU clocks to settle (short bursts run slower)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--layers", type=int, default=0, help="caches rotated per step (0 = auto)")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed decode calls before the warm-up steps, to bring the GPU to its "
                         "steady clock (they leave every cache unchanged)")
    ap.add_argument("--cpu-budget", type=float, default=16.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only kernels of known traffic (calibrates the HBM byte counters)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("DECODE_FETCH", "DECODE_WRITE", "PROBE_FETCH",
                                                         "COPY_WRITE"),
                    help="add this schedule (--workload, --steps, --warmup, --layers) to "
                         "profiles/decode_traffic_<workload>.json from rocprofv3 --pmc "
                         "counter_collection.csv files of the bench and of --copy-probe (no GPU)")
    args = ap.parse_args()
    w = wl.get(args.workload)
    L = n_layers(w, args.layers)
    if args.steps is None:
        args.steps = default_steps(w, L)

    if args.write_traffic:
        write_traffic(w, args.steps, args.warmup, args.layers, *args.write_traffic)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this path runs on one GPU; a run on %d GPUs is not provided "
              "(the decode shards with no exchange over (sequence, kv-head) slices)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_kv_kvq_amd as kvq
    from workloads.torch_io import TORCH_DTYPES, to_torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_probe:
        copy_probe(torch, dev, kvq)
        return

    lens0 = wl.prefill_lengths(w)
    ragged = len(set(lens0)) > 1
    total_steps = args.warmup + args.steps
    per_layer_steps = (total_steps + L - 1) // L
    max_tokens = w.prefill + per_layer_steps

    print("bench: workload %s, %d layers, %d warmup + %d timed steps" %
          (w.name, L, args.warmup, args.steps), file=sys.stderr, flush=True)
    Kp, Vp = wl.prefill_batch(w)
    Kd, Vd = to_torch(Kp, w.dtype, dev), to_torch(Vp, w.dtype, dev)
    del Kp, Vp
    # paged records: a pool of exactly the pages the sequences reach in the run
    pool_pages = 0
    if w.page_groups:
        pool_pages = sum(-(-(slice_counts(w, n0 + per_layer_steps)[1] // w.k_group) // w.page_groups)
                         for n0 in lens0)
    rounds = wl.prefill_rounds(w)
    caches = []
    for _ in range(L):
        c = kvq.Cache(batch=w.batch, n_kv_heads=w.n_kv_heads, n_q_heads=w.n_q_heads,
                      head_dim=w.head_dim, bits=w.bits, k_group=w.k_group, v_group=w.v_group,
                      residual=w.residual, n_sink=w.n_sink, dtype=TORCH_DTYPES[w.dtype],
                      max_tokens=max_tokens, device=dev, codec=w.codec,
                      retention=kvq.KVQ_RETAIN_LOG if w.log_window else kvq.KVQ_RETAIN_WINDOW,
                      page_groups=w.page_groups, pool_pages=pool_pages, outliers=w.outliers,
                      key_axis=w.key_axis)
        if args.split_tokens:
            c.set_split_tokens(args.split_tokens)
        if len(rounds) == 1 and not ragged:
            c.append(Kd, Vd)
        else:  # in the workload's prefill rounds
            for t0, n_new in rounds:
                n = max(n_new)
                c.append_ragged(Kd[:, :, t0:t0 + n].contiguous(), Vd[:, :, t0:t0 + n].contiguous(), n_new)
        caches.append(c)
    del Kd, Vd
    Ks, Vs = wl.steps_batch(w)
    Ks = to_torch(Ks, w.dtype, dev)[:, :, :, None].contiguous()   # [steps, B, Hkv, 1, D]
    Vs = to_torch(Vs, w.dtype, dev)[:, :, :, None].contiguous()
    Q = to_torch(wl.queries_batch(w), w.dtype, dev)                 # [nq, B, Hq, D]
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.n_q_heads), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    print("bench: caches ready", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    hip = HipEvents()
    # Every stride-th timed step, the library records two events at the start and
    # end of the decode kernel itself (kvq_set_timing_events); these give the
    # kernel duration of the roofline.  Half a stride later, two events recorded on
    # the stream around the call give the call's duration, dispatch gaps included
    # (reported beside it).
    stride = event_stride(args.steps)
    timed_steps = [k for k in range(args.steps) if k % stride == 0]
    call_steps = [k for k in range(args.steps) if k % stride == stride // 2]
    ev = {k: (hip.create(), hip.create()) for k in timed_steps}
    ev_call = {k: (hip.create(), hip.create()) for k in call_steps}

    # The timed loop calls the C-ABI directly with arguments prepared here, so that
    # the host enqueues a step faster than the GPU runs it: the GPU never waits
    # for the host inside the timed region, and the events around each decode
    # time the kernel alone.
    lib = kvq.lib()
    append_fn, decode_fn = lib.kvq_append, lib.kvq_decode_attention
    fused_fn = lib.kvq_append_decode
    set_events = lib.kvq_set_timing_events
    sp = ctypes.c_void_p(stream.cuda_stream)
    out_p, lse_p = ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr())
    # The step is one kvq_append_decode call when every sequence's token joins its
    # residual without filling it; otherwise (a sink or a flush somewhere) the
    # library appends and decodes in two launches, and the bench makes the same two
    # calls itself so that the events bracket the decode alone.
    schedule = step_plan(w, L, total_steps)
    plan, step_bytes = [], []
    for s_, (fused, nbytes) in enumerate(schedule):
        c = caches[s_ % L]
        i = (s_ // L) % w.steps
        plan.append((fused, ctypes.c_void_p(c.handle), ctypes.c_void_p(Ks[i].data_ptr()),
                     ctypes.c_void_p(Vs[i].data_ptr()), ctypes.c_void_p(Q[i % Q.shape[0]].data_ptr()),
                     ctypes.c_void_p(c._ws_ptr), c.ws_bytes))
        step_bytes.append(nbytes)

    def step(s: int, k):
        fused, h, kp, vp, qp, wsp, wsb = plan[s]
        if not fused:
            st = append_fn(h, kp, vp, 1, sp)
            if st:
                raise kvq.KVQError(st, kvq.kvq_last_error())
        if k in ev:
            set_events(h, ev[k][0], ev[k][1])
        if k in ev_call:
            hip.record(ev_call[k][0], sp)
        if fused:
            st = fused_fn(h, kp, vp, qp, out_p, lse_p, wsp, wsb, sp)
        else:
            st = decode_fn(h, qp, out_p, lse_p, wsp, wsb, sp)
        if st:
            raise kvq.KVQError(st, kvq.kvq_last_error())
        if k in ev:
            set_events(h, None, None)
        if k in ev_call:
            hip.record(ev_call[k][1], sp)

    # Clock settling: decode calls of every layer with the first query, which read
    # the caches and change nothing, until settle_ms have passed.
    t_set = time.perf_counter()
    while (time.perf_counter() - t_set) * 1e3 < args.settle_ms:
        for c in caches:
            st = decode_fn(ctypes.c_void_p(c.handle), ctypes.c_void_p(Q[0].data_ptr()), out_p, lse_p,
                           ctypes.c_void_p(c._ws_ptr), c.ws_bytes, sp)
            if st:
                raise kvq.KVQError(st, kvq.kvq_last_error())
        torch.cuda.synchronize()
    for s in range(args.warmup):
        step(s, None)
    torch.cuda.synchronize()
    # the cache state the schedule predicts is the one the library reports
    for li, c in enumerate(caches):
        n_done = len(range(li, args.warmup, L))
        assert c.seq_lengths() == [n0 + n_done for n0 in lens0], (li, c.seq_lengths())
        n = w.prefill + n_done
        assert tuple(c.state()) == (n,) + slice_counts(w, n), (li, c.state())
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k, k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_bytes = step_bytes[args.warmup:]

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    dec_ms = [hip.elapsed_ms(*ev[k]) for k in timed_steps]
    call_ms = [hip.elapsed_ms(*ev_call[k]) for k in call_steps]
    hip.destroy([e for d in (ev, ev_call) for pair in d.values() for e in pair])
    dec_avg_ms = sum(dec_ms) / len(dec_ms)
    bytes_avg = sum(step_bytes) / len(step_bytes)
    value = bytes_avg / (ms_per_step * 1e-3) / 1e9
    timed_bytes = [step_bytes[k] for k in timed_steps]
    launch_bytes = sum(timed_bytes) / len(timed_bytes)
    achieved = sum(timed_bytes) / (sum(dec_ms) * 1e-3) / 1e9
    traffic = traffic_from_profile(w, args.steps, args.warmup, L)

    ceiling = stream_read_ceiling(torch, dev, kvq)

    cpu = None
    if args.cpu_budget > 0:
        print("bench: CPU baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_budget)

    mf = (w.gqa >= 2 or w.bits == 8) and w.k_group >= 64 and w.v_group >= 64
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # what the path computes in: packed integer codes times a fixed-point image
        # (2^-19 relative) of the folded query and of the softmax weights, summed in
        # int32; scales, softmax and accumulation in fp32
        "dtype": "int%d codes x fixed-point, int32 %s; f32 softmax" % (
            w.bits, "MFMA" if mf else "dot products"),
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_kv_heads": w.n_kv_heads,
                   "n_q_heads": w.n_q_heads, "head_dim": w.head_dim, "context": w.prefill,
                   **({"contexts": lens0} if ragged else {}),
                   "bits": w.bits, "k_group": w.k_group, "v_group": w.v_group,
                   "residual": w.residual, "n_sink": w.n_sink, "storage": w.dtype,
                   "codec": "symmetric" if w.codec else "asymmetric",
                   **({"retention": "log-sparse", "log_window": w.log_window} if w.log_window else {}),
                   **({"outliers": "one per quantization vector"} if w.outliers else {}),
                   **({"keys": "per token over head_dim (head-granular)"} if w.key_axis else {}),
                   **({"page_groups": w.page_groups, "pool_pages": pool_pages,
                       "prefill_chunk": w.prefill_chunk} if w.page_groups else {}),
                   "layers_rotated": L, "parallelism": "single GPU"},
        "tokens_per_s": round(w.batch / (ms_per_step * 1e-3), 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_kernel_us": round(dec_avg_ms * 1e3, 3),
        "decode_call_us": round(sum(call_ms) / max(1, len(call_ms)) * 1e3, 3),
        "stream_read_ceiling": ceiling,
        "frac_of_stream_ceiling": round(achieved / ceiling["gbs"], 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(launch_bytes),
                     "timed_launches": len(timed_steps)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
