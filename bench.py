#!/usr/bin/env python3
"""Benchmark of dense MLA decode on one MI355X; prints one JSON line.

A step is one decode call (split-KV kernel + combine kernel) over one batch of
the synthetic workload, inputs resident in HBM.  Steps run from a HIP graph,
as serving engines run decode (the attention-kernel page's CUDA-graph
section), over several rotating copies of q and the KV pool so that the
256 MB memory-side cache cannot hand one step's pages to the next.  The tile
plan is made once per decode step and reused by every call of that step (the
pages prescribe this for all layers of a decode step); its host time is
reported separately as ``plan_us``.

Per workload the line carries:
  * the timed region: exactly --steps steps (one replay of a graph of that
    many steps, synchronised on both sides), which gives ``value``;
  * the spread over at least 100 further steps (replays of the same graph):
    median, p10 and p90 of the per-step time;
  * the GPU clock the firmware reported while those steps ran;
  * per-kernel durations (split-KV and combine) from HIP events the library
    attaches to each dispatch, enqueued behind a warm graph replay;
  * rooflines: the split-KV kernel's and the whole step's rate against the
    nominal peak, the attainable roof min(MFMA peak, HBM peak x intensity)
    and the measured read ceilings (a streaming read of the same bytes and a
    2 GB streaming read, from the measurement library);
  * the CPU oracle on a bounded sample of the same workload.

Headline workload: TP-sharded memory-bound decode (batch 16, h_q 16,
L ~ U[1024, 4096]) -> effective HBM GB/s.  The h_q = 128 workloads
(compute-bound, ragged MTP with and without the causal mask, long context),
the sparse workload and the FP8-cache lines are reported under ``extra``.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import threading
import time

import numpy as np

METRIC = "MLA decode TFLOPs (h_q=128) and effective HBM GB/s (h_q=16), 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRCS = [os.path.join(ROOT, "decode_attention_mla_amd", "csrc", f) for f in ("mla_kernels.h", "mla_internal.h")]
MIN_SPREAD_STEPS = 100


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash() -> str:
    """First 16 hex digits of the sha256 of the kernels' code (comments and
    whitespace dropped, so that rewording a comment keeps the committed
    counter measurements valid)."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        h.update(_code_only(open(path).read()).encode())
    return h.hexdigest()[:16]


def main_kernel_name(rows: int, sparse: bool = False, fp8: bool = False) -> str:
    """The split-KV kernel the library launches for h_q * s_q = rows."""
    sp, f8 = ("true" if sparse else "false"), ("true" if fp8 else "false")
    if rows <= 16:
        return f"mla_splitkv_small_kernel<{sp}, {f8}>"
    if rows >= 128 or sparse or fp8:
        return f"mla_splitkv_wide_kernel<{'true' if rows <= 128 else 'false'}, {sp}, {f8}>"
    return "mla_splitkv_kernel"


def measured_traffic(config_name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    e = d.get(config_name)
    if not e or e.get("kernel_sha256_16") != kernel_hash():
        return None
    return e.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# Clock sampling (firmware-averaged graphics clock, read through amdsmi)

class ClockSampler:
    """Samples the GPU's reported graphics clock every ~2 ms in a background
    thread while active; ``mhz()`` returns the median of the samples taken
    (None if the metrics cannot be read on this machine)."""

    def __init__(self):
        self.handle = None
        self.samples = []
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            if hs:
                self.handle = hs[0]
                self._amdsmi = amdsmi
                self._read()
        except Exception as e:   # pragma: no cover - depends on the machine
            log(f"[bench] clock sampling unavailable: {e}")
            self.handle = None

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        for key in ("current_gfxclk", "average_gfxclk_frequency"):
            v = m.get(key)
            if isinstance(v, (int, float)) and 0 < v < 10000:
                return float(v)
        v = m.get("current_gfxclks")
        if isinstance(v, (list, tuple)):
            vals = [float(x) for x in v if isinstance(x, (int, float)) and 0 < x < 10000]
            if vals:
                return float(np.mean(vals))
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v is not None:
                    self.samples.append(v)
            except Exception:
                pass
            time.sleep(0.002)

    def start(self):
        self.samples = []
        if self.handle is None:
            return
        self._stop.clear()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None
        return self.mhz()

    def mhz(self):
        return float(np.median(self.samples)) if self.samples else None

    def spread(self):
        """[p10, p90, number of samples] of the last run's readings (None if none)."""
        if not self.samples:
            return None
        return [float(np.percentile(self.samples, 10)), float(np.percentile(self.samples, 90)), len(self.samples)]


CLOCK = None


# ---------------------------------------------------------------------------
# Timing

def time_steps(step, rot: int, steps: int, warmup: int):
    """Times decode calls ``step(i)`` (i picks the rotating input copy):

    * warm-up: ``warmup`` eager steps, then untimed replays of the graph
      (about 30 ms of GPU time, so the clock has left its idle state);
    * timed region: one replay of a graph of exactly ``steps`` steps,
      synchronised on both sides; GPU time from events on the capture
      stream, host wall time beside it;
    * spread: further replays of that graph until at least 100 steps have
      run, one per-step time per replay -> median, p10, p90; the GPU clock
      is sampled meanwhile;
    * kernels: ``steps`` eager calls with the library's per-kernel HIP events
      (recorded by the dispatches themselves), enqueued behind a graph replay
      so the GPU is busy and the host ahead -> average main / combine kernel
      durations;
    * eager: plain back-to-back calls from Python, wall clock (reference)."""
    import torch
    import decode_attention_mla_amd as mla
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step(0)                       # warm the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            for i in range(steps):
                step(i % rot)
    torch.cuda.synchronize()
    # untimed warm replays, about 30 ms of GPU time, so that the clock has
    # left its idle state before the timed region
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    graph.replay()
    ev[1].record()
    torch.cuda.synchronize()
    for _ in range(min(200, int(np.ceil(30.0 / max(ev[0].elapsed_time(ev[1]), 1e-3))))):
        graph.replay()
    torch.cuda.synchronize()
    # --- timed region: exactly `steps` steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(s):
        ev[0].record(s)
        graph.replay()
        ev[1].record(s)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    timed_ms = ev[0].elapsed_time(ev[1])
    # --- spread: at least 100 steps and about 50 ms of GPU time (so that the
    # clock sampler sees the run)
    reps = max(3, -(-MIN_SPREAD_STEPS // steps), int(np.ceil(50.0 / max(timed_ms, 1e-3))))
    reps = min(reps, 400)
    per = []
    if CLOCK is not None:
        CLOCK.start()
    with torch.cuda.stream(s):
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            graph.replay()
            b.record(s)
            per.append((a, b))
    torch.cuda.synchronize()
    clock = CLOCK.stop() if CLOCK is not None else None
    clock_spread = CLOCK.spread() if CLOCK is not None else None
    per_step = np.array([a.elapsed_time(b) / steps for a, b in per])
    # --- per-kernel durations: eager calls behind a warm replay, five blocks
    # of `steps` calls; the median of the blocks' means (one slow block, e.g.
    # a clock change, does not move it)
    blocks = []
    for _ in range(5):
        with torch.cuda.stream(s):
            graph.replay()
            mla.profile_start(steps)
            for i in range(steps):
                step(i % rot)
            main_ms, comb_ms, calls = mla.profile_stop()
        torch.cuda.synchronize()
        assert calls == steps, (calls, steps)
        blocks.append((main_ms / calls, comb_ms / calls))
    main_ms = float(np.median([b[0] for b in blocks])) * steps
    comb_ms = float(np.median([b[1] for b in blocks])) * steps
    calls = steps
    del graph
    t0 = time.perf_counter()
    for i in range(steps):
        step(i % rot)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps
    return dict(ms_per_step=timed_ms / steps, wall_ms_per_step=wall_ms / steps,
                spread_steps=int(reps * steps), median_ms=float(np.median(per_step)),
                p10_ms=float(np.percentile(per_step, 10)), p90_ms=float(np.percentile(per_step, 90)),
                main_kernel_ms=main_ms / calls, combine_kernel_ms=comb_ms / calls, eager_ms_per_step=eager_ms,
                clock_mhz=clock, clock_mhz_p10_p90_n=clock_spread)


# ---------------------------------------------------------------------------
# Read ceilings and launch cost (measurement library)

def _bench_lib():
    from decode_attention_mla_amd import build
    if not os.path.exists(build.BENCH_LIB_PATH):
        raise RuntimeError(f"{build.BENCH_LIB_PATH} is missing: build it with __graft_entry__.build()")
    B = ctypes.CDLL(build.BENCH_LIB_PATH)
    B.mla_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p]
    B.mla_bench_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
    B.mla_bench_last_error.restype = ctypes.c_char_p
    return B


def _graph_time(fn, reps=20):
    """Per-call GPU time of fn(stream) captured once in a graph of 8 calls."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for i in range(8):
            fn(i, s.cuda_stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(8):
                fn(i, s.cuda_stream)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    out = []
    with torch.cuda.stream(s):
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            g.replay()
            b.record(s)
            out.append((a, b))
    torch.cuda.synchronize()
    del g
    return float(np.median([a.elapsed_time(b) / 8 for a, b in out]))


_CEILINGS = {}


def read_ceiling(nbytes: int):
    """Streaming read of nbytes, eight rotating buffers in a graph (so each
    read comes mostly from HBM, as a decode step's pages do): GB/s and us."""
    import torch
    key = int(nbytes)
    if key in _CEILINGS:
        return _CEILINGS[key]
    B = _bench_lib()
    dev = torch.device("cuda", 0)
    n = (key + 15) // 16 * 16
    bufs = [torch.full((n,), 3, dtype=torch.uint8, device=dev) for _ in range(8)]
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)

    def fn(i, st):
        rc = B.mla_bench_stream_read(bufs[i].data_ptr(), n, sink.data_ptr(), 2048, st)
        assert rc == 0, B.mla_bench_last_error()
    ms = _graph_time(fn)
    del bufs
    torch.cuda.empty_cache()
    _CEILINGS[key] = dict(bytes=n, us=ms * 1e3, gbs=n / (ms * 1e-3) / 1e9)
    return _CEILINGS[key]


def sustained_read_ceiling():
    """One streaming read of 2 GiB (a multiple of the memory-side cache):
    the sustained HBM read rate, GB/s."""
    import torch
    B = _bench_lib()
    dev = torch.device("cuda", 0)
    n = 2 << 30
    buf = torch.full((n,), 3, dtype=torch.uint8, device=dev)
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    ts = []
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        assert B.mla_bench_stream_read(buf.data_ptr(), n, sink.data_ptr(), 4096, st) == 0
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    del buf
    torch.cuda.empty_cache()
    ms = float(np.median(ts[1:]))
    return dict(bytes=n, us=ms * 1e3, gbs=n / (ms * 1e-3) / 1e9)


def empty_launch_us():
    """GPU time of one empty 256-workgroup kernel in a graph (the fixed cost
    of a kernel node)."""
    B = _bench_lib()
    return _graph_time(lambda i, st: B.mla_bench_empty(256, st)) * 1e3


# ---------------------------------------------------------------------------
# CPU oracle baseline

def cpu_info():
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return cores, model


def cpu_baseline(run_request, work_of, nreq: int, scale: float, unit: str, budget_s: float):
    """The oracle, as it stands, on this host's cores: whole requests in
    order (wrapping around) until about budget_s of wall time; returns the
    algorithmic work done / seconds / scale."""
    import oracle  # noqa: F401  (the oracle package is imported by the callers' closures)
    from threadpoolctl import threadpool_limits
    cores, model = cpu_info()
    with threadpool_limits(limits=cores):
        done, work, t0 = 0, 0.0, time.perf_counter()
        while True:
            r = done % nreq
            run_request(r)
            work += work_of(r)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    return dict(value=work / el / scale, unit=unit, cores=cores, kind="oracle", cpu_model=model,
                sample=f"{done} request(s) of the workload (whole requests in order) in {el:.1f}s; "
                       f"float64 NumPy oracle, {cores} BLAS threads")


# ---------------------------------------------------------------------------
# Workloads

def _rooflines(flops, nbytes, step_ms, main_ms, spread, ceil_same, ceil_sustained):
    """Rates of the step and of the split-KV kernel against the nominal
    peaks, the attainable roof and the measured read ceilings."""
    inten = flops / nbytes
    attain_tf = min(MFMA_PEAK_TFLOPS, HBM_PEAK_GBS * inten / 1e3)
    out = {}
    for tag, ms in (("step", step_ms), ("main_kernel", main_ms), ("step_median", spread)):
        tf = flops / (ms * 1e-3) / 1e12
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[tag] = dict(ms=ms, tflops=tf, gbs=gbs, frac_mfma_peak=tf / MFMA_PEAK_TFLOPS,
                        frac_hbm_peak=gbs / HBM_PEAK_GBS, frac_attainable=tf / attain_tf,
                        frac_read_ceiling_same_bytes=gbs / ceil_same["gbs"] if ceil_same else None,
                        frac_read_ceiling_sustained=gbs / ceil_sustained["gbs"] if ceil_sustained else None)
    out["intensity_flop_per_byte"] = inten
    out["attainable_tflops"] = attain_tf
    out["bound_at_nominal_peaks"] = "mfma" if MFMA_PEAK_TFLOPS <= HBM_PEAK_GBS * inten / 1e3 else "hbm"
    return out


def run_workload(idx: int, steps: int, warmup: int, min_rot_bytes: float = 640e6, causal: bool = False,
                 fp8: bool = False, cpu_budget: float = 0.0):
    """Times one dense workload (see time_steps), one step per rotating copy
    of q and the KV pool so that no step finds its pages in cache."""
    import torch
    import decode_attention_mla_amd as mla
    from decode_attention_mla_amd import workloads as W

    t = time.perf_counter()
    inp = W.config_inputs(idx)
    log(f"[bench] config {idx} {inp.name}: inputs drawn in {time.perf_counter() - t:.1f}s")
    kv_row = W.FP8_RECORD if fp8 else 2 * W.D_QK
    flops, nbytes = W.algorithmic_work(inp.cache_seqlens, inp.s_q, inp.h_q, causal=causal, kv_row_bytes=kv_row)
    dev = torch.device("cuda", 0)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    rec = W.to_fp8_records(inp.kv_cache) if fp8 else None
    kv0 = torch.from_numpy(rec).to(dev) if fp8 else bf16(inp.kv_cache)
    q0 = bf16(inp.q)
    kv_bytes = kv0.numel() * kv0.element_size()
    rot = int(min(8, max(1, np.ceil(min_rot_bytes / kv_bytes))))
    kvs = [kv0] + [kv0.clone() for _ in range(rot - 1)]
    qs = [q0] + [q0.clone() for _ in range(rot - 1)]
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl = torch.from_numpy(inp.cache_seqlens).to(dev)

    # Plan once per decode step (host), timed separately; the plan carries
    # each part's first page (the step's block table is known when it is
    # planned, and every layer of the step shares both).
    reps = 50
    nblocks = int(inp.kv_cache.shape[0])
    t = time.perf_counter()
    for _ in range(reps):
        sched_np, ns_np, total = mla.get_mla_metadata_host(inp.cache_seqlens, inp.h_q, inp.s_q, fp8=fp8,
                                                           block_table=inp.block_table, num_blocks=nblocks)
    plan_us = (time.perf_counter() - t) / reps * 1e6
    sched = torch.from_numpy(sched_np).to(dev)
    ns = torch.from_numpy(ns_np).to(dev)
    # The same plan on the GPU (device lengths; capturable with the decode),
    # timed as graph replays of 20 planner launches (no host launch cost).
    mla.get_mla_metadata_device(sl, inp.h_q, inp.s_q, fp8=fp8, block_table=bt, num_blocks=nblocks)
    torch.cuda.synchronize()
    plan_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(plan_graph):
        for _ in range(20):
            mla.get_mla_metadata_device(sl, inp.h_q, inp.s_q, fp8=fp8, block_table=bt, num_blocks=nblocks)
    plan_graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        plan_graph.replay()
    e1.record()
    torch.cuda.synchronize()
    plan_device_us = e0.elapsed_time(e1) / 100 * 1e3
    del plan_graph
    b = inp.batch
    out = torch.empty((b, inp.s_q, inp.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((b, inp.h_q, inp.s_q), dtype=torch.float32, device=dev)
    ws = torch.empty(max(256, mla.mla_workspace_bytes(sched.shape[0] + b - 1, inp.h_q, inp.s_q)),
                     dtype=torch.uint8, device=dev)

    def step(i):
        mla.mla_decode_fwd(qs[i % rot], kvs[i % rot], bt, sl, inp.softmax_scale, sched, ns, out=out, lse=lse,
                           workspace=ws, causal=causal, fp8=fp8)

    tm = time_steps(step, rot, steps, warmup)
    del kvs, qs
    torch.cuda.empty_cache()
    ceil_same = read_ceiling(int(nbytes))
    roof = _rooflines(flops, nbytes, tm["ms_per_step"], tm["main_kernel_ms"], tm["median_ms"], ceil_same,
                      SUSTAINED)
    res = dict(workload=inp.name + ("_causal" if causal else "") + ("_fp8" if fp8 else ""), batch=b, s_q=inp.s_q,
               h_q=inp.h_q, sum_seqlen=int(inp.cache_seqlens.sum()), parts=int(sched.shape[0]),
               total_splits=int(total), rotating_copies=rot, flops=flops, bytes=nbytes, plan_us=plan_us,
               plan_device_us=plan_device_us, kernel=main_kernel_name(inp.h_q * inp.s_q, fp8=fp8),
               read_ceiling_same_bytes=ceil_same, **tm, roofline=roof)
    if cpu_budget > 0:
        import oracle
        kv_o = oracle.dequantize_fp8_cache(rec) if fp8 else inp.kv_cache
        per_req = [W.algorithmic_work(inp.cache_seqlens[i:i + 1], inp.s_q, inp.h_q, causal=causal,
                                      kv_row_bytes=kv_row) for i in range(b)]
        hbm = inp.h_q * inp.s_q <= 64
        res["cpu_baseline"] = cpu_baseline(
            lambda r: oracle.mla_decode(inp.q, kv_o, inp.block_table, inp.cache_seqlens, inp.softmax_scale,
                                        requests=[r], causal=causal),
            (lambda r: per_req[r][1]) if hbm else (lambda r: per_req[r][0]), b,
            1e9 if hbm else 1e12, "GB/s" if hbm else "TFLOP/s", cpu_budget)
    log(f"[bench] config {idx}{' causal' if causal else ''}{' fp8' if fp8 else ''}: step {tm['ms_per_step'] * 1e3:.2f} us "
        f"(median {tm['median_ms'] * 1e3:.2f}, p10 {tm['p10_ms'] * 1e3:.2f}, p90 {tm['p90_ms'] * 1e3:.2f}), main "
        f"{tm['main_kernel_ms'] * 1e3:.2f} us, combine {tm['combine_kernel_ms'] * 1e3:.2f} us, clock {tm['clock_mhz']}")
    return inp, res


def run_sparse_workload(steps: int, warmup: int, min_rot_bytes: float = 640e6, fp8: bool = False,
                        cpu_budget: float = 0.0):
    """Times the sparse workload (batch 128, s_q 2, h_q 128, topk 2048; each
    query token's 2048 keys drawn from its request's 4096..8192-token
    context) the same way as the dense ones."""
    import torch
    import decode_attention_mla_amd as mla
    from decode_attention_mla_amd import workloads as W

    t = time.perf_counter()
    inp = W.sparse_config_inputs()
    log(f"[bench] sparse {inp.name}: inputs drawn in {time.perf_counter() - t:.1f}s")
    kv_row = W.FP8_RECORD if fp8 else 2 * W.D_QK
    flops, nbytes = W.sparse_algorithmic_work(inp.indices, inp.h_q, inp.topk_length, kv_row_bytes=kv_row)
    dev = torch.device("cuda", 0)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    rec = W.to_fp8_records(inp.kv_cache) if fp8 else None
    kv0 = torch.from_numpy(rec).to(dev) if fp8 else bf16(inp.kv_cache)
    q0 = bf16(inp.q)
    rot = int(min(8, max(1, np.ceil(min_rot_bytes / (kv0.numel() * kv0.element_size())))))
    kvs = [kv0] + [kv0.clone() for _ in range(rot - 1)]
    qs = [q0] + [q0.clone() for _ in range(rot - 1)]
    idx = torch.from_numpy(inp.indices).to(dev)
    sched, ns = mla.get_mla_metadata_sparse(inp.topk_length, inp.batch, inp.s_q, inp.h_q, inp.topk)
    n = inp.batch * inp.s_q
    out = torch.empty((inp.batch, inp.s_q, inp.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((inp.batch, inp.h_q, inp.s_q), dtype=torch.float32, device=dev)
    ws = torch.empty(max(256, mla.mla_workspace_bytes(sched.shape[0] + n - 1, inp.h_q, 1)), dtype=torch.uint8,
                     device=dev)

    def step(i):
        mla.mla_decode_sparse_fwd(qs[i % rot], kvs[i % rot], idx, inp.softmax_scale, sched, ns, out=out, lse=lse,
                                  workspace=ws, fp8=fp8)

    tm = time_steps(step, rot, steps, warmup)
    del kvs, qs
    torch.cuda.empty_cache()
    ceil_same = read_ceiling(int(nbytes))
    roof = _rooflines(flops, nbytes, tm["ms_per_step"], tm["main_kernel_ms"], tm["median_ms"], ceil_same,
                      SUSTAINED)
    res = dict(workload=inp.name + ("_fp8" if fp8 else ""), batch=inp.batch, s_q=inp.s_q, h_q=inp.h_q, topk=inp.topk,
               parts=int(sched.shape[0]), total_splits=int(ns[-1].item()), rotating_copies=rot, flops=flops,
               bytes=nbytes, kernel=main_kernel_name(inp.h_q, sparse=True, fp8=fp8),
               read_ceiling_same_bytes=ceil_same, **tm, roofline=roof)
    if cpu_budget > 0:
        import oracle
        kv_o = oracle.dequantize_fp8_cache(rec) if fp8 else inp.kv_cache
        unit_flops = flops / max(1, n)   # every list holds topk keys here

        def one(r):
            bi, si = divmod(r, inp.s_q)
            qrows = oracle.bf16_to_f64(inp.q[bi, si])
            oracle.attend(qrows, oracle.sparse_keys(kv_o, inp.indices[bi, si], inp.topk), inp.softmax_scale)
        res["cpu_baseline"] = cpu_baseline(one, lambda r: unit_flops, n, 1e12, "TFLOP/s", cpu_budget)
    log(f"[bench] sparse{' fp8' if fp8 else ''}: step {tm['ms_per_step'] * 1e3:.2f} us (median "
        f"{tm['median_ms'] * 1e3:.2f}), main {tm['main_kernel_ms'] * 1e3:.2f} us, clock {tm['clock_mhz']}")
    return inp, res


SUSTAINED = None


def _extra_entry(r):
    """The per-workload record under ``extra`` (everything but the raw inputs)."""
    return {k: v for k, v in r.items()}


def main():
    global CLOCK, SUSTAINED
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2,
                    help="headline workload (1..5); 6 times the sparse workload alone, 7 workload 2 on an FP8 "
                         "cache and 8 the sparse workload on an FP8 cache (for profiling)")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time for the headline")
    ap.add_argument("--extra-cpu-budget", type=float, default=3.0, help="seconds of oracle time per extra workload")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the decode path is single-GPU); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import decode_attention_mla_amd as mla
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mla.lib()
    CLOCK = ClockSampler()
    if args.config in (6, 7, 8):   # profiling entry points: one workload, no headline line
        SUSTAINED = None
        if args.config == 7:
            _, r = run_workload(2, args.steps, args.warmup, fp8=True)
            metric, value, unit = "decode GB/s, FP8 cache", r["bytes"] / (r["ms_per_step"] * 1e-3) / 1e9, "GB/s"
        else:
            _, r = run_sparse_workload(args.steps, args.warmup, fp8=args.config == 8)
            metric, value, unit = "sparse decode TFLOP/s", r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12, "TFLOP/s"
        print(json.dumps(dict(metric=metric, value=value, unit=unit, n_gpus=1, steps=args.steps, warmup=args.warmup,
                              ms_per_step=r["ms_per_step"], higher_is_better=True, dtype="bf16", data="synthetic",
                              detail=r)), flush=True)
        return

    SUSTAINED = sustained_read_ceiling()
    empty_us = empty_launch_us()
    log(f"[bench] sustained read {SUSTAINED['gbs']:.0f} GB/s, empty kernel node {empty_us:.2f} us")
    inp, head = run_workload(args.config, args.steps, args.warmup,
                             cpu_budget=0.0 if args.no_cpu else args.cpu_budget)
    bound_hbm = head["h_q"] * head["s_q"] <= 64
    traffic = measured_traffic(head["workload"])
    rf = head["roofline"]
    if bound_hbm:
        achieved = rf["main_kernel"]["gbs"]
        roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s", frac=achieved / HBM_PEAK_GBS,
                    traffic=traffic)
        value, unit = rf["step"]["gbs"], "GB/s"
    else:
        achieved = rf["main_kernel"]["tflops"]
        roof = dict(bound="mfma", achieved=achieved, peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=achieved / MFMA_PEAK_TFLOPS, traffic=traffic)
        value, unit = rf["step"]["tflops"], "TFLOP/s"
    roof["kernel"] = head["kernel"]
    roof["algorithmic_per_launch"] = head["bytes"] if bound_hbm else head["flops"]
    roof["kernel_ms"] = head["main_kernel_ms"]
    roof["step"] = dict(achieved=value, frac=value / (HBM_PEAK_GBS if bound_hbm else MFMA_PEAK_TFLOPS))
    roof["frac_attainable_main"] = rf["main_kernel"]["frac_attainable"]
    roof["frac_read_ceiling_same_bytes_main"] = rf["main_kernel"]["frac_read_ceiling_same_bytes"]
    cpu = head.pop("cpu_baseline", None)
    del inp

    extra = {}
    if not args.no_extra:
        eb = 0.0 if args.no_cpu else args.extra_cpu_budget
        for idx, causal in ((3, False), (4, False), (4, True), (5, False)):
            if idx == args.config and not causal:
                continue
            _, r = run_workload(idx, args.steps, args.warmup, causal=causal, cpu_budget=eb)
            extra[f"config{idx}" + ("_causal" if causal else "")] = _extra_entry(r)
        if args.config != 1:
            _, r = run_workload(1, args.steps, args.warmup, cpu_budget=eb)
            extra["config1"] = _extra_entry(r)
        _, r = run_workload(2, args.steps, args.warmup, fp8=True, cpu_budget=eb)
        extra["config2_fp8"] = _extra_entry(r)
        for fp8 in (False, True):
            # (the oracle of the FP8 sparse line would need the whole 0.9 GB pool
            # dequantized to float64 on the host: its CPU baseline is skipped)
            _, r = run_sparse_workload(args.steps, args.warmup, fp8=fp8, cpu_budget=0.0 if fp8 else eb)
            extra["sparse_fp8" if fp8 else "sparse"] = _extra_entry(r)

    line = dict(
        metric=METRIC, value=value, unit=unit, n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=head["ms_per_step"], higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16", data="synthetic",
        config=dict(workload=head["workload"], batch=head["batch"], s_q=head["s_q"], h_q=head["h_q"],
                    d_qk=576, d_v=512, page=64, sum_seqlen=head["sum_seqlen"], parts=head["parts"],
                    total_splits=head["total_splits"], rotating_kv_copies=head["rotating_copies"]),
        roofline=roof, cpu_baseline=cpu,
        detail=dict(timing="graph replay of exactly `steps` steps (GPU events), spread over further replays",
                    **{k: v for k, v in head.items() if k not in ("workload",)},
                    sustained_read_ceiling=SUSTAINED, empty_kernel_node_us=empty_us,
                    kernel_sha256_16=kernel_hash()),
        extra=extra,
    )
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
