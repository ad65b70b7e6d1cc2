#!/usr/bin/env python3
"""Benchmark of dense MLA decode on one MI355X; prints one JSON line.

A step is one dense MLA decode call (split-KV kernel + combine kernel) over
one batch of the synthetic workload, inputs resident in HBM.  Steps are
replayed from a HIP graph, as serving engines run decode (the
attention-kernel page's CUDA-graph section); the plain eager rate is
reported beside it.  The tile plan is made once per decode step and reused
by every call of that step (as the pages prescribe for all layers of a
decode step); its host time is measured and reported separately as
``plan_us``.  Several copies of q and the KV pool are rotated between steps
so that the 256 MB memory-side cache cannot serve one step's pages to the
next.

Headline workload: TP-sharded memory-bound decode (batch 16, h_q 16,
L ~ U[1024, 4096]) -> effective HBM GB/s.  The h_q = 128 workloads
(compute-bound, ragged MTP, long context) are reported under ``extra`` in
TFLOP/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

METRIC = "MLA decode TFLOPs (h_q=128) and effective HBM GB/s (h_q=16), 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRCS = [os.path.join(ROOT, "decode_attention_mla_amd", "csrc", f) for f in ("mla_decode.hip", "mla_internal.h")]


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


def main_kernel_name(rows: int) -> str:
    """The split-KV kernel the library launches for h_q * s_q = rows."""
    if rows <= 16:
        return "mla_splitkv_small_kernel<false, false>"
    if rows >= 128:
        return ("mla_splitkv_wide_kernel<true, false, false>" if rows <= 128
                else "mla_splitkv_wide_kernel<false, false, false>")
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


def time_steps(step, rot: int, steps: int, warmup: int):
    """Times decode calls ``step(i)`` (i picks the rotating input copy):

    * graph: ``rot`` steps captured once in a HIP graph and replayed -- how
      serving engines run a decode step; the whole-job rate reported;
    * kernels: eager calls enqueued behind a GPU sleep so the host runs
      ahead, with the library's per-kernel HIP events (recorded by the
      dispatch itself) -> the average main / combine kernel durations;
    * eager: plain back-to-back calls from Python, wall clock (reference).
    Returns (ms_per_step, graph_steps, main_ms, combine_ms, eager_ms)."""
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
            for i in range(rot):
                step(i)
    torch.cuda.synchronize()
    replays = max(1, steps // rot)
    for _ in range(max(1, warmup // rot)):
        graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(replays):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    graph_wall_ms = (time.perf_counter() - t0) * 1e3
    graph_steps = replays * rot
    ms_per_step = max(graph_wall_ms, ev0.elapsed_time(ev1)) / graph_steps
    del graph
    torch.cuda._sleep(int(2.0e9 * 0.002 * steps))   # ~2 ms of GPU time per 100 calls at 2 GHz
    mla.profile_start(steps)
    for i in range(steps):
        step(i)
    main_ms, comb_ms, calls = mla.profile_stop()
    torch.cuda.synchronize()
    assert calls == steps, (calls, steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps
    return ms_per_step, graph_steps, main_ms / calls, comb_ms / calls, eager_ms


def run_workload(idx: int, steps: int, warmup: int, min_rot_bytes: float = 640e6, causal: bool = False,
                 fp8: bool = False):
    """Times one dense workload (see time_steps), one step per rotating copy
    of q and the KV pool so that no step finds its pages in cache."""
    import torch
    import decode_attention_mla_amd as mla
    from decode_attention_mla_amd import workloads as W

    t = time.perf_counter()
    inp = W.config_inputs(idx)
    log(f"[bench] config {idx} {inp.name}: inputs drawn in {time.perf_counter() - t:.1f}s")
    flops, nbytes = W.algorithmic_work(inp.cache_seqlens, inp.s_q, inp.h_q, causal=causal,
                                       kv_row_bytes=W.FP8_RECORD if fp8 else 2 * W.D_QK)
    dev = torch.device("cuda", 0)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    kv0 = torch.from_numpy(W.to_fp8_records(inp.kv_cache)).to(dev) if fp8 else bf16(inp.kv_cache)
    q0 = bf16(inp.q)
    kv_bytes = kv0.numel() * kv0.element_size()
    rot = int(min(8, max(1, np.ceil(min_rot_bytes / kv_bytes))))
    kvs = [kv0] + [kv0.clone() for _ in range(rot - 1)]
    qs = [q0] + [q0.clone() for _ in range(rot - 1)]
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl = torch.from_numpy(inp.cache_seqlens).to(dev)

    # Plan once per decode step (host), timed separately.
    reps = 50
    t = time.perf_counter()
    for _ in range(reps):
        sched_np, ns_np, total = mla.get_mla_metadata_host(inp.cache_seqlens, inp.h_q, inp.s_q, fp8=fp8)
    plan_us = (time.perf_counter() - t) / reps * 1e6
    sched = torch.from_numpy(sched_np).to(dev)
    ns = torch.from_numpy(ns_np).to(dev)
    # The same plan on the GPU (device lengths; capturable with the decode),
    # timed as graph replays of 20 planner launches (no host launch cost).
    mla.get_mla_metadata_device(sl, inp.h_q, inp.s_q, fp8=fp8)
    torch.cuda.synchronize()
    plan_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(plan_graph):
        for _ in range(20):
            mla.get_mla_metadata_device(sl, inp.h_q, inp.s_q, fp8=fp8)
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

    ms_per_step, graph_steps, main_avg, comb_avg, eager_ms = time_steps(step, rot, steps, warmup)

    res = dict(
        workload=inp.name + ("_causal" if causal else "") + ("_fp8" if fp8 else ""), batch=b, s_q=inp.s_q, h_q=inp.h_q,
        sum_seqlen=int(inp.cache_seqlens.sum()),
        parts=int(sched.shape[0]), total_splits=int(total), rotating_copies=rot, graph_steps=graph_steps,
        flops=flops, bytes=nbytes, ms_per_step=ms_per_step, eager_ms_per_step=eager_ms,
        main_kernel_ms=main_avg, combine_kernel_ms=comb_avg, plan_us=plan_us, plan_device_us=plan_device_us,
        tflops=flops / (ms_per_step * 1e-3) / 1e12, gbs=nbytes / (ms_per_step * 1e-3) / 1e9,
        main_kernel_tflops=flops / (main_avg * 1e-3) / 1e12, main_kernel_gbs=nbytes / (main_avg * 1e-3) / 1e9,
    )
    log(f"[bench] config {idx}{' causal' if causal else ''}{' fp8' if fp8 else ''}: "
        f"{json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in res.items()})}")
    del kvs, qs
    torch.cuda.empty_cache()
    return inp, res


def run_sparse_workload(steps: int, warmup: int, min_rot_bytes: float = 640e6, fp8: bool = False):
    """Times the sparse workload (batch 128, s_q 2, h_q 128, topk 2048; each
    query token's 2048 keys drawn from its request's 4096..8192-token
    context) the same way as the dense ones."""
    import torch
    import decode_attention_mla_amd as mla
    from decode_attention_mla_amd import workloads as W

    t = time.perf_counter()
    inp = W.sparse_config_inputs()
    log(f"[bench] sparse {inp.name}: inputs drawn in {time.perf_counter() - t:.1f}s")
    flops, nbytes = W.sparse_algorithmic_work(inp.indices, inp.h_q, inp.topk_length,
                                              kv_row_bytes=W.FP8_RECORD if fp8 else 2 * W.D_QK)
    dev = torch.device("cuda", 0)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    kv0 = torch.from_numpy(W.to_fp8_records(inp.kv_cache)).to(dev) if fp8 else bf16(inp.kv_cache)
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

    ms_per_step, graph_steps, main_avg, comb_avg, eager_ms = time_steps(step, rot, steps, warmup)
    res = dict(
        workload=inp.name + ("_fp8" if fp8 else ""), batch=inp.batch, s_q=inp.s_q, h_q=inp.h_q, topk=inp.topk,
        parts=int(sched.shape[0]),
        total_splits=int(ns[-1].item()), rotating_copies=rot, graph_steps=graph_steps, flops=flops, bytes=nbytes,
        ms_per_step=ms_per_step, eager_ms_per_step=eager_ms, main_kernel_ms=main_avg, combine_kernel_ms=comb_avg,
        tflops=flops / (ms_per_step * 1e-3) / 1e12, gbs=nbytes / (ms_per_step * 1e-3) / 1e9,
        main_kernel_tflops=flops / (main_avg * 1e-3) / 1e12, main_kernel_gbs=nbytes / (main_avg * 1e-3) / 1e9,
    )
    log(f"[bench] sparse{' fp8' if fp8 else ''}: {json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in res.items()})}")
    del kvs, qs
    torch.cuda.empty_cache()
    return inp, res


def cpu_baseline(inp, work: float, scale: float, unit: str, budget_s: float = 10.0):
    """The oracle, as it stands, on this host: whole passes over the workload
    until ~budget_s of CPU work; returns work * passes / seconds / scale."""
    import oracle
    threads = 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()
                             if i.get("user_api") == "blas"])
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.mla_decode(inp.q, inp.kv_cache, inp.block_table, inp.cache_seqlens, inp.softmax_scale)
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return dict(value=work * passes / el / scale, unit=unit, cores=threads, kind="oracle",
                sample=f"{passes} full pass(es) of the workload in {el:.1f}s (numpy fp64, BLAS threads={threads})")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2,
                    help="headline workload (1..5); 6 times the sparse workload alone, 7 workload 2 on an FP8 "
                         "cache and 8 the sparse workload on an FP8 cache (for profiling)")
    ap.add_argument("--no-extra", action="store_true", help="skip the h_q=128 workloads")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
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
    if args.config in (6, 7, 8):   # profiling entry points: one workload, no headline line
        if args.config == 7:
            _, r = run_workload(2, args.steps, args.warmup, fp8=True)
            metric, value, unit = "decode GB/s, FP8 cache", r["gbs"], "GB/s"
        else:
            _, r = run_sparse_workload(args.steps, args.warmup, fp8=args.config == 8)
            metric, value, unit = "sparse decode TFLOP/s", r["tflops"], "TFLOP/s"
        print(json.dumps(dict(metric=metric, value=value, unit=unit, n_gpus=1, steps=args.steps, warmup=args.warmup,
                              ms_per_step=r["ms_per_step"], higher_is_better=True, dtype="bf16", data="synthetic",
                              detail=r)), flush=True)
        return

    inp, head = run_workload(args.config, args.steps, args.warmup)
    bound_hbm = head["h_q"] * head["s_q"] <= 64
    traffic = measured_traffic(head["workload"])
    if bound_hbm:
        achieved = head["bytes"] / (head["main_kernel_ms"] * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s", frac=achieved / HBM_PEAK_GBS,
                    traffic=traffic)
        value, unit = head["gbs"], "GB/s"
    else:
        achieved = head["flops"] / (head["main_kernel_ms"] * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=achieved, peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=achieved / MFMA_PEAK_TFLOPS, traffic=traffic)
        value, unit = head["tflops"], "TFLOP/s"
    roof["kernel"] = main_kernel_name(head["h_q"] * head["s_q"])
    cpu = None
    if not args.no_cpu:
        cpu = (cpu_baseline(inp, head["bytes"], 1e9, "GB/s") if bound_hbm
               else cpu_baseline(inp, head["flops"], 1e12, "TFLOP/s"))
    del inp

    extra = {}
    if not args.no_extra:
        for idx, causal in ((3, False), (4, False), (4, True), (5, False)):
            if idx == args.config and not causal:
                continue
            _, r = run_workload(idx, args.extra_steps, max(2, args.extra_steps // 5), causal=causal)
            extra[f"config{idx}" + ("_causal" if causal else "")] = dict(
                workload=r["workload"], tflops=r["tflops"], frac_mfma_peak=r["tflops"] / MFMA_PEAK_TFLOPS,
                gbs=r["gbs"], frac_hbm_peak=r["gbs"] / HBM_PEAK_GBS, ms_per_step=r["ms_per_step"],
                eager_ms_per_step=r["eager_ms_per_step"], main_kernel_tflops=r["main_kernel_tflops"],
                main_kernel_ms=r["main_kernel_ms"], combine_kernel_ms=r["combine_kernel_ms"],
                parts=r["parts"], total_splits=r["total_splits"], plan_us=r["plan_us"],
                plan_device_us=r["plan_device_us"])
        _, r = run_workload(2, args.extra_steps, max(2, args.extra_steps // 5), fp8=True)
        extra["config2_fp8"] = dict(
            workload=r["workload"], gbs=r["gbs"], frac_hbm_peak=r["gbs"] / HBM_PEAK_GBS, tflops=r["tflops"],
            ms_per_step=r["ms_per_step"], eager_ms_per_step=r["eager_ms_per_step"],
            main_kernel_gbs=r["main_kernel_gbs"], main_kernel_ms=r["main_kernel_ms"],
            combine_kernel_ms=r["combine_kernel_ms"], parts=r["parts"], total_splits=r["total_splits"])
        for fp8 in (False, True):
            _, r = run_sparse_workload(args.extra_steps, max(2, args.extra_steps // 5), fp8=fp8)
            extra["sparse_fp8" if fp8 else "sparse"] = dict(
                workload=r["workload"], tflops=r["tflops"], frac_mfma_peak=r["tflops"] / MFMA_PEAK_TFLOPS,
                gbs=r["gbs"], frac_hbm_peak=r["gbs"] / HBM_PEAK_GBS, ms_per_step=r["ms_per_step"],
                eager_ms_per_step=r["eager_ms_per_step"], main_kernel_tflops=r["main_kernel_tflops"],
                main_kernel_ms=r["main_kernel_ms"], combine_kernel_ms=r["combine_kernel_ms"],
                parts=r["parts"], total_splits=r["total_splits"])

    line = dict(
        metric=METRIC, value=value, unit=unit, n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=head["ms_per_step"], higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16", data="synthetic",
        config=dict(workload=head["workload"], batch=head["batch"], s_q=head["s_q"], h_q=head["h_q"],
                    d_qk=576, d_v=512, page=64, sum_seqlen=head["sum_seqlen"], parts=head["parts"],
                    total_splits=head["total_splits"], rotating_kv_copies=head["rotating_copies"]),
        roofline=roof, cpu_baseline=cpu,
        detail=dict(timing="graph replay", eager_ms_per_step=head["eager_ms_per_step"],
                    graph_steps=head["graph_steps"], main_kernel_ms=head["main_kernel_ms"],
                    combine_kernel_ms=head["combine_kernel_ms"], plan_us=head["plan_us"],
                    plan_device_us=head["plan_device_us"],
                    algorithmic_bytes=head["bytes"], algorithmic_flops=head["flops"],
                    kernel_sha256_16=kernel_hash()),
        extra=extra,
    )
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
