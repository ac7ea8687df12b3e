"""Benchmark of the attention forward pass on one MI355X.

One step = one fa_fwd call over the whole workload (the full hot path:
Q/K/V tiles -> scores -> online softmax -> P V -> O and lse), inputs already
resident in HBM.  Default workload: B4 H16 N4096 D128, bf16, non-causal.
Throughput counts 4*B*H*N^2*D FLOPs per step (half for causal).

The default run also times every other configuration of the five synthetic
workloads (tiny fp32; small bf16 both modes and fp32; the headline shape
causal; wide D = 64; long-context causal) with the same step and warm-up
counts and reports them in the JSON line's "workloads" object, and the next
rows of the path on their own workloads (the backward pass, the key split,
packed sequences and FP8 inputs, both modes, a fifth of the steps) in its
"next_rows" object.  Warm-up runs at least --warmup steps and at least
--warm-seconds of GPU work, so that the clocks have settled before the timed
steps.

Prints ONE JSON line on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s + % of bf16 MFMA peak, B4 H16 N4096 D128"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3, "e4m3": 5000.0}  # MI355X dense MFMA, published
# the forward kernel's sources: the kernel file and the device headers it includes
KERNEL_SRCS = [os.path.join(ROOT, "attention_fa_fwd_02_amd", "csrc", f)
               for f in ("fa_fwd.hip", "fa_fwd_common.h", "fa_device.h")]
# the headline's rocprofv3 summary (kernel trace, SQ counters, HBM bytes)
COUNTERS = os.path.join(ROOT, "profiles", "fa_fwd_pp_kernel_bf16_d128_B4H16N4096.txt")

WORKLOADS = {
    # name: (B, H, N, D, dtype, causal, sigma)
    "headline": (4, 16, 4096, 128, "bf16", False, (1.0, 1.0, 1.0)),
    "headline_causal": (4, 16, 4096, 128, "bf16", True, (1.0, 1.0, 1.0)),
    "small": (2, 8, 1024, 64, "bf16", False, (1.0, 1.0, 1.0)),
    "small_causal": (2, 8, 1024, 64, "bf16", True, (1.0, 1.0, 1.0)),
    "small_f32": (2, 8, 1024, 64, "f32", False, (1.0, 1.0, 1.0)),
    "tiny_f32": (1, 1, 128, 64, "f32", False, (1.0, 1.0, 1.0)),
    "wide": (32, 32, 4096, 64, "bf16", False, (1.0, 1.0, 1.0)),
    "long_causal": (1, 8, 131072, 128, "bf16", True, (0.5, 0.5, 1.0)),
    "d256": (4, 8, 4096, 256, "bf16", False, (1.0, 1.0, 1.0)),
    "d256_causal": (4, 8, 4096, 256, "bf16", True, (1.0, 1.0, 1.0)),
    "d96": (4, 16, 4096, 96, "bf16", False, (1.0, 1.0, 1.0)),
    "d192": (4, 8, 4096, 192, "bf16", False, (1.0, 1.0, 1.0)),
    "d32": (4, 16, 4096, 32, "bf16", False, (1.0, 1.0, 1.0)),
    "d160": (4, 8, 4096, 160, "bf16", False, (1.0, 1.0, 1.0)),
    "d224": (4, 8, 4096, 224, "bf16", False, (1.0, 1.0, 1.0)),
    "few_heads": (1, 2, 8192, 128, "bf16", False, (1.0, 1.0, 1.0)),
    "few_heads_causal": (1, 2, 8192, 128, "bf16", True, (1.0, 1.0, 1.0)),
}
# the configurations of the five synthetic workloads, in order, with their labels
CONFIG_SET = [("tiny_f32", "C1 tiny fp32"), ("small", "C2 small bf16"), ("small_causal", "C2 small bf16 causal"),
              ("small_f32", "C2 small fp32"), ("headline", "C3 headline bf16"),
              ("headline_causal", "C3 headline bf16 causal"), ("wide", "C4 wide D64 bf16"),
              ("long_causal", "C5 long-context causal bf16")]
# the same workloads through fa_fwd_split (key splits + lse merge; split count
# from fa_fwd_split_choose for the device's compute units)
SPLIT_WORKLOADS = {"few_heads_split": "few_heads", "few_heads_causal_split": "few_heads_causal"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        h.update(open(path, "rb").read())
    return h.hexdigest()


def read_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (else None)."""
    if not os.path.exists(COUNTERS):
        return None
    vals = {}
    for line in open(COUNTERS):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_sha():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def device_inputs(B, H, N, D, dtype, sigma, seed=1004):
    import numpy as np
    import torch

    import fa_inputs as fi
    q, k, v = fi.make_qkv(B, H, N, D, dtype, seed, *sigma)

    def up(x):
        if dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
        return torch.from_numpy(x).to("cuda")
    return (q, k, v), tuple(up(x) for x in (q, k, v))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(host_qkv, dev_out, B, H, N, D, dtype, causal, budget_s=15.0):
    """The fp64 oracle, as it stands, on a bounded row sample of the same workload;
    also checks those rows of the GPU output.  Returns the JSON object."""
    import numpy as np

    import fa_inputs as fi
    import oracle
    q, k, v = host_qkv
    o_dev, lse_dev = dev_out
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    scale = oracle.gpu_scale(1.0 / math.sqrt(D))
    heads = [(b, h) for b in range(B) for h in range(H)]
    o_host = o_dev.view(-1).cpu()
    l_host = lse_dev.view(-1).cpu().numpy()
    import torch
    o_bits = o_host.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else o_host.numpy()
    o_np = o_bits.reshape(B, H, N, D)
    l_np = l_host.reshape(B, H, N)

    def run(rows_per_head, nheads):
        flops = 0.0
        worst_o = worst_l = 0.0
        t0 = time.perf_counter()
        for (b, h) in heads[:nheads]:
            rows = fi.sample_rows(N, rows_per_head, seed=77 + 100 * b + h)
            qw = oracle.widen(q[b, h][rows], dtype)
            kw = oracle.widen(k[b, h], dtype)
            vw = oracle.widen(v[b, h], dtype)
            o_ref, l_ref = oracle.attention_rows(qw, kw, vw, rows, scale, causal, n_threads=threads)
            nk = (rows + 1) if causal else np.full(rows.shape, N)
            flops += float(np.sum(4.0 * nk * D))
            worst_o = max(worst_o, float(np.abs(oracle.widen(o_np[b, h][rows], dtype) - o_ref).max()))
            worst_l = max(worst_l, float(np.abs(l_np[b, h][rows].astype(np.float64) - l_ref).max()))
        return time.perf_counter() - t0, flops, worst_o, worst_l

    # calibrate on a small sample that still gives every thread several rows,
    # then size the sample to about budget_s seconds
    t, f, _, _ = run(min(N, 8 * threads), min(4, len(heads)))
    rate = f / max(t, 1e-6)
    per_head = 4.0 * N * D * (N / 2 if causal else N)  # flops for all rows of one head
    total_rows = max(8, int(budget_s * rate / (per_head / N)))
    nheads = len(heads)
    rows_per_head = max(2, min(N, total_rows // nheads))
    t, f, eo, el = run(rows_per_head, nheads)
    log("cpu oracle: %d heads x %d rows, %.2f s, %.3f GFLOP/s, %d threads; sampled GPU rows max|dO|=%.3g max|dlse|=%.3g"
        % (nheads, rows_per_head, t, f / t / 1e9, threads, eo, el))
    # the oracle's work for every row of the workload (a causal row i has i + 1 keys)
    full_flops = 4.0 * B * H * D * (N * (N + 1) / 2.0 if causal else float(N) * N)
    return {"value": f / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cores_note": "oracle threads used (the job's CPU share is 16 cores per GPU)",
            "host_cores": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(),
            "extrapolated_full_workload_s": round(full_flops / (f / t), 1),
            "sample": "%d heads x %d seeded query rows (all %d keys%s), fp64 three-pass oracle, %.1f s"
                      % (nheads, rows_per_head, N, ", causal prefix" if causal else "", t),
            "check_max_abs_dO": eo, "check_max_abs_dlse": el}


def warm_up(step, warmup, warm_seconds):
    """At least `warmup` steps and at least `warm_seconds` of wall time, in
    synchronised chunks; returns the number of steps run."""
    import torch
    t0 = time.perf_counter()
    n = 0
    chunk = max(1, min(warmup, 50)) if warmup > 0 else 10
    while n < warmup or time.perf_counter() - t0 < warm_seconds:
        for _ in range(chunk):
            step()
        n += chunk
        torch.cuda.synchronize()
    return n


def bench_one(name, steps, warmup, copy_calibration=False, flush=False, warm_seconds=0.0):
    import torch

    import attention_fa_fwd_02_amd as fa
    import fa_inputs as fi
    split = name in SPLIT_WORKLOADS
    B, H, N, D, dtype, causal, sigma = WORKLOADS[SPLIT_WORKLOADS.get(name, name)]
    host, (q, k, v) = device_inputs(B, H, N, D, dtype, sigma)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    code = {"f32": fa.FA_DTYPE_F32, "bf16": fa.FA_DTYPE_BF16, "f16": fa.FA_DTYPE_F16}[dtype]
    scale = 1.0 / math.sqrt(D)

    def step():
        st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, H, N, D, scale, int(causal), code, stream.cuda_stream)
        if st != fa.FA_OK:
            raise fa.FaError(st)

    n_splits = 1
    if split:
        n_cus = torch.cuda.get_device_properties(0).multi_processor_count
        n_splits = fa.fa_fwd_split_choose(B, H, N, D, int(causal), n_cus)
        ws_bytes = fa.fa_fwd_split_workspace_bytes(B, H, N, D, n_splits)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

        def step():  # noqa: F811 -- the split path replaces the single launch
            st = fa.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 B, H, N, D, scale, int(causal), code, n_splits, ws.data_ptr(), ws_bytes,
                                 stream.cuda_stream)
            if st != fa.FA_OK:
                raise fa.FaError(st, "fa_fwd_split")

    if copy_calibration:
        # a plain device copy of known size, for scaling HBM byte counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    n_warm = warm_up(step, warmup, warm_seconds)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    # the timed steps: exactly `steps` calls back to back between two events
    # (the throughput; per-call events would add host work between the calls)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for _ in range(steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_begin.elapsed_time(t_end)
    # the same number of calls again, each between its own pair of events on the
    # launch stream (kernel time per call: average, median, minimum).  Cold-cache
    # variant: a 1 GiB fill between calls evicts the inputs from L2 and the 256 MB
    # Infinity Cache; only these per-call events count then.
    junk = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if flush else None
    for i in range(steps):
        if flush:
            junk.fill_(i & 255)
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    del junk
    torch.cuda.synchronize()
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    kern_ms = sum(per) / len(per)
    flops = fi.workload_flops(B, H, N, D, causal)
    ms_per_step = total_ms / steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]
    if flush:
        log("%s, cold caches: B%d H%d N%d D%d %s causal=%d  kernel avg %.4f ms (min %.4f, median %.4f)  %.1f TFLOP/s  %.1f%% of %s peak"
            % (name, B, H, N, D, dtype, causal, kern_ms, per[0], per[len(per) // 2], achieved, 100 * achieved / peak, dtype))
    else:
        log("%s: B%d H%d N%d D%d %s causal=%d%s  step %.4f ms (kernel avg %.4f, min %.4f, median %.4f)  %.1f TFLOP/s  %.1f%% of %s peak"
            % (name, B, H, N, D, dtype, causal, " splits=%d" % n_splits if split else "", ms_per_step, kern_ms, per[0], per[len(per) // 2], value,
               100 * achieved / peak, dtype))
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    kernel = fa.fa_fwd_kernel_name(B, H, N, D, int(causal), code, n_cus)
    if split:
        # the key split's instance (mode 1, one key group): the ping-pong kernel at
        # D <= 128, the one-barrier kernel above, the fp32 kernel for fp32
        cs = "true" if causal else "false"
        e = {"bf16": "Bf16", "f16": "F16"}.get(dtype)
        if dtype == "f32":
            kernel = "fa_fwd_f32_kernel<%d, %s, 1, 1>" % (D, cs)
        elif D <= 128:
            kernel = "fa_fwd_pp_kernel<%s, %d, %s, 1, 1>" % (e, D, cs)
        else:
            kernel = "fa_fwd_mfma_kernel<%s, %d, %s, 1>" % (e, D, cs)
        kernel = "%s (%d splits) + fa_merge_kernel" % (kernel, n_splits)
    res = dict(name=name, B=B, H=H, N=N, D=D, dtype=dtype, causal=causal, ms_per_step=ms_per_step,
               kernel_ms=kern_ms, kernel_min_ms=per[0], kernel_median_ms=per[len(per) // 2], value=value,
               achieved=achieved, peak=peak, flops=flops, kernel=kernel, warmup_steps_run=n_warm)
    # inputs and outputs stay alive for the CPU-oracle leg, which runs after all GPU timing
    return res, (host, (o, lse), B, H, N, D, dtype, causal)


def time_steps(step, steps, warmup, warm_seconds):
    """Warm up (at least `warmup` calls and `warm_seconds` of wall time), then
    time `steps` back-to-back calls between two events on the current stream;
    returns ms per call."""
    import torch
    stream = torch.cuda.current_stream()
    warm_up(step, warmup, warm_seconds)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def next_row(name, config, ms, flops, peak_dtype):
    tf = flops / (ms * 1e-3) / 1e12
    return {"name": name, "config": config, "ms_per_step": round(ms, 5), "tflops": round(tf, 3),
            "peak": PEAK_TFLOPS[peak_dtype], "peak_dtype": peak_dtype,
            "frac": round(tf / PEAK_TFLOPS[peak_dtype], 4)}


def bench_varlen(name, steps, warmup, warm_seconds=0.0):
    """The packed length-mix workload through fa_fwd_varlen; logs a stderr
    line and returns the result record."""
    import numpy as np
    import torch

    import attention_fa_fwd_02_amd as fa
    import fa_inputs as fi
    causal = name.endswith("causal")
    w = fi.VARLEN_WORKLOAD
    lens = fi.make_seqlens(w["n_seqs"], w["lo"], w["hi"], w["seed"])
    cu = fi.cu_seqlens(lens)
    H, D, dtype = w["H"], w["D"], w["dtype"]
    total = int(cu[-1])
    q, k, v = fi.make_packed(H, total, total, D, dtype, w["seed"], *w["sigma"])
    up = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
    dq, dk, dv = up(q), up(k), up(v)
    dcu = torch.from_numpy(cu).to("cuda")
    o = torch.empty_like(dq)
    lse = torch.empty((H, total), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    scale = 1.0 / math.sqrt(D)
    max_len = int(lens.max())

    def step():
        st = fa.fa_fwd_varlen(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              dcu.data_ptr(), dcu.data_ptr(), len(lens), H, total, total, max_len, D, scale,
                              int(causal), fa.FA_DTYPE_BF16, stream.cuda_stream)
        if st != fa.FA_OK:
            raise fa.FaError(st, "fa_fwd_varlen")

    ms = time_steps(step, steps, warmup, warm_seconds)
    flops = fi.varlen_flops(lens, lens, H, D, causal)
    log("%s: %d packed sequences (%d..%d rows, %d total) H%d D%d bf16 causal=%d  step %.4f ms  %.1f TFLOP/s  %.1f%% of bf16 peak"
        % (name, len(lens), int(lens.min()), max_len, total, H, D, causal, ms, flops / (ms * 1e-3) / 1e12,
           100 * flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"]))
    return next_row(name, "fa_fwd_varlen: %d packed sequences of %d..%d rows (%d total), H%d D%d bf16 %s"
                    % (len(lens), int(lens.min()), max_len, total, H, D, "causal" if causal else "non-causal"),
                    ms, flops, "bf16")


def bench_bwd(name, steps, warmup, warm_seconds=0.0):
    """fa_bwd on the headline shape, at D = 32 / 96 for "bwd_d32*" / "bwd_d96*",
    B4 H8 N4096 at D = 160 / 192 / 224 / 256 for "bwd_d160*" / "bwd_d192*" /
    "bwd_d224*" / "bwd_d256*", or the headline shape in fp32
    for "bwd_f32*" (stderr line only).  FLOPs: the five contractions of the
    backward pass, 10*B*H*N^2*D (2.5x the forward's count, halved for causal);
    the kernels recompute S and dP once more (seven; eight at D = 256).
    Returns the result record."""
    import torch

    import attention_fa_fwd_02_amd as fa
    import fa_inputs as fi
    causal = name.endswith("causal")
    D = int(name[5:].split("_")[0]) if name.startswith("bwd_d") else 128
    B, H, N, dtype = 4, (8 if D > 128 else 16), 4096, ("f32" if name.startswith("bwd_f32") else "bf16")
    host, (q, k, v) = device_inputs(B, H, N, D, dtype, (1.0, 1.0, 1.0))
    _, (do, _, _) = device_inputs(B, H, N, D, dtype, (1.0, 1.0, 1.0), seed=1004 + 7919)
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsb = fa.fa_bwd_workspace_bytes(B, H, N, D)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    code = fa.FA_DTYPE_F32 if dtype == "f32" else fa.FA_DTYPE_BF16

    def step():
        st = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, D, scale, int(causal),
                       code, ws.data_ptr(), wsb, stream.cuda_stream)
        if st != fa.FA_OK:
            raise fa.FaError(st, "fa_bwd")

    ms = time_steps(step, steps, warmup, warm_seconds)
    flops = 2.5 * fi.workload_flops(B, H, N, D, causal)
    tf = flops / (ms * 1e-3) / 1e12
    log("%s: B%d H%d N%d D%d %s causal=%d  step %.4f ms  %.1f TFLOP/s  %.1f%% of %s peak"
        % (name, B, H, N, D, dtype, causal, ms, tf, 100 * tf / PEAK_TFLOPS[dtype], dtype))
    return next_row(name, "fa_bwd: B%d H%d N%d D%d %s %s (10 B H N^2 D flops, halved for causal)"
                    % (B, H, N, D, dtype, "causal" if causal else "non-causal"), ms, flops, dtype)


def bench_fp8(name, steps, warmup, warm_seconds=0.0):
    """fa_fwd_fp8 on the headline shape (B4 H16 N4096 D128, E4M3 inputs, bf16 O),
    or B4 H8 N4096 at another head dim (stderr line only).  FLOPs as for
    the 16-bit path; peak: dense FP8 MFMA."""
    import numpy as np
    import torch

    import attention_fa_fwd_02_amd as fa
    import fa_inputs as fi
    causal = name.endswith("causal")
    # fp8 / fp8_causal: the headline shape; fp8_d<D>[_causal]: B4 H8 N4096 at head dim D
    D = int(name.split("_d")[1].split("_")[0]) if "_d" in name else 128
    B, H, N = (4, 16, 4096) if D == 128 else (4, 8, 4096)
    q, k, v = fi.make_qkv(B, H, N, D, "e4m3", 1004)
    dq, dk, dv = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in (q, k, v))
    o = torch.empty((B, H, N, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    wsb = fa.fa_fwd_fp8_workspace_bytes(B, H, N, D)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    scale = 1.0 / math.sqrt(D)

    def step():
        st = fa.fa_fwd_fp8(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, D,
                           scale, 1.0, 1.0, 1.0, int(causal), ws.data_ptr(), wsb, stream.cuda_stream)
        if st != fa.FA_OK:
            raise fa.FaError(st, "fa_fwd_fp8")

    ms = time_steps(step, steps, warmup, warm_seconds)
    flops = fi.workload_flops(B, H, N, D, causal)
    tf = flops / (ms * 1e-3) / 1e12
    log("%s: B%d H%d N%d D%d e4m3 causal=%d  step %.4f ms (V transpose included)  %.1f TFLOP/s  %.1f%% of fp8 peak"
        % (name, B, H, N, D, causal, ms, tf, 100 * tf / PEAK_TFLOPS["e4m3"]))
    return next_row(name, "fa_fwd_fp8: B%d H%d N%d D%d e4m3 %s (V transpose included)"
                    % (B, H, N, D, "causal" if causal else "non-causal"), ms, flops, "e4m3")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="headline", choices=sorted(WORKLOADS) + sorted(SPLIT_WORKLOADS))
    ap.add_argument("--warm-seconds", type=float, default=1.0,
                    help="minimum warm-up wall time before the timed steps (on top of --warmup steps)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="time only --workload (no per-configuration object; for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 256 MiB device copy first (for scaling HBM byte counters)")
    ap.add_argument("--all", action="store_true", help="also time every other workload (stderr)")
    ap.add_argument("--flush", action="store_true",
                    help="also time the headline, both modes, with caches flushed before every call (stderr)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(each (batch, head) slice is independent, so the work would shard by slice, "
              "or by key range with the lse merge)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    main_res, main_ctx = bench_one(args.workload, args.steps, args.warmup, args.copy_calibration,
                                   warm_seconds=args.warm_seconds)
    workloads = None
    if not args.no_workloads:
        # every configuration of the five workloads, same step and warm-up counts
        workloads = {}
        for name, label in CONFIG_SET:
            if name == args.workload:
                r = main_res
            else:
                r, _ = bench_one(name, args.steps, args.warmup, warm_seconds=min(args.warm_seconds, 0.5))
            workloads[name] = {
                "label": label,
                "config": "B%d H%d N%d D%d %s %s" % (r["B"], r["H"], r["N"], r["D"], r["dtype"],
                                                   "causal" if r["causal"] else "non-causal"),
                "tflops": round(r["value"], 3), "ms_per_step": round(r["ms_per_step"], 5),
                "achieved": round(r["achieved"], 3), "peak": r["peak"], "peak_dtype": r["dtype"],
                "frac": round(r["achieved"] / r["peak"], 4), "kernel": r["kernel"],
                "kernel_avg_ms": round(r["kernel_ms"], 5), "kernel_median_ms": round(r["kernel_median_ms"], 5),
                "kernel_min_ms": round(r["kernel_min_ms"], 5)}
    next_rows = None
    if not args.no_workloads:
        # the next rows of the path on their own workloads (backward, key split,
        # packed sequences, FP8), both modes, fewer steps
        ns, nw = max(10, args.steps // 5), max(10, args.warmup // 5)
        next_rows = {}
        for name in ("bwd", "bwd_causal"):
            next_rows[name] = bench_bwd(name, ns, nw, warm_seconds=0.3)
        for name in SPLIT_WORKLOADS:
            r, _ = bench_one(name, ns, nw, warm_seconds=0.3)
            next_rows[name] = next_row(name, "fa_fwd_split: B%d H%d N%d D%d %s %s, %s" % (
                r["B"], r["H"], r["N"], r["D"], r["dtype"], "causal" if r["causal"] else "non-causal", r["kernel"]),
                r["ms_per_step"], r["flops"], r["dtype"])
        for name in ("varlen", "varlen_causal"):
            next_rows[name] = bench_varlen(name, ns, nw, warm_seconds=0.3)
        for name in ("fp8", "fp8_causal"):
            next_rows[name] = bench_fp8(name, ns, nw, warm_seconds=0.3)
    if args.all:
        # every GPU timing comes before the CPU-oracle leg, whose minutes of host
        # work would otherwise leave the GPU idle (and down-clocked) right before
        if next_rows is None:  # --no-workloads: the next rows on stderr only
            ns, nw = max(10, args.steps // 5), max(10, args.warmup // 5)
            for name in ("bwd", "bwd_causal"):
                bench_bwd(name, ns, nw)
            for name in SPLIT_WORKLOADS:
                bench_one(name, ns, nw, warm_seconds=min(args.warm_seconds, 0.5))
            for name in ("varlen", "varlen_causal"):
                bench_varlen(name, ns, nw)
            for name in ("fp8", "fp8_causal"):
                bench_fp8(name, ns, nw)
        for name in WORKLOADS:
            if name != args.workload:
                bench_one(name, max(10, args.steps // 5), max(10, args.warmup // 5),
                          warm_seconds=min(args.warm_seconds, 0.5))
        for name in ("bwd_d32", "bwd_d96", "bwd_d96_causal", "bwd_d160", "bwd_d192", "bwd_d224", "bwd_d256",
                     "bwd_d256_causal", "bwd_f32", "bwd_f32_causal"):
            bench_bwd(name, max(10, args.steps // 5), max(10, args.warmup // 5))
        for name in ("fp8_d32", "fp8_d96", "fp8_d160", "fp8_d192", "fp8_d224", "fp8_d256", "fp8_d256_causal"):
            bench_fp8(name, max(10, args.steps // 5), max(10, args.warmup // 5))
    if args.flush:
        for name in ("headline", "headline_causal"):
            bench_one(name, max(10, args.steps // 5), max(10, args.warmup // 5), flush=True)
    r = main_res
    if not args.no_cpu_baseline:
        r["cpu_baseline"] = cpu_baseline(*main_ctx)
    traffic = read_traffic() if r["name"] == "headline" else None
    out = {
        "metric": METRIC,
        "value": round(r["value"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["dtype"],
        "data": "synthetic",
        "config": {"workload": "B%d H%d N%d D%d %s %s" % (r["B"], r["H"], r["N"], r["D"], r["dtype"],
                                                          "causal" if r["causal"] else "non-causal"),
                   "B": r["B"], "H": r["H"], "N": r["N"], "D": r["D"], "causal": r["causal"],
                   "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100.0 * r["achieved"] / r["peak"], 2),
        "roofline": {"bound": "mfma", "achieved": round(r["achieved"], 3), "peak": r["peak"],
                     "unit": "TFLOP/s", "frac": round(r["achieved"] / r["peak"], 4),
                     "traffic": traffic,
                     "kernel": r["kernel"],
                     "kernel_avg_ms": round(r["kernel_ms"], 5),
                     "kernel_median_ms": round(r["kernel_median_ms"], 5),
                     "kernel_min_ms": round(r["kernel_min_ms"], 5)},
        "cpu_baseline": r.get("cpu_baseline"),
    }
    if workloads is not None:
        out["workloads"] = workloads
    if next_rows is not None:
        out["next_rows"] = next_rows
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
