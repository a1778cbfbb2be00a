"""Benchmark of the Engram layer forward hot path on one MI355X.

One step = one engram_forward (row gather -> wkv projection -> gate/residual)
over the prefill workload: T = 8192 tokens, dim 4096, hc 4, 16 hash columns of
head_dim 128 (K = 2048, N = 20480), bf16 tables (33.6 M rows, 8.6 GB,
HBM-resident) and bf16 wkv, Zipf(1.1) ids, no mask. Inputs are seeded and
synthetic and already resident in HBM when the timed region starts.

Prints one JSON line. ``value`` is prefill tokens/s; ``decode_t16`` carries
the decode workload (T = 16, MXFP8 wkv) measured cold: 16 copies of the
weight are rotated so no step finds it in the 256 MB Infinity Cache.
``roofline`` is the dominant kernel (the wkv GEMM with the gate epilogue that
the default forward launches, MFMA-bound) with its duration taken from HIP
events on the launch stream, around calls of engram_wkv_gate_partials in the
same launch configuration, made just before the timed steps.
``cpu_baseline`` is the CPU oracle on a bounded sample of the same workload.
``measured_peaks`` are ceilings measured on the same GPU with the library's
probes (register-only MFMA loops, a streaming read and copy of 4 GiB); each
fraction of a datasheet peak has a ``frac_of_measured`` beside it.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Engram forward tokens/s at dim 4096 (T=8192 prefill; T=16 decode) + % roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _source_sha(rel: str) -> str:
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(kernel: str, src: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != _source_sha(src):
        return None
    return rec.get("hbm_bytes_per_launch")


def _events_time(fn, iters, stream):
    """Average duration (ms) of fn() over iters launches, from HIP events on
    the stream the work is enqueued on."""
    import torch

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    for i in range(iters):
        starts[i].record(stream)
        fn(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in zip(starts, ends)]


def _pct(v, q):
    """q-th percentile (0..100) of a list, nearest rank."""
    v = sorted(v)
    return v[min(len(v) - 1, max(0, int(round(q / 100.0 * (len(v) - 1)))))]


def bench_prefill(steps, warmup):
    import torch

    from gram_memory_layer_engram_amd import engram as E
    from gram_memory_layer_engram_amd import workloads as W

    wl = W.WORKLOADS["prefill"]
    inp = W.make_inputs(wl, "cuda")
    stream = torch.cuda.current_stream()
    out = torch.empty_like(inp["hidden"])
    args = E.forward_args(inp["table"], inp["ids"], inp["w"], None, inp["hidden"], inp["q"],
                          inp["k"], None, wl.eps, wl.clamp, out)
    ws = torch.empty(E.forward_workspace_size(args), dtype=torch.uint8, device="cuda")

    def fwd(_=0, store_kv=False):
        E.forward(inp["table"], inp["ids"], inp["w"], None, inp["hidden"], inp["q"], inp["k"],
                  None, wl.eps, wl.clamp, out=out, workspace=ws, store_kv=store_kv)

    for _ in range(warmup):
        fwd()

    # Per-kernel durations, before the timed steps so that those start from
    # the clocks and caches of a running loop: the default forward (the
    # GEMM's gate epilogue, keys never stored) and the store-kv forward
    # (kv stored, plain gate), alternated call by call so both see the same
    # clocks; then the steps of each route called one by one through
    # pre-marshalled C calls. All event-timed on the launch stream.
    t_both = _events_time(lambda i: fwd(i, i % 2 == 1), 2 * steps, stream)
    t_fwd, t_fwd_kv = t_both[0::2], t_both[1::2]
    rows = torch.empty((wl.T, wl.C, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((wl.T, wl.N), dtype=torch.bfloat16, device="cuda")
    x = rows.view(wl.T, wl.K)
    L = E.load_library()
    sp = stream.cuda_stream
    ids = inp["ids"]
    look = (inp["table"].data_ptr(), inp["table"].shape[0], wl.head_dim, ids.data_ptr(), ids.stride(0),
            ids.stride(1), wl.T, wl.C, rows.data_ptr(), None, sp)
    t_lookup = _events_time(lambda i: L.engram_lookup(*look), steps, stream)
    value = torch.empty((wl.T, wl.dim), dtype=torch.bfloat16, device="cuda")
    parts = torch.empty((wl.hc, wl.T, wl.dim // 256, 2), dtype=torch.float32, device="cuda")
    fused = (x.data_ptr(), wl.T, wl.K, inp["w"].data_ptr(), None, E.W_BF16, wl.hc, wl.dim,
             inp["hidden"].data_ptr(), inp["q"].data_ptr(), inp["k"].data_ptr(), value.data_ptr(),
             parts.data_ptr(), None, 0, sp)
    if L.engram_wkv_gate_partials(*fused) != 0:
        raise RuntimeError("engram_wkv_gate_partials refused the prefill shapes")
    t_fused = _events_time(lambda i: L.engram_wkv_gate_partials(*fused), steps, stream)
    t_wkv = _events_time(lambda i: E.wkv(x, inp["w"], kv=kv), steps, stream)
    t_gate = _events_time(lambda i: E.gate(inp["hidden"], kv, inp["q"], inp["k"], None, wl.eps,
                                           wl.clamp, out=out), steps, stream)

    # the timed region: K forward steps between two synchronizations
    fwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps

    # the same gather from the table stored as fp8 (e4m3 + ue8m0 per 32), dequantized on lookup
    del inp["table"]
    torch.cuda.empty_cache()
    codes, scales = W.make_table_fp8(wl, "cuda")
    look8 = (codes.data_ptr(), scales.data_ptr(), codes.shape[0], wl.head_dim, ids.data_ptr(), ids.stride(0),
             ids.stride(1), wl.T, wl.C, rows.data_ptr(), None, sp)
    for _ in range(warmup):
        L.engram_lookup_fp8(*look8)
    t_lookup8 = _events_time(lambda i: L.engram_lookup_fp8(*look8), steps, stream)
    return wl, dt, {"lookup": t_lookup, "wkv_gate_partials": t_fused, "wkv": t_wkv, "gate": t_gate,
                    "lookup_fp8": t_lookup8, "forward": t_fwd, "forward_store_kv": t_fwd_kv}


def bench_decode(steps, warmup, copies=16):
    import torch

    from gram_memory_layer_engram_amd import engram as E
    from gram_memory_layer_engram_amd import workloads as W

    wl = W.WORKLOADS["decode_t16"]
    base = W.make_inputs(wl, "cuda")
    # cold cache: distinct weight copies (16 x 40 MiB) and per-copy activations
    sets = []
    for v in range(copies):
        sets.append({
            "w": base["w"].clone(), "w_scales": base["w_scales"].clone(),
            "ids": torch.from_numpy(W.make_ids(wl, variant=v)).cuda(),
            "hidden": W.make_hidden(wl, device="cuda", variant=v),
            "mask": torch.from_numpy(W.make_mask(wl, variant=v)).cuda(),
        })
    out = torch.empty_like(base["hidden"])
    stream = torch.cuda.current_stream()
    # one prepared forward per rotated set: a step is a single C call
    plans = [E.ForwardPlan(base["table"], s["ids"], s["w"], s["w_scales"], s["hidden"], base["q"],
                           base["k"], s["mask"], wl.eps, wl.clamp, out=out) for s in sets]

    def fwd(i):
        plans[i % copies].run()

    for i in range(warmup):
        fwd(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fwd(i)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps

    # the GEMV alone (quantize included: that is engram_wkv), cold
    x = torch.empty((wl.T, wl.K), dtype=torch.bfloat16, device="cuda")
    E.lookup(base["table"], base["ids"], rows_out=x.view(wl.T, wl.C, wl.head_dim))
    kv = torch.empty((wl.T, wl.N), dtype=torch.bfloat16, device="cuda")
    wws = torch.empty(max(1, E.load_library().engram_wkv_workspace_size(wl.T, wl.K, wl.N, E.W_MXFP8)),
                      dtype=torch.uint8, device="cuda")
    # engram_wkv through a pre-marshalled C call (the Python wrapper's own
    # checks would otherwise leave the GPU idle between launches)
    L = E.load_library()
    sptr = stream.cuda_stream
    wkv_args = [(x.data_ptr(), wl.T, wl.K, st["w"].data_ptr(), st["w_scales"].data_ptr(), E.W_MXFP8, wl.N,
                 kv.data_ptr(), wws.data_ptr(), wws.numel(), sptr) for st in sets]
    t_wkv = _events_time(lambda i: L.engram_wkv(*wkv_args[i % copies]), steps, stream)
    # the measured ceiling for that weight stream: one streaming-read launch
    # over the same rotated copies
    probe = E.probe_out()
    read_args = [(st["w"].data_ptr(), st["w"].numel(), probe.data_ptr(), sptr) for st in sets]
    t_read = _events_time(lambda i: L.engram_probe_read(*read_args[i % copies]), steps, stream)
    t_fwd = _events_time(fwd, steps, stream)
    # the single-launch variant of the same forward, same rotation
    plans_1 = [E.ForwardPlan(base["table"], s["ids"], s["w"], s["w_scales"], s["hidden"], base["q"],
                             base["k"], s["mask"], wl.eps, wl.clamp, out=out, single_launch=True) for s in sets]
    for i in range(warmup):
        plans_1[i % copies].run()
    t_one = _events_time(lambda i: plans_1[i % copies].run(), steps, stream)
    return wl, dt, {"wkv": t_wkv, "forward": t_fwd, "single_launch": t_one, "read_w": t_read}


def bench_long(steps=5, warmup=2):
    """The long-prefill workload (T 32768, dim 7168, K 3072, MXFP8 wkv, Zipf
    ids, 10% masked): event-timed forward and projection (quantize + GEMM),
    reported beside the headline."""
    import torch

    from gram_memory_layer_engram_amd import engram as E
    from gram_memory_layer_engram_amd import workloads as W

    wl = W.WORKLOADS["long"]
    inp = W.make_inputs(wl, "cuda")
    stream = torch.cuda.current_stream()
    out = torch.empty_like(inp["hidden"])
    plan = E.ForwardPlan(inp["table"], inp["ids"], inp["w"], inp["w_scales"], inp["hidden"], inp["q"],
                         inp["k"], inp["mask"], wl.eps, wl.clamp, out=out)
    for _ in range(warmup):
        plan.run()
    t_fwd = _events_time(lambda i: plan.run(), steps, stream)
    x = torch.empty((wl.T, wl.K), dtype=torch.bfloat16, device="cuda")
    E.lookup(inp["table"], inp["ids"], rows_out=x.view(wl.T, wl.C, wl.head_dim))
    kv = torch.empty((wl.T, wl.N), dtype=torch.bfloat16, device="cuda")
    for _ in range(warmup):
        E.wkv(x, inp["w"], inp["w_scales"], kv=kv)
    t_wkv = _events_time(lambda i: E.wkv(x, inp["w"], inp["w_scales"], kv=kv), steps, stream)
    # the MXFP8 activation quantize alone (engram_mx_quantize) on the same rows
    xq = torch.empty((wl.T, wl.K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((wl.T, wl.K // 32), dtype=torch.uint8, device="cuda")
    L = E.load_library()
    qargs = (x.data_ptr(), wl.T, wl.K, xq.data_ptr(), xs.data_ptr(), stream.cuda_stream)
    if L.engram_mx_quantize(*qargs) != 0:
        raise RuntimeError("engram_mx_quantize refused the long-prefill rows")
    t_q = _events_time(lambda i: L.engram_mx_quantize(*qargs), max(steps, 20), stream)
    return wl, {"forward": t_fwd, "wkv": t_wkv, "mx_quantize": t_q}


def measured_peaks(reps=5):
    """Ceilings measured on this GPU with the library's probes (HIP events,
    mean over reps launches after one warm-up): the register-only MFMA loop
    in bf16 and MXFP8, a streaming read of 4 GiB (16 times the 256 MB
    Infinity Cache, so HBM serves it), and 1:1 and 2:1 read/write streams
    over the same 4 GiB."""
    import torch

    from gram_memory_layer_engram_amd import engram as E

    L = E.load_library()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    out = E.probe_out()
    res = {}
    for name, fmt, iters in (("mfma_bf16_TFLOPs", E.W_BF16, 20000), ("mfma_mxfp8_TFLOPs", E.W_MXFP8, 10000)):
        flops = E.probe_mfma(fmt, iters, out)
        t = _events_time(lambda i: E.probe_mfma(fmt, iters, out), reps, stream)
        res[name] = round(flops / (statistics.fmean(t) * 1e-3) / 1e12, 1)
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    L.engram_probe_read(buf.data_ptr(), nbytes, out.data_ptr(), sp)
    t = _events_time(lambda i: L.engram_probe_read(buf.data_ptr(), nbytes, out.data_ptr(), sp), reps, stream)
    res["hbm_read_GBs"] = round(nbytes / (statistics.fmean(t) * 1e-3) / 1e9, 1)
    # R:1 read/write streams: a copy, and 2 reads per write (the plain gate
    # reads hidden and kv and writes out: 2.25 to 1)
    for name, ratio in (("hbm_copy_GBs", 1), ("hbm_stream_2to1_GBs", 2)):
        wb = nbytes // (ratio + 1) // 16 * 16
        src, dst = buf[:ratio * wb], buf[ratio * wb:(ratio + 1) * wb]
        args = (src.data_ptr(), dst.data_ptr(), wb, ratio, sp)
        L.engram_probe_stream(*args)
        t = _events_time(lambda i: L.engram_probe_stream(*args), reps, stream)
        res[name] = round((ratio + 1) * wb / (statistics.fmean(t) * 1e-3) / 1e9, 1)
    del buf, src, dst
    torch.cuda.empty_cache()
    return res


def cpu_baseline(budget_s=12.0):
    """The oracle as it stands, on the prefill workload in 512-token blocks,
    passing over the 8192 tokens again until about budget_s seconds of work."""
    import numpy as np
    import torch

    from gram_memory_layer_engram_amd import workloads as W
    from oracle import engram_oracle as o

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = None
    wl = W.WORKLOADS["prefill"]
    ids = W.make_ids(wl)
    uniq, inv = np.unique(ids, return_inverse=True)
    inv = inv.reshape(ids.shape)
    table = W.make_table(wl, "cuda")
    sub = table[torch.from_numpy(uniq).cuda().long()].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    del table
    torch.cuda.empty_cache()
    w, _ = W.make_weight(wl, "cpu")
    wb = w.view(torch.int16).numpy().view(np.uint16)
    hidden = W.make_hidden(wl).view(torch.int16).numpy().view(np.uint16)
    q, k = W.make_qk(wl)
    qb = q.view(torch.int16).numpy().view(np.uint16)
    kb = k.view(torch.int16).numpy().view(np.uint16)
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and done < 4 * wl.T:
        start = done % wl.T
        blk = slice(start, start + 512)
        o.forward(sub, inv[blk], wb, None, hidden[blk], qb, kb, None, wl.eps, wl.clamp)
        done += 512
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": threads or len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"prefill workload (T=8192, dim 4096, bf16 wkv [20480, 2048]), {done} tokens "
                      f"in 512-token blocks, NumPy fp64 oracle, {el:.1f} s; host cpus "
                      f"{len(os.sched_getaffinity(0))}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 512 MiB device copy (reference for the HBM byte counters)")
    a = ap.parse_args()
    if a.gpus != 1:
        print("bench.py measures one GPU: the Engram hot path here has no multi-GPU mode "
              "(every token is independent, so it would shard by tokens with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if a.calib_copy:
        n = 512 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n, "launches": 5}))
        return

    from gram_memory_layer_engram_amd import engram as E

    E.load_library()

    wl, dt, kt = bench_prefill(a.steps, a.warmup)
    med = {k: statistics.median(v) for k, v in kt.items()}
    avg = {k: statistics.fmean(v) for k, v in kt.items()}
    flops = 2.0 * wl.T * wl.K * wl.N
    fused_s = avg["wkv_gate_partials"] * 1e-3
    achieved = flops / fused_s / 1e12
    roofline = {
        "kernel": "gemm_bf16_kernel with the gate epilogue (engram_wkv_gate_partials, the default "
                  "forward's projection: 8192 x 20480 x 2048)",
        "bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
        "traffic": _traffic("gemm_bf16_kernel_gate_epilogue", "gram_memory_layer_engram_amd/csrc/gemm.hip"),
        "traffic_unit": "bytes per launch past L2 (rocprofv3 FETCH_SIZE + WRITE_SIZE, each copy-calibrated)",
    }
    # the HBM-bound kernels of the same step, against 8 TB/s
    lookup_bytes = wl.T * wl.C * (4 + 2 * 2 * wl.head_dim)
    lookup8_bytes = wl.T * wl.C * (4 + wl.head_dim + wl.head_dim // 32 + 2 * wl.head_dim)
    gate_bytes = wl.T * (2 * wl.hc * wl.dim + (wl.hc + 1) * wl.dim) * 2
    kernels = {
        "lookup_us": round(avg["lookup"] * 1e3, 2),
        "lookup_GBs": round(lookup_bytes / (avg["lookup"] * 1e-3) / 1e9, 1),
        "lookup_fp8_table_us": round(avg["lookup_fp8"] * 1e3, 2),
        "lookup_fp8_table_GBs": round(lookup8_bytes / (avg["lookup_fp8"] * 1e-3) / 1e9, 1),
        "wkv_gate_partials_us": round(avg["wkv_gate_partials"] * 1e3, 2),
        "wkv_gate_partials_us_p10_p90": [round(_pct(kt["wkv_gate_partials"], 10) * 1e3, 2),
                                         round(_pct(kt["wkv_gate_partials"], 90) * 1e3, 2)],
        "wkv_us": round(avg["wkv"] * 1e3, 2), "wkv_us_median": round(med["wkv"] * 1e3, 2),
        "wkv_us_p10_p90": [round(_pct(kt["wkv"], 10) * 1e3, 2), round(_pct(kt["wkv"], 90) * 1e3, 2)],
        "wkv_mfma_frac": round(flops / (avg["wkv"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "gate_us": round(avg["gate"] * 1e3, 2),
        "gate_us_p10_p90": [round(_pct(kt["gate"], 10) * 1e3, 2), round(_pct(kt["gate"], 90) * 1e3, 2)],
        "gate_GBs": round(gate_bytes / (avg["gate"] * 1e-3) / 1e9, 1),
        "forward_us_events": round(avg["forward"] * 1e3, 2),
        "forward_store_kv_us_events": round(avg["forward_store_kv"] * 1e3, 2),
    }

    dwl, ddt, dkt = bench_decode(max(a.steps, 100), a.warmup)
    d_wkv = statistics.fmean(dkt["wkv"]) * 1e-3
    d_fwd = statistics.fmean(dkt["forward"]) * 1e-3
    w_bytes = dwl.N * dwl.K + dwl.N * dwl.K // 1024
    d_alg = w_bytes + dwl.T * dwl.C * (4 + 2 * 2 * dwl.head_dim) + dwl.T * 2 * dwl.hc * dwl.dim * 2 \
        + 2 * dwl.hc * dwl.dim * 2 + dwl.T
    decode = {
        "workload": "decode T=16, dim 4096, MXFP8 wkv [20480, 2048] (40 MiB), 16 weight copies rotated",
        "value": round(dwl.T / ddt, 1), "unit": "tokens/s", "ms_per_step": round(ddt * 1e3, 4),
        "forward_us_events": round(d_fwd * 1e6, 2),
        "forward_us_median_p10_p90": [round(statistics.median(dkt["forward"]) * 1e3, 2),
                                      round(_pct(dkt["forward"], 10) * 1e3, 2),
                                      round(_pct(dkt["forward"], 90) * 1e3, 2)],
        "forward_hbm_frac": round(d_alg / d_fwd / 1e9 / HBM_PEAK_GBS, 4),
        "single_launch_us_events": round(statistics.fmean(dkt["single_launch"]) * 1e3, 2),
        "wkv_us": round(d_wkv * 1e6, 2),
        "wkv_GBs": round((w_bytes + dwl.T * dwl.N * 2) / d_wkv / 1e9, 1),
        "wkv_hbm_frac": round((w_bytes + dwl.T * dwl.N * 2) / d_wkv / 1e9 / HBM_PEAK_GBS, 4),
    }

    lwl, lkt = bench_long()
    peaks = measured_peaks()
    roofline["measured_peak"] = peaks["mfma_bf16_TFLOPs"]
    roofline["frac_of_measured"] = round(achieved / peaks["mfma_bf16_TFLOPs"], 4)
    roofline["measured_peak_source"] = "register-only bf16 MFMA loop on this GPU (engram_probe_mfma)"
    kernels["gate_frac_of_measured_2to1"] = round(kernels["gate_GBs"] / peaks["hbm_stream_2to1_GBs"], 4)
    d_read = statistics.fmean(dkt["read_w"]) * 1e-3
    decode["forward_frac_of_measured_read"] = round(d_alg / d_fwd / 1e9 / peaks["hbm_read_GBs"], 4)
    decode["read_40MiB_cold_us"] = round(d_read * 1e6, 2)
    decode["read_40MiB_cold_GBs"] = round(dwl.N * dwl.K / d_read / 1e9, 1)
    decode["wkv_us_vs_read_40MiB_cold"] = round(d_wkv / d_read, 3)
    l_fwd = statistics.fmean(lkt["forward"]) * 1e-3
    l_wkv = statistics.fmean(lkt["wkv"]) * 1e-3
    l_q = statistics.fmean(lkt["mx_quantize"]) * 1e-3
    long = {
        "workload": "long prefill T=32768, dim 7168, hc 4, K 3072, MXFP8 wkv [35840, 3072], Zipf ids, "
                    "10% masked",
        "forward_us_events": round(l_fwd * 1e6, 1),
        "tokens_per_s": round(lwl.T / l_fwd, 1),
        "wkv_us": round(l_wkv * 1e6, 1),
        "wkv_mfma_frac": round(2.0 * lwl.T * lwl.K * lwl.N / l_wkv / 1e12 / FP8_PEAK_TFLOPS, 4),
        "wkv_frac_of_measured_mfma": round(2.0 * lwl.T * lwl.K * lwl.N / l_wkv / 1e12 / peaks["mfma_mxfp8_TFLOPs"], 4),
        # activation quantize: per token 2K bytes read, K + K/32 written
        "mx_quantize_us": round(l_q * 1e6, 2),
        "mx_quantize_GBs": round(lwl.T * (3 * lwl.K + lwl.K // 32) / l_q / 1e9, 1),
        "mx_quantize_frac_of_measured_2to1": round(lwl.T * (3 * lwl.K + lwl.K // 32) / l_q / 1e9
                                                   / peaks["hbm_stream_2to1_GBs"], 4),
    }

    cpu = None if a.no_cpu_baseline else cpu_baseline()
    line = {
        "metric": METRIC, "value": round(wl.T / dt, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(dt * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill: T=8192, dim=4096, hc=4, n_hash_cols=16, head_dim=128, "
                               "bf16 tables 33556876 rows (HBM), bf16 wkv [20480, 2048], Zipf(1.1) ids, no mask",
                   "global_batch": wl.T, "parallelism": "none (1 GPU)"},
        "roofline": roofline, "kernels": kernels, "decode_t16": decode, "long_prefill": long,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
