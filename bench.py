"""Benchmark of the Engram layer forward hot path on one MI355X.

One step = one engram_forward (row gather -> wkv projection -> gate/residual)
over the prefill workload: T = 8192 tokens, dim 4096, hc 4, 16 hash columns of
head_dim 128 (K = 2048, N = 20480), bf16 tables (33.6 M rows, 8.6 GB,
HBM-resident) and bf16 wkv, Zipf(1.1) ids, no mask. Inputs are seeded and
synthetic and already resident in HBM when the timed region starts.

The timed region comes right after the W warm-up steps, with nothing else
run in between: K forwards between two synchronizations. Everything else is
measured afterwards.

Prints one JSON line. ``value`` is prefill tokens/s. ``roofline`` is the
dominant kernel (the wkv GEMM with the gate epilogue that the default
forward launches, MFMA-bound), its duration taken from HIP events on the
launch stream around engram_wkv_gate_partials, called between the
forward's other two launches (engram_lookup before it, engram_gate_finish
after it: the forward's own kernels in its order, so the GEMM runs in the
cache and clock state the forward gives it). ``configs`` has one row per workload the layer is specified
on (tiny, mid, prefill, decode at T = 1, 4, 16, 64, long): forward time,
tokens/s, the bound and the fraction of that bound's peak. The decode rows
are measured cold: 16 copies of the 40 MiB weight are rotated so no step
finds its weight in the 256 MB Infinity Cache. ``kernels`` breaks the
prefill step down (gather, GEMM, gate), each with its fraction of peak.
``cpu_baseline`` is the CPU oracle on a bounded sample of the prefill
workload. ``measured_peaks`` are ceilings measured on the same GPU with the
library's probes; each fraction of a datasheet peak that has a measured
counterpart is also given against it.
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
DECODE_COPIES = 16


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
    """Per-call durations (ms) of fn(i), i < iters, from HIP events recorded
    on the stream the work is enqueued on."""
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


def _us(v):
    """median, p10, p90 of a list of ms, in us."""
    return [round(statistics.median(v) * 1e3, 2), round(_pct(v, 10) * 1e3, 2), round(_pct(v, 90) * 1e3, 2)]


def alg_bytes(wl) -> int:
    """Algorithmic HBM bytes of one forward: the weight (+ E8M0 scales), the
    ids, the gathered table rows, hidden in and out, q and k, the mask. kv
    and the staged rows are the implementation's own traffic, not counted."""
    w = wl.N * wl.K * (2 if wl.w_format == "bf16" else 1)
    if wl.w_format != "bf16":
        w += (wl.N // 32) * (wl.K // 32)
    rows = wl.T * wl.C * wl.head_dim * 2
    ids = wl.T * wl.C * 4
    hid = 2 * wl.T * wl.hc * wl.dim * 2
    qk = 2 * wl.hc * wl.dim * 2
    mask = wl.T if wl.mask_frac is not None else 0
    return w + rows + ids + hid + qk + mask


def _plan(E, inp, wl, out, **kw):
    return E.ForwardPlan(inp["table"], inp["ids"], inp["w"], inp["w_scales"], inp["hidden"], inp["q"],
                         inp["k"], inp["mask"], wl.eps, wl.clamp, out=out, **kw)


def bench_prefill(steps, warmup, offload=True):
    """The headline: W warm-up forwards, then K timed forwards; afterwards
    the per-kernel durations of the same step."""
    import torch

    from gram_memory_layer_engram_amd import engram as E
    from gram_memory_layer_engram_amd import workloads as W

    wl = W.WORKLOADS["prefill"]
    inp = W.make_inputs(wl, "cuda")
    stream = torch.cuda.current_stream()
    out = torch.empty_like(inp["hidden"])
    plan = _plan(E, inp, wl, out)
    for _ in range(warmup):
        plan.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        plan.run()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps

    # per-kernel durations of the same step, each event-timed on the launch
    # stream through pre-marshalled C calls
    n = max(steps, 20)
    t_fwd = _events_time(lambda i: plan.run(), n, stream)
    plan_kv = _plan(E, inp, wl, out, store_kv=True, workspace=plan.workspace)
    t_fwd_kv = _events_time(lambda i: plan_kv.run(), n, stream)
    rows = torch.empty((wl.T, wl.C, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((wl.T, wl.N), dtype=torch.bfloat16, device="cuda")
    x = rows.view(wl.T, wl.K)
    L = E.load_library()
    sp = stream.cuda_stream
    ids = inp["ids"]
    look = (inp["table"].data_ptr(), inp["table"].shape[0], wl.head_dim, ids.data_ptr(), ids.stride(0),
            ids.stride(1), wl.T, wl.C, rows.data_ptr(), None, sp)
    value = torch.empty((wl.T, wl.dim), dtype=torch.bfloat16, device="cuda")
    parts = torch.empty((wl.hc, wl.T, wl.dim // 256, 2), dtype=torch.float32, device="cuda")
    fused = (x.data_ptr(), wl.T, wl.K, inp["w"].data_ptr(), None, E.W_BF16, wl.hc, wl.dim,
             inp["hidden"].data_ptr(), inp["q"].data_ptr(), inp["k"].data_ptr(), value.data_ptr(),
             parts.data_ptr(), None, 0, sp)
    if L.engram_wkv_gate_partials(*fused) != 0:
        raise RuntimeError("engram_wkv_gate_partials refused the prefill shapes")
    finish = (inp["hidden"].data_ptr(), value.data_ptr(), parts.data_ptr(), None, wl.T, wl.hc, wl.dim, wl.eps,
              wl.clamp, out.data_ptr(), None, sp)
    # the default forward's three launches as separate C calls in the same
    # order (the same kernels, bit for bit the forward's output), an event
    # between each: every kernel is timed in the cache and clock state the
    # forward gives it (the projection GEMM runs ~5% slower there than
    # back to back, after the finish kernel's 580 MB of traffic)
    t_lookup, t_fused, t_finish = [], [], []
    for _ in range(n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(stream)
        L.engram_lookup(*look)
        ev[1].record(stream)
        L.engram_wkv_gate_partials(*fused)
        ev[2].record(stream)
        L.engram_gate_finish(*finish)
        ev[3].record(stream)
        torch.cuda.synchronize()
        t_lookup.append(ev[0].elapsed_time(ev[1]))
        t_fused.append(ev[1].elapsed_time(ev[2]))
        t_finish.append(ev[2].elapsed_time(ev[3]))
    # the same GEMM launched back to back (W and x stay in the caches)
    t_fused_alone = _events_time(lambda i: L.engram_wkv_gate_partials(*fused), n, stream)
    wkv = (x.data_ptr(), wl.T, wl.K, inp["w"].data_ptr(), None, E.W_BF16, wl.N, kv.data_ptr(), None, 0, sp)
    t_wkv = _events_time(lambda i: L.engram_wkv(*wkv), n, stream)
    gate = (inp["hidden"].data_ptr(), kv.data_ptr(), inp["q"].data_ptr(), inp["k"].data_ptr(), None, wl.T,
            wl.hc, wl.dim, wl.eps, wl.clamp, out.data_ptr(), None, sp)
    t_gate = _events_time(lambda i: L.engram_gate(*gate), n, stream)

    offload = bench_background_and_host_table(E, inp, wl) if offload else None

    # the same gather from the table stored as fp8 (e4m3 + ue8m0 per 32), dequantized on lookup
    del plan, plan_kv, inp["table"]
    torch.cuda.empty_cache()
    codes, scales = W.make_table_fp8(wl, "cuda")
    look8 = (codes.data_ptr(), scales.data_ptr(), codes.shape[0], wl.head_dim, ids.data_ptr(), ids.stride(0),
             ids.stride(1), wl.T, wl.C, rows.data_ptr(), None, sp)
    for _ in range(warmup):
        L.engram_lookup_fp8(*look8)
    t_lookup8 = _events_time(lambda i: L.engram_lookup_fp8(*look8), n, stream)
    del codes, scales, inp
    torch.cuda.empty_cache()
    return wl, dt, {"lookup": t_lookup, "wkv_gate_partials": t_fused, "wkv": t_wkv, "gate": t_gate,
                    "gate_finish": t_finish, "wkv_gate_partials_alone": t_fused_alone,
                    "lookup_fp8": t_lookup8, "forward": t_fwd, "forward_store_kv": t_fwd_kv}, offload


def chunked_prefill(L, calls, chunks, background, main, side):
    """One prefill forward as `chunks` token chunks in the kv-stored
    composition (lookup -> engram_wkv -> engram_gate), each call through
    pre-marshalled C arguments (`calls[c]` = the chunk's three argument
    tuples, the stream slot last and filled here). background: chunk c+1's
    lookup runs on `side` with engram_lookup_background while `main` runs
    chunk c's projection and gate (events order each projection after its
    gather, each gather after the projection that last read its row
    buffer); else every step runs on `main` in order."""
    import torch

    gathered = [torch.cuda.Event() for _ in range(chunks)]
    consumed = [torch.cuda.Event() for _ in range(chunks)]
    sm, ss = main.cuda_stream, side.cuda_stream

    def gather(c):
        if not background:
            L.engram_lookup(*calls[c][0], sm)
            return
        if c >= 2:
            side.wait_event(consumed[c - 2])
        L.engram_lookup_background(*calls[c][0], ss)
        gathered[c].record(side)

    if background:
        side.wait_stream(main)
        gather(0)
    for c in range(chunks):
        if background:
            if c + 1 < chunks:
                gather(c + 1)
            main.wait_event(gathered[c])
        else:
            gather(c)
        L.engram_wkv(*calls[c][1], sm)
        if background:
            consumed[c].record(main)
        L.engram_gate(*calls[c][2], sm)


def bench_background_and_host_table(E, inp, wl, reps=10, chunks=4):
    """The two ways the pages move the gather off the critical path:
    (a) the chunked prefill with background lookups on a side stream, against
    the same chunks run in order on one stream (wall time per forward);
    (b) the table in page-locked host memory, read over the host link by
    the same gather: the prefill lookup (Zipf ids) and a decode-size one
    (16 tokens of uniform ids), beside the same gathers from the device
    table."""
    import torch

    L = E.load_library()
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ct = wl.T // chunks
    bufs = [torch.empty((ct, wl.C, wl.head_dim), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    kv = torch.empty((ct, wl.N), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(inp["hidden"])
    tbl, ids, hid = inp["table"], inp["ids"], inp["hidden"]
    calls = []
    for c in range(chunks):
        t0 = c * ct
        rows = bufs[c % 2]
        calls.append((
            (tbl.data_ptr(), tbl.shape[0], wl.head_dim, ids[t0].data_ptr(), ids.stride(0), ids.stride(1), ct, wl.C,
             rows.data_ptr(), None),
            (rows.data_ptr(), ct, wl.K, inp["w"].data_ptr(), None, E.W_BF16, wl.N, kv.data_ptr(), None, 0),
            (hid[t0].data_ptr(), kv.data_ptr(), inp["q"].data_ptr(), inp["k"].data_ptr(), None, ct, wl.hc, wl.dim,
             wl.eps, wl.clamp, out[t0].data_ptr(), None)))
    res = {}
    for bg in (False, True):
        for _ in range(2):
            chunked_prefill(L, calls, chunks, bg, main, side)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            chunked_prefill(L, calls, chunks, bg, main, side)
        torch.cuda.synchronize()
        res["chunked_background_us" if bg else "chunked_serial_us"] = round((time.perf_counter() - t0) / reps * 1e6, 1)
    del bufs, kv, out
    ht = E.HostTable(inp["table"].shape[0], wl.head_dim).copy_from(inp["table"])
    try:
        rows = torch.empty((wl.T, wl.C, wl.head_dim), dtype=torch.bfloat16, device="cuda")
        E.lookup(ht, inp["ids"], rows_out=rows)
        t = _events_time(lambda i: E.lookup(ht, inp["ids"], rows_out=rows), reps, main)
        link = wl.T * wl.C * wl.head_dim * 2
        res["host_table_lookup_us"] = round(statistics.median(t) * 1e3, 1)
        res["host_table_rows_GBs"] = round(link / (statistics.median(t) * 1e-3) / 1e9, 2)
        # decode-size gathers with the decode workload's uniform ids, 16
        # id sets rotated so rows repeat rarely (the same table layout)
        from gram_memory_layer_engram_amd import workloads as W
        dwl = W.WORKLOADS["decode_t16"]
        ids16 = [torch.from_numpy(W.make_ids(dwl, variant=v)).cuda() for v in range(16)]
        r16 = torch.empty((16, wl.C, wl.head_dim), dtype=torch.bfloat16, device="cuda")
        t16 = _events_time(lambda i: E.lookup(ht, ids16[i % 16], rows_out=r16), 64, main)
        d16 = _events_time(lambda i: E.lookup(inp["table"], ids16[i % 16], rows_out=r16), 64, main)
        res["host_table_lookup_t16_us"] = round(statistics.median(t16) * 1e3, 2)
        res["device_table_lookup_t16_us"] = round(statistics.median(d16) * 1e3, 2)
        res["host_table_bytes"] = inp["table"].numel() * 2
    finally:
        ht.close()
    return res


def bench_small(name, iters=200, warmup=20):
    """tiny and mid: event-timed forwards (warm: these inputs fit the
    Infinity Cache, as they would in a running model), and for mid the
    default forward's projection GEMM on its own."""
    import torch

    from gram_memory_layer_engram_amd import engram as E
    from gram_memory_layer_engram_amd import workloads as W

    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, "cuda")
    stream = torch.cuda.current_stream()
    out = torch.empty_like(inp["hidden"])
    plan = _plan(E, inp, wl, out)
    for _ in range(warmup):
        plan.run()
    t_fwd = _events_time(lambda i: plan.run(), iters, stream)
    res = {"forward": t_fwd}
    if name == "mid":
        L = E.load_library()
        sp = stream.cuda_stream
        x = E.lookup(inp["table"], inp["ids"]).view(wl.T, wl.K)
        value = torch.empty((wl.T, wl.dim), dtype=torch.bfloat16, device="cuda")
        parts = torch.empty((wl.hc, wl.T, wl.dim // 256, 2), dtype=torch.float32, device="cuda")
        fused = (x.data_ptr(), wl.T, wl.K, inp["w"].data_ptr(), None, E.W_BF16, wl.hc, wl.dim,
                 inp["hidden"].data_ptr(), inp["q"].data_ptr(), inp["k"].data_ptr(), value.data_ptr(),
                 parts.data_ptr(), None, 0, sp)
        if L.engram_wkv_gate_partials(*fused) != 0:
            raise RuntimeError("engram_wkv_gate_partials refused the mid shapes")
        res["wkv_gate_partials"] = _events_time(lambda i: L.engram_wkv_gate_partials(*fused), iters, stream)
    del inp, plan
    torch.cuda.empty_cache()
    return wl, res


def bench_decode(steps, warmup, copies=DECODE_COPIES):
    """Decode at T = 1, 4, 16, 64 (MXFP8 wkv [20480, 2048]), cold: `copies`
    weight copies (40 MiB each, together well past the 256 MB Infinity
    Cache) and per-copy ids / hidden / mask rotated call by call."""
    import torch

    from gram_memory_layer_engram_amd import engram as E
    from gram_memory_layer_engram_amd import workloads as W

    base_wl = W.WORKLOADS["decode_t16"]
    table = W.make_table(base_wl, "cuda")
    w0, ws0 = W.make_weight(base_wl, "cuda")
    q, k = W.make_qk(base_wl, "cuda")
    weights = [(w0.clone(), ws0.clone()) for _ in range(copies)]
    del w0, ws0
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    L = E.load_library()
    probe = E.probe_out()
    res = {}
    for T in (1, 4, 16, 64):
        wl = W.WORKLOADS[f"decode_t{T}"]
        sets = []
        for v in range(copies):
            m = W.make_mask(wl, variant=v)
            sets.append({"ids": torch.from_numpy(W.make_ids(wl, variant=v)).cuda(),
                         "hidden": W.make_hidden(wl, device="cuda", variant=v),
                         "mask": torch.from_numpy(m).cuda()})
        out = torch.empty_like(sets[0]["hidden"])
        plans = [E.ForwardPlan(table, s["ids"], weights[i][0], weights[i][1], s["hidden"], q, k, s["mask"],
                               wl.eps, wl.clamp, out=out) for i, s in enumerate(sets)]
        for i in range(warmup):
            plans[i % copies].run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            plans[i % copies].run()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        t_fwd = _events_time(lambda i: plans[i % copies].run(), steps, stream)
        # the projection alone (engram_wkv: MX quantize + decode GEMV), same rotation
        x = E.lookup(table, sets[0]["ids"]).view(T, wl.K)
        kv = torch.empty((T, wl.N), dtype=torch.bfloat16, device="cuda")
        wws = torch.empty(max(1, L.engram_wkv_workspace_size(T, wl.K, wl.N, E.W_MXFP8)), dtype=torch.uint8,
                          device="cuda")
        wkv_args = [(x.data_ptr(), T, wl.K, wc.data_ptr(), wsc.data_ptr(), E.W_MXFP8, wl.N, kv.data_ptr(),
                     wws.data_ptr(), wws.numel(), sp) for wc, wsc in weights]
        t_wkv = _events_time(lambda i: L.engram_wkv(*wkv_args[i % copies]), steps, stream)
        r = {"forward": t_fwd, "wall_s": wall, "wkv": t_wkv}
        if T == 16:
            # the measured ceiling for the weight stream: one streaming-read
            # launch over the same rotated copies; and the single-launch forward
            read_args = [(wc.data_ptr(), wc.numel(), probe.data_ptr(), sp) for wc, _ in weights]
            r["read_w"] = _events_time(lambda i: L.engram_probe_read(*read_args[i % copies]), steps, stream)
            plans1 = [E.ForwardPlan(table, s["ids"], weights[i][0], weights[i][1], s["hidden"], q, k, s["mask"],
                                    wl.eps, wl.clamp, out=out, single_launch=True) for i, s in enumerate(sets)]
            for i in range(warmup):
                plans1[i % copies].run()
            r["single_launch"] = _events_time(lambda i: plans1[i % copies].run(), steps, stream)
        res[T] = (wl, r)
        del sets, plans, x, kv
    del table, weights
    torch.cuda.empty_cache()
    return res


def bench_long(steps=5, warmup=2):
    """The long-prefill workload (T 32768, dim 7168, K 3072, MXFP8 wkv, Zipf
    ids, 10% masked): event-timed forward and projection (quantize + GEMM),
    and the MXFP8 activation quantize on its own."""
    import torch

    from gram_memory_layer_engram_amd import engram as E
    from gram_memory_layer_engram_amd import workloads as W

    wl = W.WORKLOADS["long"]
    inp = W.make_inputs(wl, "cuda")
    stream = torch.cuda.current_stream()
    out = torch.empty_like(inp["hidden"])
    plan = _plan(E, inp, wl, out)
    for _ in range(warmup):
        plan.run()
    t_fwd = _events_time(lambda i: plan.run(), steps, stream)
    x = torch.empty((wl.T, wl.K), dtype=torch.bfloat16, device="cuda")
    E.lookup(inp["table"], inp["ids"], rows_out=x.view(wl.T, wl.C, wl.head_dim))
    kv = torch.empty((wl.T, wl.N), dtype=torch.bfloat16, device="cuda")
    for _ in range(warmup):
        E.wkv(x, inp["w"], inp["w_scales"], kv=kv)
    t_wkv = _events_time(lambda i: E.wkv(x, inp["w"], inp["w_scales"], kv=kv), steps, stream)
    xq = torch.empty((wl.T, wl.K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((wl.T, wl.K // 32), dtype=torch.uint8, device="cuda")
    L = E.load_library()
    qargs = (x.data_ptr(), wl.T, wl.K, xq.data_ptr(), xs.data_ptr(), stream.cuda_stream)
    if L.engram_mx_quantize(*qargs) != 0:
        raise RuntimeError("engram_mx_quantize refused the long-prefill rows")
    t_q = _events_time(lambda i: L.engram_mx_quantize(*qargs), max(steps, 20), stream)
    del inp, plan, x, kv, xq, xs
    torch.cuda.empty_cache()
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
    ap.add_argument("--headline-only", action="store_true",
                    help="only the prefill forward and its kernels (for profiler runs)")
    ap.add_argument("--overlap-demo", action="store_true",
                    help="only the chunked prefill with background lookups and the host-table gather")
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

    if a.overlap_demo:
        from gram_memory_layer_engram_amd import workloads as W
        wl = W.WORKLOADS["prefill"]
        inp = W.make_inputs(wl, "cuda")
        print(json.dumps(bench_background_and_host_table(E, inp, wl, reps=5)), flush=True)
        return

    wl, dt, kt, offload = bench_prefill(a.steps, a.warmup, offload=not a.headline_only)
    avg = {k: statistics.fmean(v) for k, v in kt.items()}
    flops = 2.0 * wl.T * wl.K * wl.N
    fused_s = avg["wkv_gate_partials"] * 1e-3
    achieved = flops / fused_s / 1e12
    roofline = {
        "kernel": "gemm_bf16_kernel with the gate epilogue (the default forward's projection, 8192 x 20480 x "
                  "2048), timed between the forward's lookup and finish launches",
        "bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
        "traffic": _traffic("gemm_bf16_kernel_gate_epilogue", "gram_memory_layer_engram_amd/csrc/gemm.hip"),
        "traffic_unit": "bytes per launch past L2 (rocprofv3 FETCH_SIZE + WRITE_SIZE, each copy-calibrated)",
    }
    # the HBM-bound kernels of the same step, against 8 TB/s
    lookup_bytes = wl.T * wl.C * (4 + 2 * 2 * wl.head_dim)
    lookup8_bytes = wl.T * wl.C * (4 + wl.head_dim + wl.head_dim // 32 + 2 * wl.head_dim)
    gate_bytes = wl.T * (2 * wl.hc * wl.dim + (wl.hc + 1) * wl.dim) * 2
    gbs = lambda b, key: b / (avg[key] * 1e-3) / 1e9  # noqa: E731
    kernels = {
        "lookup_us": round(avg["lookup"] * 1e3, 2),
        "lookup_GBs": round(gbs(lookup_bytes, "lookup"), 1),
        "lookup_hbm_frac": round(gbs(lookup_bytes, "lookup") / HBM_PEAK_GBS, 4),
        "lookup_fp8_table_us": round(avg["lookup_fp8"] * 1e3, 2),
        "lookup_fp8_table_GBs": round(gbs(lookup8_bytes, "lookup_fp8"), 1),
        "lookup_fp8_table_hbm_frac": round(gbs(lookup8_bytes, "lookup_fp8") / HBM_PEAK_GBS, 4),
        "wkv_gate_partials_us": round(avg["wkv_gate_partials"] * 1e3, 2),
        "wkv_gate_partials_us_med_p10_p90": _us(kt["wkv_gate_partials"]),
        "wkv_gate_partials_mfma_frac": roofline["frac"],
        "wkv_gate_partials_back_to_back_us": round(avg["wkv_gate_partials_alone"] * 1e3, 2),
        "wkv_gate_partials_back_to_back_mfma_frac": round(flops / (avg["wkv_gate_partials_alone"] * 1e-3) / 1e12
                                                          / BF16_PEAK_TFLOPS, 4),
        "gate_finish_us": round(avg["gate_finish"] * 1e3, 2),
        "gate_finish_hbm_frac": round(wl.T * (2 * wl.hc * wl.dim * 2 + wl.dim * 2 + wl.hc * (wl.dim // 256) * 8)
                                      / (avg["gate_finish"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "wkv_us": round(avg["wkv"] * 1e3, 2),
        "wkv_us_med_p10_p90": _us(kt["wkv"]),
        "wkv_mfma_frac": round(flops / (avg["wkv"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "gate_us": round(avg["gate"] * 1e3, 2),
        "gate_us_med_p10_p90": _us(kt["gate"]),
        "gate_GBs": round(gbs(gate_bytes, "gate"), 1),
        "gate_hbm_frac": round(gbs(gate_bytes, "gate") / HBM_PEAK_GBS, 4),
        "forward_us_events": round(avg["forward"] * 1e3, 2),
        "forward_us_med_p10_p90": _us(kt["forward"]),
        "forward_store_kv_us_events": round(avg["forward_store_kv"] * 1e3, 2),
    }
    if a.headline_only:
        print(json.dumps({"metric": METRIC, "value": round(wl.T / dt, 1), "ms_per_step": round(dt * 1e3, 4),
                          "roofline": roofline, "kernels": kernels}), flush=True)
        return

    configs = {}
    pf_alg = alg_bytes(wl)
    configs["prefill"] = {
        "T": wl.T, "forward_us": round(dt * 1e6, 2), "tokens_per_s": round(wl.T / dt, 1),
        "bound": "mfma", "frac": roofline["frac"],
        "frac_kernel": "projection GEMM with the gate epilogue, of 2.5 PFLOP/s bf16",
        "alg_bytes": pf_alg, "alg_GBs": round(pf_alg / dt / 1e9, 1),
    }
    for name in ("tiny", "mid"):
        swl, sr = bench_small(name)
        f = statistics.median(sr["forward"]) * 1e-3
        ab = alg_bytes(swl)
        row = {"T": swl.T, "forward_us": round(f * 1e6, 2), "forward_us_med_p10_p90": _us(sr["forward"]),
               "tokens_per_s": round(swl.T / f, 1), "alg_bytes": ab, "alg_GBs": round(ab / f / 1e9, 1)}
        if name == "tiny":
            # 0.56 MB and 25 MFLOP: three launches' fixed cost, not bandwidth or MFMA, bound it
            row.update({"bound": "launch", "hbm_frac": round(ab / f / 1e9 / HBM_PEAK_GBS, 5)})
        else:
            g = statistics.median(sr["wkv_gate_partials"]) * 1e-3
            gfl = 2.0 * swl.T * swl.K * swl.N
            row.update({"bound": "mfma", "wkv_gate_partials_us": round(g * 1e6, 2),
                        "frac": round(gfl / g / 1e12 / BF16_PEAK_TFLOPS, 4),
                        "frac_kernel": "projection GEMM with the gate epilogue, of 2.5 PFLOP/s bf16"})
        configs[name] = row

    dec = bench_decode(max(a.steps, 100), a.warmup)
    for T, (dwl, r) in dec.items():
        f = statistics.median(r["forward"]) * 1e-3
        wk = statistics.median(r["wkv"]) * 1e-3
        ab = alg_bytes(dwl)
        w_bytes = dwl.N * dwl.K + (dwl.N // 32) * (dwl.K // 32)
        row = {"T": T, "forward_us": round(f * 1e6, 2), "forward_us_med_p10_p90": _us(r["forward"]),
               "forward_us_wall": round(r["wall_s"] * 1e6, 2),
               "tokens_per_s": round(T / f, 1), "bound": "hbm", "alg_bytes": ab,
               "frac": round(ab / f / 1e9 / HBM_PEAK_GBS, 4),
               "frac_kernel": "whole forward, algorithmic bytes of 8 TB/s (cold weights)",
               "wkv_us": round(wk * 1e6, 2),
               "wkv_hbm_frac": round((w_bytes + T * (dwl.K + dwl.K // 32) + T * dwl.N * 2) / wk / 1e9
                                     / HBM_PEAK_GBS, 4)}
        if "read_w" in r:
            rd = statistics.median(r["read_w"]) * 1e-3
            row["read_40MiB_cold_us"] = round(rd * 1e6, 2)
            row["wkv_us_vs_read_40MiB_cold"] = round(wk / rd, 3)
            row["single_launch_us"] = round(statistics.median(r["single_launch"]) * 1e6 * 1e-3, 2)
        configs[f"decode_t{T}"] = row

    lwl, lkt = bench_long()
    l_fwd = statistics.median(lkt["forward"]) * 1e-3
    l_wkv = statistics.median(lkt["wkv"]) * 1e-3
    l_q = statistics.median(lkt["mx_quantize"]) * 1e-3
    lflops = 2.0 * lwl.T * lwl.K * lwl.N
    configs["long"] = {
        "T": lwl.T, "forward_us": round(l_fwd * 1e6, 1), "tokens_per_s": round(lwl.T / l_fwd, 1),
        "bound": "mfma", "frac": round(lflops / l_wkv / 1e12 / FP8_PEAK_TFLOPS, 4),
        "frac_kernel": "MXFP8 projection (quantize + scaled GEMM), of 5.0 PFLOP/s",
        "wkv_us": round(l_wkv * 1e6, 1),
        "mx_quantize_us": round(l_q * 1e6, 2),
        "mx_quantize_hbm_frac": round(lwl.T * (3 * lwl.K + lwl.K // 32) / l_q / 1e9 / HBM_PEAK_GBS, 4),
    }

    peaks = measured_peaks()
    roofline["measured_peak"] = peaks["mfma_bf16_TFLOPs"]
    roofline["frac_of_measured"] = round(achieved / peaks["mfma_bf16_TFLOPs"], 4)
    roofline["measured_peak_source"] = "register-only bf16 MFMA loop on this GPU (engram_probe_mfma)"
    kernels["gate_frac_of_measured_2to1"] = round(kernels["gate_GBs"] / peaks["hbm_stream_2to1_GBs"], 4)
    configs["long"]["frac_of_measured"] = round(lflops / l_wkv / 1e12 / peaks["mfma_mxfp8_TFLOPs"], 4)
    for T in (1, 4, 16, 64):
        row = configs[f"decode_t{T}"]
        row["frac_of_measured_read"] = round(row["frac"] * HBM_PEAK_GBS / peaks["hbm_read_GBs"], 4)

    cpu = None if a.no_cpu_baseline else cpu_baseline()
    line = {
        "metric": METRIC, "value": round(wl.T / dt, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(dt * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill: T=8192, dim=4096, hc=4, n_hash_cols=16, head_dim=128, "
                               "bf16 tables 33556876 rows (HBM), bf16 wkv [20480, 2048], Zipf(1.1) ids, no mask",
                   "global_batch": wl.T, "parallelism": "none (1 GPU)"},
        "roofline": roofline, "kernels": kernels, "configs": configs, "gather_offload": offload,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
