#!/usr/bin/env python3
"""Absorbed-latent MLA decode benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload v3_decode] [--cache-dtype bf16]

(--workload v2lite_prefill / v3_prefill times the prefill attention instead:
one mla_prefill_attn call over a 4,096-position prompt per step, in TFLOP/s.)

One step = one pass of the whole decode hot path over one batch, all inputs
already resident in HBM: append the batch's new tokens (quantising if the cache
is quantised), absorb W_UK into the queries, split-KV attention over the paged
latent cache, log-sum-exp combine, W_UV expansion.  Inputs are seeded synthetic
data with the workload's shapes (no checkpoint or dataset is read).

Prints ONE JSON line.  `value` is the latent-cache bytes the step attends over
divided by the step time (GB/s).  `roofline` is for the dominant kernel,
mla_decode_attn, timed alone with HIP events on the stream it runs on;
`cpu_baseline` times the CPU oracle's float32 form on a bounded sample (median
of three runs).  Before --warmup, untimed steps run until the card's clock has
settled under the load (at least --settle-s seconds; recorded in the line).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_PEAK_TFLOPS_16 = 2500.0   # MI355X dense fp16/bf16 matrix peak, vendor figure

WORKLOADS = {
    # name: (generator, description)
    "v3_decode": ("v3_decode", "DeepSeek-V3-shaped absorbed decode: H=128, B=64, 8192 tokens/seq, paged bf16 "
                               "cache, 64-token pages, shuffled block table"),
    "v2lite_decode": ("v2lite_decode", "V2-Lite-shaped decode attention: H=16, B=32, 4096 tokens/seq, contiguous"),
    "v3_ragged": ("v3_ragged", "V3-shaped ragged decode: H=128, B=128, log-uniform lengths in [128, 65536]"),
    "v2lite_quant": ("v2lite_quant", "quantised latent cache, V2-Lite shapes: H=16, B=64, 16384 tokens/seq"),
}
PREFILL_WORKLOADS = {
    "v2lite_prefill": ("v2lite_prefill", "V2-Lite-shaped prompt chunk: H=16, 4096 positions, no cached prefix, "
                                         "causal unabsorbed attention"),
    "v3_prefill": ("v3_prefill", "V3-shaped prompt chunk: H=128, 4096 positions, no cached prefix, "
                                 "causal unabsorbed attention"),
    "v2lite_prompt_layer": ("v2lite_layer", "one V2-Lite layer over a 4096-token prompt: front (projections, "
                                            "RMSNorm, RoPE), causal unabsorbed attention, W_O + residual"),
}
DTYPES = {"bf16": 0, "int8": 1, "int4": 2, "int4s": 3, "int8t": 4, "fp8t": 5, "int4k4": 6, "int8c": 7}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _host_info():
    """CPU model, the threads numpy's BLAS uses, and which BLAS it is."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        info = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if info:
            blas = "%s %s" % (info[0].get("internal_api"), info[0].get("version"))
            threads = int(info[0].get("num_threads", threads))
    except Exception:       # threadpoolctl missing: keep the affinity count
        pass
    return model, blas, threads


def cpu_baseline(case, cache_dtype, budget_s=20.0):
    """Time the oracle's float32 absorbed decode (numpy with its BLAS, all host
    cores) on whole sequences of the workload; quantised caches include
    dequantising the sample.  The sample is sized so that three runs take about
    budget_s; the median of the three is reported as GB/s of latent cache."""
    from oracle import mla_ref, quant
    f32 = np.float32
    wk = mla_ref.bf16_to_f64(case.w_uk).astype(f32)
    wv = mla_ref.bf16_to_f64(case.w_uv).astype(f32)
    bpt = quant.token_bytes(cache_dtype)

    def prepare(b):
        c_bits, r_bits = case.seq_cache(b)
        qn = mla_ref.bf16_to_f64(case.q_nope[b]).astype(f32)
        qp = mla_ref.bf16_to_f64(case.q_pe[b]).astype(f32)
        if cache_dtype == 0:
            return (qn, qp, mla_ref.bf16_to_f64(c_bits).astype(f32), mla_ref.bf16_to_f64(r_bits).astype(f32))
        return (qn, qp, quant.encode_tokens(cache_dtype, c_bits, r_bits))

    def one(item):
        if cache_dtype == 0:
            qn, qp, c, r = item
        else:
            qn, qp, fields = item
            c, r = quant.dequant_fields(cache_dtype, fields)
        mla_ref.absorbed_decode_f32(qn, qp, c, r, wk, wv, case.softmax_scale)

    order = sorted(range(case.B), key=lambda b: int(case.seq_lens[b]))
    sample, t_one = [], 0.0
    for b in order:                       # grow the sample until one pass costs budget_s / 3
        item = prepare(b)
        t0 = time.perf_counter()
        one(item)
        t_one += time.perf_counter() - t0
        sample.append((b, item))
        if t_one >= budget_s / 3:
            break
    # a timed run repeats the sample (the whole workload when it is small) so that
    # the three runs together take about budget_s
    reps = max(1, int(round(budget_s / 3 / max(t_one, 1e-3))))
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        for _ in range(reps):
            for _, item in sample:
                one(item)
        runs.append(time.perf_counter() - t0)
    t_med = float(np.median(runs))
    tokens = reps * int(sum(int(case.seq_lens[b]) for b, _ in sample))
    model, blas, threads = _host_info()
    return {"value": round(tokens * bpt / t_med / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of %d sequences (%d tokens) x %d passes per run, float32 numpy absorbed decode incl. "
                      "W_UK/W_UV%s; median of 3 runs (%s s)" % (len(sample), case.B, tokens // reps, reps,
                                                             "" if cache_dtype == 0 else " and dequantisation",
                                                             ", ".join("%.2f" % r for r in runs)),
            "cpu_model": model, "blas": blas,
            "tflops": round(2176.0 * case.H * tokens / t_med / 1e12, 5)}


def prefill_flops(case):
    """Algorithmic FLOPs of one mla_prefill_attn call: the K/V expansion
    (2 x 512 x 256 per position and head) and the attention (2 x (192 + 128) per
    query, visible key and head)."""
    pos = case.L - case.T + np.arange(case.T, dtype=np.int64)
    return case.H * (2.0 * 512 * 256 * case.L + 640.0 * float(np.sum(pos + 1)))


def cpu_baseline_prefill(case, budget_s=15.0):
    """Time the oracle's prefill (fp64 numpy) on leading sub-chunks of the prompt
    (positions 0..n-1, n doubling from 64) until ~budget_s; report TFLOP/s."""
    from oracle import mla_ref, prefill
    f = mla_ref.bf16_to_f64
    wk, wv = f(case.w_uk), f(case.w_uv)
    n, t_total, flops, done = 64, 0.0, 0.0, []
    while n <= case.L:
        t0 = time.perf_counter()
        prefill.prefill_unabsorbed(f(case.q_nope[:n]), f(case.q_pe[:n]), f(case.c[:n]), f(case.r[:n]), wk, wv,
                                   case.softmax_scale)
        dt = time.perf_counter() - t0
        t_total += dt
        flops += case.H * (2.0 * 512 * 256 * n + 640.0 * n * (n + 1) / 2)
        done.append(n)
        n *= 2
        if t_total + 3 * dt > 2 * budget_s:         # the next size costs about 2-4x this one
            break
    cores = len(os.sched_getaffinity(0))
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "fp64 numpy prefill of the prompt's first n positions, n in %s, %.1f s" % (done, t_total)}


def bench_prefill(args):
    import torch
    import mla_synth
    from mla_absorbed_latent_amd import api

    gen, desc = PREFILL_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.workload == "v2lite_prompt_layer":
        from mla_absorbed_latent_amd.runner import PrefillLayer
        case = mla_synth.v2lite_layer(T=4096)
        case.L = case.T
        cfg = api.config(case.H, 0, case.softmax_scale)
        layer = PrefillLayer(cfg, case.T, case.hidden, dev)
        x0 = bits(case.x)
        x1 = torch.empty_like(x0)
        w = [bits(a) for a in (case.w_q, case.w_dkv, case.w_uk, case.w_uv, case.w_o)]
        proj = 2.0 * case.T * case.hidden * (case.H * 192 + 576 + case.H * 128)

        def step():
            layer.forward(x0, *w, x1)
    else:
        case = getattr(mla_synth, gen)()
        cfg = api.config(case.H, 0, case.softmax_scale)
        q_nope, q_pe, c, r = bits(case.q_nope), bits(case.q_pe), bits(case.c), bits(case.r)
        w_uk, w_uv = bits(case.w_uk), bits(case.w_uv)
        ws = torch.empty(api.prefill_workspace_bytes(cfg, case.L), dtype=torch.uint8, device=dev)
        out = torch.empty(case.T, case.H, 128, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(case.T, case.H, dtype=torch.float32, device=dev)
        proj = 0.0

        def step():
            api.prefill_attn(cfg, q_nope, q_pe, c, r, w_uk, w_uv, ws, out, lse)

    settled = settle(torch, step, min_s=args.settle_s, chunk=5) if args.settle_s > 0 else None
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(starts, ends)]))
    flops = prefill_flops(case) + proj
    tf = flops / (call_ms * 1e-3) / 1e12
    line = {
        "metric": ("MLA prompt layer (front, unabsorbed causal attention, W_O): TFLOP/s" if proj
                   else "MLA prefill attention (unabsorbed, causal): TFLOP/s"),
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; shapes and distributions of the workload, no checkpoint)",
        "config": {"workload": args.workload, "description": desc, "heads": case.H, "queries": case.T,
                   "positions": case.L},
        "tokens_per_s": round(case.T / (ms_step * 1e-3), 1),
        "roofline": {"bound": "mfma", "kernel": ("PrefillLayer.forward (front, prefill, W_O + residual)" if proj
                                                 else "mla_prefill_attn (expand_kv + prefill_attn)"),
                     "achieved": round(tf, 2), "peak": MFMA_PEAK_TFLOPS_16, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_PEAK_TFLOPS_16, 4), "traffic": None, "launch_ms": round(call_ms, 5),
                     "flops_per_launch": flops},
        "settle": settled,
    }
    if not args.no_cpu_baseline and not proj:
        log("timing the CPU oracle on a sample ...")
        line["cpu_baseline"] = cpu_baseline_prefill(case)
    print(json.dumps(line), flush=True)


def _bench_lib():
    from mla_absorbed_latent_amd import _lib
    return _lib.load()


def clock_probe_ghz(torch, dev):
    """The shader clock now: a one-wave spin timed by the shader-clock counter
    against the constant 100 MHz counter (mla_bench_clock_probe)."""
    import ctypes as C
    out = torch.zeros(3, dtype=torch.int64, device=dev)
    err = _bench_lib().mla_bench_clock_probe(40000, C.c_void_p(out.data_ptr()),
                                             C.c_void_p(torch.cuda.current_stream().cuda_stream))
    if err:
        raise RuntimeError("mla_bench_clock_probe: hipError %d" % err)
    torch.cuda.synchronize()
    cyc, ticks, _ = (int(v) for v in out.cpu())
    return round(cyc / ticks * 0.1, 3) if ticks > 0 else None


def measured_peaks(torch, dev):
    """Achievable rates on this card in this run (context for the vendor peaks),
    from the library's own microbenchmarks: a 4 GiB streaming read with 16-byte
    loads, and independent chains of 32x32x16 fp16 / bf16 MFMAs on registers over
    the whole chip (each: best of 5 after a warm-up)."""
    import ctypes as C
    lib = _bench_lib()
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    blocks = 8192
    red = torch.empty(blocks, dtype=torch.int32, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        best = []
        for _ in range(reps):
            ev0.record()
            fn()
            ev1.record()
            torch.cuda.synchronize()
            best.append(ev0.elapsed_time(ev1) * 1e-3)
        return min(best), float(np.median(best))

    def read():
        err = lib.mla_bench_stream_read(C.c_void_p(buf.data_ptr()), nbytes, C.c_void_p(red.data_ptr()), blocks, stream)
        if err:
            raise RuntimeError("mla_bench_stream_read: hipError %d" % err)

    t_read, t_read_med = timed(read)
    read_clock = clock_probe_ghz(torch, dev)
    del buf, red
    wgs, iters = 512, 4000
    out = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    flop = 2.0 * 32 * 32 * 16 * 8 * iters * 4 * wgs
    res = {}
    for name, bf in (("f16", 0), ("bf16", 1)):
        def mm(bf=bf):
            err = lib.mla_bench_mfma_loop(bf, iters, wgs, C.c_void_p(out.data_ptr()), stream)
            if err:
                raise RuntimeError("mla_bench_mfma_loop: hipError %d" % err)
        t, _ = timed(mm)
        res[name] = flop / t / 1e12
        res[name + "_clock"] = clock_probe_ghz(torch, dev)
    # per-CU intake from L2: one 512-thread work-group per CU, each on its own
    # 64 KB slice (16 MB in all: resident in the 8 x 4 MB L2s)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    slices = torch.ones(cus * 16384, dtype=torch.float32, device=dev)
    sink = torch.empty(cus * 8, dtype=torch.int32, device=dev)
    cyc = torch.empty(cus, dtype=torch.int64, device=dev)
    cu_read = {}
    for name, dma in (("plain", 0), ("lds_dma", 1)):
        for it in (50, 2000):        # warm-up, then measured
            err = lib.mla_bench_cu_read(C.c_void_p(slices.data_ptr()), cus, it, dma, C.c_void_p(sink.data_ptr()),
                                        C.c_void_p(cyc.data_ptr()), stream)
            if err:
                raise RuntimeError("mla_bench_cu_read: hipError %d" % err)
        torch.cuda.synchronize()
        cu_read[name] = round(2000 * 65536 / float(cyc.double().mean()), 1)
    del slices, sink, cyc
    return {"hbm_read_gbs": round(nbytes / t_read / 1e9, 1), "hbm_read_gbs_median": round(nbytes / t_read_med / 1e9, 1),
            "mfma_f16_tflops": round(res["f16"], 1), "mfma_bf16_tflops": round(res["bf16"], 1),
            "l2_read_bytes_per_cu_cycle": cu_read,
            "clock_ghz_after": {"read": read_clock, "mfma_f16": res["f16_clock"], "mfma_bf16": res["bf16_clock"]},
            "how": "mla_bench_stream_read over 4 GiB (16-byte non-temporal loads, 8192 work-groups); "
                   "mla_bench_mfma_loop: 512 work-groups x 4 waves x 8 independent 32x32x16 chains x 4000; "
                   "best of 5 after one warm-up; mla_bench_cu_read: one 512-thread work-group per CU re-reading "
                   "its own L2-resident 64 KB slice 2000 times, plain or direct-to-LDS 16-byte loads, "
                   "shader cycles from s_memtime"}


def settle(torch, step, min_s=1.0, max_s=6.0, chunk=20):
    """Run untimed steps until the card's clock has settled under this load:
    at least min_s of wall time and two consecutive chunks of `chunk` steps
    within 1.5 % of each other (at most max_s).  From idle the clock takes some
    tens of milliseconds to ramp up, so runs with a short warm-up read slow."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.time()
    ms, n = [], 0
    while True:
        ev0.record()
        for _ in range(chunk):
            step()
        ev1.record()
        torch.cuda.synchronize()
        n += chunk
        ms.append(ev0.elapsed_time(ev1) / chunk)
        el = time.time() - t0
        if el >= max_s or (el >= min_s and len(ms) >= 2 and abs(ms[-1] - ms[-2]) <= 0.015 * ms[-1]):
            break
    return {"seconds": round(time.time() - t0, 3), "steps": n,
            "first_chunks_ms_per_step": [round(v, 5) for v in ms[:3]],
            "last_chunks_ms_per_step": [round(v, 5) for v in ms[-2:]]}


def recorded_traffic(workload, cache_dtype):
    """HBM bytes per launch of mla_decode_attn measured with rocprofv3 FETCH_SIZE /
    WRITE_SIZE (scaled by a plain-copy calibration), as recorded in
    profiles/decode_attn_<workload>_<cache dtype>.md -- or None when that record is
    missing or was taken on a different version of the kernel source."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "decode_attn_%s_%s.md" % (workload, cache_dtype))
    src = os.path.join(ROOT, "mla_absorbed_latent_amd", "csrc", "kernels", "decode_attn.hip")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path, encoding="utf-8").read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha or rec.get("cache_dtype") != cache_dtype:
        return None
    return rec.get("traffic_bytes")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    # From idle the card's clock takes some tens of milliseconds of sustained
    # load to ramp up: untimed steps run first until it has settled (recorded
    # in the JSON line), whatever --warmup is.
    ap.add_argument("--settle-s", type=float, default=1.0)
    ap.add_argument("--workload", default="v3_decode", choices=sorted(WORKLOADS) + sorted(PREFILL_WORKLOADS))
    ap.add_argument("--cache-dtype", default="bf16", choices=sorted(DTYPES))
    ap.add_argument("--chunk-pages", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")     # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4, "copies": 3}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the decode shards by sequence "
              "with no exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.workload in PREFILL_WORKLOADS:
        return bench_prefill(args)

    import torch
    import mla_synth
    from mla_absorbed_latent_amd import api
    from mla_absorbed_latent_amd.runner import DecodeRunner

    gen, desc = WORKLOADS[args.workload]
    case = getattr(mla_synth, gen)()
    cache_dtype = DTYPES[args.cache_dtype]
    dev = torch.device("cuda:0")
    cfg = api.config(case.H, cache_dtype, case.softmax_scale)
    # The step appends each sequence's newest token (position L - 1) again.  For
    # the per-channel INT8 cache that position closes a 32-token block, and
    # closing it again over the block's already-quantised rows would read codes
    # as bf16: there the step's tokens go to one spare page per sequence (outside
    # the block table), so every step does the same closing work on valid data.
    spare = case.B if cache_dtype == 7 else 0
    run = DecodeRunner(cfg, case.B, case.num_pages + spare, dev)

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- fill the cache through the library (bulk append), then the step's inputs
    t0 = time.time()
    last_c, last_r, last_s = [], [], []
    pend = ([], [], [])
    n_pend = 0
    for b in range(case.B):
        c, r = case.seq_cache(b)
        s = case.slots_of(b)
        pend[0].append(c)
        pend[1].append(r)
        pend[2].append(s)
        n_pend += len(s)
        last_c.append(c[-1])
        last_r.append(r[-1])
        last_s.append(s[-1])
        if n_pend >= (1 << 19) or b == case.B - 1:
            run.append(bits(np.concatenate(pend[0])), bits(np.concatenate(pend[1])),
                       torch.from_numpy(np.concatenate(pend[2])).to(dev))
            pend = ([], [], [])
            n_pend = 0
    new_c = bits(np.stack(last_c))
    new_r = bits(np.stack(last_r))
    if spare:
        last_s = [(case.num_pages + b) * 64 + int(s) % 64 for b, s in enumerate(last_s)]
    new_s = torch.from_numpy(np.array(last_s, np.int64)).to(dev)
    q_nope, q_pe = bits(case.q_nope), bits(case.q_pe)
    w_uk, w_uv = bits(case.w_uk), bits(case.w_uv)
    block_table = torch.from_numpy(case.block_table).to(dev)
    seq_lens = torch.from_numpy(case.seq_lens.astype(np.int32)).to(dev)
    n_items = run.plan(case.seq_lens, chunk_pages=args.chunk_pages)
    torch.cuda.synchronize()
    log("setup %.1f s: %s, %d tokens, %d work items" % (time.time() - t0, desc, case.total_tokens, n_items))

    # A cache smaller than 1 GiB could stay in the 256 MB Infinity Cache between
    # steps: rotate identical copies of the pool so that every step streams from HBM.
    pools = [run.pool]
    while len(pools) * run.pool.numel() < (1 << 30) and len(pools) < 16:
        pools.append(run.pool.clone())
    rot = [0]

    def next_pool():
        run.pool = pools[rot[0] % len(pools)]
        rot[0] += 1

    def step():
        next_pool()
        run.step(q_nope, q_pe, w_uk, w_uv, block_table, seq_lens, new_c, new_r, new_s, keep_latent=False)

    clock_idle = clock_probe_ghz(torch, dev)
    settled = settle(torch, step, min_s=args.settle_s) if args.settle_s > 0 else None
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    clock_after = clock_probe_ghz(torch, dev)

    # ---- the dominant kernel alone: mla_decode_attn back to back, one pair of
    # events on its launch stream around all of them (an event pair per launch
    # would add its markers' gaps to every launch)
    stream = torch.cuda.current_stream()
    run.absorb(q_nope, q_pe, w_uk)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        next_pool()
        run.attend(block_table, seq_lens)
    ev1.record(stream)
    torch.cuda.synchronize()
    attn_ms = ev0.elapsed_time(ev1) / args.steps
    # combine alone (for t_attn = decode_attn + combine)
    ev0.record()
    for _ in range(args.steps):
        run.combine()
    ev1.record()
    torch.cuda.synchronize()
    comb_ms = ev0.elapsed_time(ev1) / args.steps

    achievable = measured_peaks(torch, dev)
    traffic = recorded_traffic(args.workload, args.cache_dtype)
    traffic_src = ("recorded: profiles/decode_attn_%s_%s.md (rocprofv3 FETCH_SIZE + WRITE_SIZE at this kernel "
                   "source hash)" % (args.workload, args.cache_dtype)) if traffic is not None else None
    bpt = api.cache_bytes_per_token(cfg)
    latent_bytes = case.total_tokens * bpt
    flops = 2176.0 * case.H * case.total_tokens
    attn_gbs = latent_bytes / (attn_ms * 1e-3) / 1e9
    step_gbs = latent_bytes / (ms_step * 1e-3) / 1e9
    t_attn_ms = attn_ms + comb_ms
    roof_t = max(latent_bytes / (HBM_PEAK_GBS * 1e9), flops / (MFMA_PEAK_TFLOPS_16 * 1e12))

    line = {
        "metric": "MLA absorbed decode: latent-cache GB/s, TFLOP/s, % roofline (H=128, B=64)",
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "f16", 1: "i8/f16", 2: "i4/f16", 3: "i4s/f16", 4: "i8t/f16", 5: "e4m3t/f16", 6: "i4s+k4/f16",
                  7: "i8c/f16"}[cache_dtype],
        "data": "synthetic (seeded; shapes and distributions of the workload, no checkpoint)",
        "config": {"workload": args.workload, "description": desc, "batch": case.B, "heads": case.H,
                   "cached_tokens": case.total_tokens, "cache_dtype": args.cache_dtype,
                   "work_items": n_items, "page_tokens": 64},
        "step_tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "tokens_per_s": round(case.B / (ms_step * 1e-3), 1),
        "t_attn_ms": round(t_attn_ms, 5),
        "attn_gbs": round(latent_bytes / (t_attn_ms * 1e-3) / 1e9, 2),
        "attn_tflops": round(flops / (t_attn_ms * 1e-3) / 1e12, 2),
        "pct_roofline_attn": round(100.0 * roof_t / (t_attn_ms * 1e-3), 2),
        "roofline": {"bound": "hbm", "kernel": "mla_decode_attn", "achieved": round(attn_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "traffic_source": traffic_src, "launch_ms": round(attn_ms, 5),
                     "bytes_per_launch": latent_bytes,
                     "mfma_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 2),
                     "mfma_frac": round(flops / (attn_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS_16, 4),
                     "frac_of_measured_hbm": round(attn_gbs / achievable["hbm_read_gbs"], 4),
                     "mfma_frac_of_measured": round(flops / (attn_ms * 1e-3) / 1e12 / achievable["mfma_f16_tflops"], 4)},
        "measured_peaks": achievable,
        "pool_copies": len(pools),
        "settle": settled,
        "shader_clock_ghz": {"idle_before": clock_idle, "right_after_timed_steps": clock_after},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        line["cpu_baseline"] = cpu_baseline(case, cache_dtype)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
