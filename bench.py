"""Benchmark of the masked varlen attention hot path on one MI355X.

One step = one pass of the prefill path over one layer's batch:
  1. build the per-query-row range table on the host (library builder) into
     pinned staging memory,
  2. upload it to its persistent device buffer (asynchronously, on a side
     stream; the kernel waits for its own upload's event),
  3. run the prefill kernel.
Inputs (Q, K, V, cu_seqlens) are resident in HBM before timing starts.

The headline layer is the chunked-prefill global layer (bf16, 8 requests of
6144 cached + 2048 new tokens, 8 q / 4 kv heads, head_dim 512, causal,
multimodal ranges clipped to the chunk), the largest of the workloads that
fit one GPU. The same run times the other prefill layers (the multimodal-prefix
sliding layer at head_dim 256, the vision-encoder window at head_dim 128 and
the global layer read from a paged cache) and the paged-decode kernels on the
64-sequence, 4K-32K context workload (full-attention and 4096-key window
layers), each with its own kernel time and roofline fraction.

Printed: one JSON line with the metric, the headline layer's useful TFLOP/s
(only visible, window-clamped pairs count, as the library's accounting
function counts them), its kernel's roofline fraction measured with HIP events
on its launch stream, and the CPU oracle timed on a bounded sample of the same
workload (`cpu_baseline`). Under "table": the median microseconds of the host
build, its upload, and the device-side build of the headline layer's table
(outside the timed steps).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "masked attn prefill useful TFLOP/s + decode KV GB/s, % of MI355X roofline"
WORKLOADS = {
    "c2": ("mm-prefix sliding layer: bf16, 4 requests x 4096 tokens, 16 q / 8 kv heads, head_dim 256, causal + "
           "window 1024, 8-16 bidirectional 256-token ranges per request"),
    "c3": ("chunked-prefill global layer: bf16, 8 requests x (6144 context + 2048 chunk), 8 q / 4 kv heads, "
           "head_dim 512, causal, mm-prefix ranges clipped to the chunk"),
    "c4": ("vision-encoder window: bf16, 16 images of 1024-4096 patches, 16 heads, head_dim 128, non-causal, "
           "window 128 both sides, key-0 sinks"),
    "c3_paged": ("chunked-prefill global layer with K/V read from a paged cache: bf16, 8 requests x (6144 context + "
                 "2048 chunk), 16-token HND pages in random order, 8 q / 4 kv heads, head_dim 512, causal, mm-prefix "
                 "ranges"),
}
HEADLINE = "c3"  # the largest single-GPU configuration
OTHER_LAYERS = ("c2", "c4", "c3_paged")
PAGE_SIZE = 16
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E


def profiled_traffic(workload):
    """HBM bytes per call measured for ``workload`` by rocprofv3 counters.

    Read from the ``traffic-record:`` lines of the summaries in ``profiles/``
    (``2.0 * FETCH_SIZE + 1.0 * WRITE_SIZE`` KiB, the factors from a 1 GiB copy).
    A record counts only while its ``source_sha256`` equals the digest of the
    current sources of that kernel (``build.KERNEL_SOURCES``); otherwise the
    counters describe other code and the result is None.
    """
    import glob

    from masked_varlen_softmax_amd import build

    digest = build.source_digest("decode" if workload.startswith("c5") else "prefill")
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("traffic-record:"):
                    continue
                rec = json.loads(line.split(":", 1)[1])
                if rec["workload"] == workload and rec["source_sha256"] == digest:
                    return int(round(1024 * (rec["fetch_kib"] * rec["fetch_factor"]
                                             + rec["write_kib"] * rec["write_factor"])))
    return None


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _to_dev(a, dev):
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _spin_up(fn, ms):
    """Untimed back-to-back calls of fn for `ms` of wall time before the warmup steps.

    The GPU raises its clocks over the first few tens of milliseconds of
    sustained work: the sliding-layer prefill kernel takes 0.40 ms in the first
    calls after idle and 0.316 ms from about 40 ms on. The timed steps measure
    the steady state a serving loop runs in, not that ramp.
    """
    import torch

    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def algorithmic_bytes(case, with_table):
    """Mandatory HBM bytes of one prefill launch: Q, K, V read once, O written once, and the table."""
    eb = 2 if case.dtype == "bf16" else 4
    nq, nk = int(case.cu_q[-1]), int(case.cu_k[-1])
    qo = 2 * nq * case.Hq * case.D * eb
    kv = 2 * nk * case.Hkv * case.D * eb
    return qo + kv + (nq * 8 if with_table else 0)


def bench_prefill(args, dev, workload, table_timing=False):
    """Time `workload`'s step (host table build + upload + kernel); HIP events bracket each kernel."""
    import torch

    import masked_varlen_softmax_amd as mvs
    from masked_varlen_softmax_amd import workloads as W

    paged = workload.endswith("_paged")
    case = W.PREFILL_CONFIGS[workload.removesuffix("_paged")]()
    N = case.q.shape[0]
    q = _to_dev(case.q, dev)
    cu_q, cu_k = _to_dev(case.cu_q, dev), _to_dev(case.cu_k, dev)
    if paged:
        kc, vc, bt = W.paged_kv(case, PAGE_SIZE, 77)
        k, v, bt = _to_dev(kc, dev), _to_dev(vc, dev), _to_dev(bt, dev)
        seq_lens_k = _to_dev(case.lens_k.astype(np.int32), dev)
        del kc, vc
    else:
        k, v = _to_dev(case.k, dev), _to_dev(case.v, dev)
    out = torch.empty_like(q)
    offs, pairs = case.ranges_csr()
    lens_k = case.lens_k.astype(np.int32)
    max_q, max_k = int(case.lens_q.max()), int(case.lens_k.max())
    stream = torch.cuda.current_stream()
    # The table of step i+1 is built on the host and uploaded on a side stream
    # while step i's kernel runs; each step's kernel waits for its own upload.
    # Staging and device tables are double buffered: buffer b is rebuilt only
    # after the kernel that last read it has finished (its event).
    upload = torch.cuda.Stream(device=dev)  # default priority
    staging = [torch.empty((N, 2), dtype=torch.int32).pin_memory() for _ in range(2)]
    table_dev = [torch.empty((N, 2), dtype=torch.int32, device=dev) for _ in range(2)]
    uploaded = [torch.cuda.Event(), torch.cuda.Event()]
    consumed = [torch.cuda.Event(), torch.cuda.Event()]
    sinks = None if case.sinks is None else torch.from_numpy(case.sinks).to(dev)
    it = [0]

    def step(ev=None):
        buf = it[0] & 1
        it[0] += 1
        consumed[buf].synchronize()
        n = mvs.build_query_range_table(staging[buf], (offs, pairs), case.cu_q, lens_k)
        tab = None
        if n:
            upload.wait_event(consumed[buf])
            with torch.cuda.stream(upload):
                table_dev[buf][:n].copy_(staging[buf][:n], non_blocking=True)
            uploaded[buf].record(upload)
            stream.wait_event(uploaded[buf])
            tab = table_dev[buf][:n]
        if ev is not None:
            ev[0].record(stream)
        if paged:
            mvs.attn_varlen_fwd_paged(q, k, v, bt, cu_q, seq_lens_k, max_q, max_k, case.scale, case.causal, case.wl,
                                      case.wr, tab, sinks, case.sink_mode, out=out, stream=stream)
        else:
            mvs.attn_varlen_fwd(q, k, v, cu_q, cu_k, max_q, max_k, case.scale, case.causal, case.wl, case.wr, tab,
                                sinks, case.sink_mode, out=out, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        consumed[buf].record(stream)
        return n

    n_rows = step()
    torch.cuda.synchronize()
    host_table = staging[0].numpy().copy() if n_rows else None
    flops = mvs.prefill_useful_flops(case.cu_q, case.cu_k, case.Hq, case.D, case.causal, case.wl, case.wr,
                                     host_table)
    _spin_up(step, args.spin_up_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # K whole steps (host build + upload + kernel), wall clock around them; HIP
    # events on the launch stream bracket each kernel inside the same region
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kms = np.array([a.elapsed_time(b) for a, b in evs])
    res = {
        "workload": workload,
        "case": case,
        "table": _time_table_builders(case, dev) if table_timing and offs.size > 1 and pairs.size else None,
        "host_table": host_table,
        "useful_flops": flops,
        "alg_bytes": algorithmic_bytes(case, n_rows > 0),
        "step_ms": step_ms,
        "kernel_ms": float(kms.mean()),
        "kernel_ms_min": float(kms.min()),
        "kernel_ms_median": float(np.median(kms)),
    }
    del q, k, v, out, table_dev
    torch.cuda.empty_cache()
    return res


def layer_record(pre):
    """The per-layer summary carried in the JSON line: kernel time, both rooflines, traffic."""
    case = pre["case"]
    tflops = pre["useful_flops"] / (pre["kernel_ms"] * 1e-3) / 1e12
    gbps = pre["alg_bytes"] / (pre["kernel_ms"] * 1e-3) / 1e9
    intensity = pre["useful_flops"] / pre["alg_bytes"]
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    bound = "mfma" if intensity >= ridge else "hbm"
    traffic = profiled_traffic(pre["workload"])
    return {
        "workload": WORKLOADS[pre["workload"]],
        "useful_gflop": round(pre["useful_flops"] / 1e9, 3),
        "algorithmic_mb": round(pre["alg_bytes"] / 1e6, 2),
        "flop_per_byte": round(intensity, 1),
        "bound": bound,
        "kernel_ms_mean": round(pre["kernel_ms"], 4),
        "kernel_ms_min": round(pre["kernel_ms_min"], 4),
        "step_ms": round(pre["step_ms"], 4),
        "tflops": round(tflops, 2),
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "hbm_GBps": round(gbps, 1),
        "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
        "frac": round((tflops / PEAK_BF16_TFLOPS) if bound == "mfma" else (gbps / PEAK_HBM_GBPS), 4),
        "traffic": traffic,
        "traffic_over_algorithmic": None if traffic is None else round(traffic / pre["alg_bytes"], 3),
        "heads": [int(case.Hq), int(case.Hkv)], "head_dim": int(case.D),
    }


def _time_table_builders(case, dev, reps=100):
    """Median microseconds of the table's host build, its upload, and the device-side build."""
    import torch

    import masked_varlen_softmax_amd as mvs

    N = case.q.shape[0]
    offs, pairs = case.ranges_csr()
    lens_k = case.lens_k.astype(np.int32)
    staging = torch.empty((N, 2), dtype=torch.int32).pin_memory()
    table = torch.empty((N, 2), dtype=torch.int32, device=dev)
    host_us, h2d_us = [], []
    for _ in range(reps):
        t0 = time.perf_counter()
        mvs.build_query_range_table(staging, (offs, pairs), case.cu_q, lens_k)
        host_us.append((time.perf_counter() - t0) * 1e6)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(reps):
        ev[0].record()
        table.copy_(staging, non_blocking=True)
        ev[1].record()
        ev[1].synchronize()
        h2d_us.append(ev[0].elapsed_time(ev[1]) * 1e3)
    qsl, sl = _to_dev(case.cu_q, dev), _to_dev(lens_k, dev)
    od, pd = _to_dev(offs, dev), _to_dev(pairs, dev)
    dev_us = []
    for _ in range(reps):
        ev[0].record()
        mvs.build_query_range_table_device(table, qsl, sl, od, pd)
        ev[1].record()
        ev[1].synchronize()
        dev_us.append(ev[0].elapsed_time(ev[1]) * 1e3)
    return {"rows": N, "ranges": int(pairs.shape[0]), "host_build_us": round(float(np.median(host_us)), 1),
            "h2d_us": round(float(np.median(h2d_us)), 1), "device_build_us": round(float(np.median(dev_us)), 1)}


def range_sweep(args, dev, counts=(1, 8, 16, 32, 46, 64)):
    """Table lookup against the range-scan baseline on the sliding layer with n frames per request."""
    import torch

    import masked_varlen_softmax_amd as mvs
    from masked_varlen_softmax_amd import workloads as W

    rows = []
    for n in counts:
        case = W.c2_range_count(n)
        N = case.q.shape[0]
        q, k, v = _to_dev(case.q, dev), _to_dev(case.k, dev), _to_dev(case.v, dev)
        cu_q, cu_k = _to_dev(case.cu_q, dev), _to_dev(case.cu_k, dev)
        host = np.full((N, 2), -1, dtype=np.int32)
        mvs.build_query_range_table(host, case.ranges_csr(), case.cu_q, case.lens_k.astype(np.int32))
        table = _to_dev(host, dev)
        ranges = _to_dev(W.padded_ranges(case, n), dev)
        out = torch.empty_like(q)
        Lq, Lk = int(case.lens_q.max()), int(case.lens_k.max())
        flops = mvs.prefill_useful_flops(case.cu_q, case.cu_k, case.Hq, case.D, True, case.wl, -1, host)
        calls = {
            "table": lambda: mvs.attn_varlen_fwd(q, k, v, cu_q, cu_k, Lq, Lk, case.scale, True, case.wl, -1, table,
                                                 out=out),
            "scan": lambda: mvs.attn_varlen_fwd_range_scan(q, k, v, cu_q, cu_k, Lq, Lk, case.scale, ranges, True,
                                                           case.wl, -1, out=out),
        }
        row = {"ranges_per_request": n, "frame_tokens": int(case.ranges[0][0][1] - case.ranges[0][0][0] + 1),
               "useful_gflop": round(flops / 1e9, 3)}
        for name, fn in calls.items():
            _spin_up(fn, args.spin_up_ms / 2)
            for _ in range(args.warmup):
                fn()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            for a, b in evs:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
            row[f"{name}_ms"] = round(ms, 4)
            row[f"{name}_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
        row["scan_over_table"] = round(row["scan_ms"] / row["table_ms"], 3)
        _log(f"range sweep n={n}: table {row['table_ms']} ms, scan {row['scan_ms']} ms")
        rows.append(row)
        del q, k, v, out
    return rows


def bench_decode(args, dev):
    import torch

    import masked_varlen_softmax_amd as mvs
    from masked_varlen_softmax_amd import workloads as W

    res = {}
    # 1 GiB read before each timed call evicts the 256 MB last-level cache. It
    # only reads: a flush that writes would leave dirty lines whose write-back
    # the decode kernel would then pay for.
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    for window in (False, True):
        case = W.c5_paged_decode(window)
        B = len(case.seq_lens)
        q = _to_dev(case.q, dev)
        kc, vc = _to_dev(case.k_cache, dev), _to_dev(case.v_cache, dev)
        bt, sl = _to_dev(case.block_table, dev), _to_dev(case.seq_lens, dev)
        out = torch.empty_like(q)
        max_len = int(case.seq_lens.max())
        ws = torch.empty(mvs.attn_paged_decode_workspace_size(B, case.Hq, case.Hkv, case.D), dtype=torch.uint8,
                         device=dev)
        stream = torch.cuda.current_stream()

        def run():
            mvs.attn_paged_decode(q, kc, vc, bt, sl, max_len, case.scale, case.wl, out=out, workspace=ws)

        _spin_up(run, args.spin_up_ms)
        for _ in range(args.warmup):
            run()
        times = []
        for _ in range(args.steps):
            flush.sum()  # outside the timed region
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        t = np.array(times)
        nbytes = mvs.decode_useful_bytes(case.seq_lens, case.Hkv, case.D, 2, case.wl)
        res["window" if window else "full"] = {
            "useful_bytes": nbytes,
            "ms": float(t.mean()),
            "ms_min": float(t.min()),
            "GBps": nbytes / (t.mean() * 1e-3) / 1e9,
        }
        del kc, vc, q, bt, sl, out, ws
        torch.cuda.empty_cache()
    del flush
    tf, tw = profiled_traffic("c5_full"), profiled_traffic("c5_window")
    traffic = tf + tw if tf is not None and tw is not None else None
    tot_b = res["full"]["useful_bytes"] + res["window"]["useful_bytes"]
    tot_t = (res["full"]["ms"] + res["window"]["ms"]) * 1e-3
    agg = tot_b / tot_t / 1e9
    return {
        "workload": "paged decode: bf16, 64 seqs, q_len 1, contexts U[4096,32768], page 16, 32 q / 8 kv heads, "
                    "head_dim 128; full layer and 4096-key window layer",
        "full_GBps": round(res["full"]["GBps"], 1),
        "window_GBps": round(res["window"]["GBps"], 1),
        "full_ms": round(res["full"]["ms"], 4),
        "window_ms": round(res["window"]["ms"], 4),
        "aggregate_GBps": round(agg, 1),
        "roofline": {"bound": "hbm", "achieved": round(agg, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(agg / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "traffic_note": "HBM bytes of one full-layer plus one window-layer call (rocprofv3 counters)"},
    }


def _span(x):
    lo, hi = int(np.min(x)), int(np.max(x))
    return str(lo) if lo == hi else f"{lo}-{hi}"


def cpu_baseline(pre, min_s=10.0):
    """The oracle on whole requests of the timed prefill workload (all query heads), timed on the host.

    Requests are taken in order, wrapping around, until at least ``min_s`` seconds of CPU work
    have run; the rate is the useful FLOPs of the requests run over their total time.
    """
    import masked_varlen_softmax_amd as mvs
    from masked_varlen_softmax_amd import workloads as W
    from oracle import ref_attention

    case = pre["case"]
    B = len(case.lens_q)
    flops, dt, done = 0, 0.0, 0
    while done == 0 or (dt < min_s and done < 4 * B):
        b = done % B
        q0, q1 = int(case.cu_q[b]), int(case.cu_q[b + 1])
        k0, k1 = int(case.cu_k[b]), int(case.cu_k[b + 1])
        q, k, v = W.as_f32(case.q[q0:q1]), W.as_f32(case.k[k0:k1]), W.as_f32(case.v[k0:k1])
        tab = None if pre["host_table"] is None else pre["host_table"][q0:q1]
        cu_q, cu_k = np.array([0, q1 - q0]), np.array([0, k1 - k0])
        t0 = time.perf_counter()
        ref_attention(q, k, v, cu_q, cu_k, case.scale, case.causal, case.wl, case.wr, tab, case.sinks, case.sink_mode)
        dt += time.perf_counter() - t0
        flops += mvs.prefill_useful_flops(cu_q, cu_k, case.Hq, case.D, case.causal, case.wl, case.wr, tab)
        done += 1
    blas = "unknown BLAS"
    try:
        from threadpoolctl import threadpool_info

        info = threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] + [1])
        libs = [f"{i.get('internal_api', '?')} {i.get('version', '')}".strip() for i in info if i.get("user_api") == "blas"]
        if libs:
            blas = ", ".join(libs)
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    shape = (f"{_span(case.lens_q)} queries x {_span(case.lens_k)} keys each, all {case.Hq} q heads, head_dim "
             f"{case.D}")
    layer = WORKLOADS.get(pre["workload"], pre["workload"]).split(":")[0]  # what the layer is, not its key
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} whole requests of the {B} of the {layer} ({shape}; taken in order and "
                      f"wrapping around), dense fp32 NumPy {np.__version__} ({blas}, {cores} threads of "
                      f"{os.cpu_count()} host CPUs), {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--spin-up-ms", type=float, default=250.0,
                    help="untimed back-to-back calls before the warmup steps, so the GPU is at steady clocks")
    ap.add_argument("--prefill-workload", choices=sorted(WORKLOADS), default=HEADLINE,
                    help="prefill layer the headline value and roofline are quoted on")
    ap.add_argument("--layers", default=",".join(OTHER_LAYERS),
                    help="other prefill layers timed in the same run (comma list, or 'none')")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="decode only (profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--range-sweep", action="store_true",
                    help="time the table path against the range-scan baseline for 1-64 frames per request")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the kernels run on one GPU's share of the work and there is "
              "no multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    layers = [] if args.layers in ("", "none") else [x for x in args.layers.split(",") if x != args.prefill_workload]
    for x in layers:
        if x not in WORKLOADS:
            ap.error(f"unknown layer {x!r}; choose from {sorted(WORKLOADS)}")
    import torch

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": src.numel() * 4, "copies": args.steps}), flush=True)
        return
    if args.range_sweep:
        print(json.dumps({"range_sweep": range_sweep(args, dev),
                          "workload": "mm-prefix sliding layer, bf16, 4 x 4096, 16 q / 8 kv heads, head_dim 256, "
                                      "causal + window 1024, n frames of min(256, 4096 / n) tokens per request",
                          "timing": f"median of {args.steps} calls (HIP events), kernel only"}), flush=True)
        return
    if args.no_prefill:
        dec = bench_decode(args, dev)
        print(json.dumps({"metric": METRIC, "decode": dec}), flush=True)
        return
    _log(f"prefill {args.prefill_workload}: building inputs")
    pre = bench_prefill(args, dev, args.prefill_workload, table_timing=True)
    _log(f"prefill {args.prefill_workload}: kernel {pre['kernel_ms']:.4f} ms, step {pre['step_ms']:.4f} ms")
    others = {}
    for x in layers:
        _log(f"prefill {x}: building inputs")
        r = bench_prefill(args, dev, x)
        _log(f"prefill {x}: kernel {r['kernel_ms']:.4f} ms, step {r['step_ms']:.4f} ms")
        others[x] = layer_record(r)
        del r
    dec = None
    if not args.no_decode:
        _log("decode: building inputs")
        dec = bench_decode(args, dev)
        _log(f"decode: full {dec['full_GBps']} GB/s, window {dec['window_GBps']} GB/s")
    cpu = None
    if not args.no_cpu_baseline:
        _log("cpu baseline: oracle on a sample")
        cpu = cpu_baseline(pre)

    head = layer_record(pre)
    flops = pre["useful_flops"]
    value = flops / (pre["step_ms"] * 1e-3) / 1e12
    if head["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": head["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": head["mfma_frac"]}
    else:
        roof = {"bound": "hbm", "achieved": head["hbm_GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": head["hbm_frac"]}
    roof.update({"traffic": head["traffic"],
                 "traffic_note": "HBM bytes per launch (rocprofv3 counters; null if the kernel changed since)",
                 "kernel": f"prefill bf16 ({'attn_varlen_fwd_paged' if args.prefill_workload.endswith('_paged') else 'attn_varlen_fwd'})",
                 "kernel_ms_mean": head["kernel_ms_mean"], "kernel_ms_min": head["kernel_ms_min"],
                 "algorithmic_mb": head["algorithmic_mb"]})
    case = pre["case"]
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, random 256-token frames)",
        "config": {
            "workload": WORKLOADS[args.prefill_workload],
            "global_batch": int(case.num_seqs), "seq_len": int(case.lens_k.max()),
            "query_tokens": int(case.cu_q[-1]),
            "num_q_heads": int(case.Hq), "num_kv_heads": int(case.Hkv), "head_dim": int(case.D),
            "useful_gflop_per_step": round(flops / 1e9, 3),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "table": pre["table"],
        "prefill_layers": others,
        "decode": dec,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
