"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu] [--no-graph]

A step is one sliding-window+sink prefill of the SWA-layer workload
(n = 32768 tokens, 64 query / 8 kv heads, d_qk 192, d_v 128, W = 128,
partial RoPE base 1e4 on 64 dims, per-head sinks): the rows A1-A7 of the
hot path in one library call.  `value` is useful TFLOP/s: 640 FLOP per
unmasked (query head, key) pair, 171.47 GFLOP per step.

Printed as one JSON line, with
  * roofline: the prefill kernel against HBM bandwidth (algorithmic bytes
    Q + K + V + O per launch over its average event-timed duration);
  * cpu_baseline: the fp64 oracle timed on a bounded row sample of the same
    workload on the host cores;
  * secondary: the siblings measured the same way (GA prefill TFLOP/s,
    16K-token prefill chunks behind empty and long cached prefixes, hybrid
    decode HBM GB/s for the ring and contiguous caches, sparse prefill
    TFLOP/s).
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import hybrid_sliding_window_amd as hswa  # noqa: E402
import synthetic  # noqa: E402

METRIC = "SWA+sink prefill TFLOP/s (W=128, 64q/8kv) + decode HBM GB/s, % of roofline"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
FLOP_PER_PAIR = 2 * (192 + 128)      # QK^T and PV per unmasked (query head, key) pair
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _ensure_built():
    if not os.path.exists(hswa.lib_path()):
        from hybrid_sliding_window_amd.build import build
        build()
    hswa.load()


def window_pairs(n, window):
    """Unmasked (query, key) pairs of a causal window per head."""
    i = np.arange(n, dtype=np.int64)
    return int(np.minimum(i + 1, window).sum()) if window > 0 else int(((i + 1)).sum())


CLOCK_SETTLE_S = 0.3


def settle_clock(fn, seconds=CLOCK_SETTLE_S):
    """Back-to-back untimed calls for `seconds`: the shader clock ramps up
    over the first ~50 ms of sustained work (a 0.5 ms call measured right
    after idle runs ~16% slower than the same call at steady state)."""
    t0 = time.perf_counter()
    batch = 1
    while True:
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return
        batch = min(2 * batch, 64)


def timed(fn, steps, warmup):
    """Settle the clock, warm up, then time `steps` calls with an event pair
    around each one on the current stream (where the library enqueues its
    kernels)."""
    settle_clock(fn)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in zip(starts, ends):
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]   # ms
    return wall, per


def batched_us(fn, calls=200):
    """Per-call time of `calls` back-to-back calls between one event pair:
    for calls of a few microseconds the per-call event pair alone costs about
    6 us on this system, so this is the rate a serving loop sees."""
    settle_clock(fn)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(calls):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / calls


def graph_us(fn, calls=64, replays=20):
    """Device time per call with the host out of the loop: `calls` calls
    captured in one HIP graph (torch.cuda.CUDAGraph on torch's current
    device), replayed `replays` times between one event pair.  For calls of
    ~10 us the host-side argument checks of each call take longer than the
    kernel, so back-to-back eager calls measure the host (us_batched); a
    serving loop replays such steps as a graph."""
    settle_clock(fn)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) * 1e3 / (replays * calls)


def small_stream_bound_us(read_bytes, write_bytes):
    """Device time per call of hswa_stream_probe moving read_bytes in (from
    rotated sources, over 400 MB in all, so that the reads are not served
    from the 256 MB last-level cache) and write_bytes out, timed as graph_us:
    the bound for a one-launch step of that many bytes, launch ramp
    included.  Best of 1, 2 and 4 workgroups of 4 wavefronts per CU."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rb = (read_bytes + 1023) // 1024 * 1024
    wb = max(1024, (write_bytes + 1023) // 1024 * 1024)
    sets = max(8, -(-400_000_000 // rb))
    srcs = [torch.empty(rb, dtype=torch.uint8, device="cuda") for _ in range(sets)]
    dst = torch.empty(wb, dtype=torch.uint8, device="cuda")
    best = None
    for per_cu in (1, 2, 4):
        blocks = per_cu * cus
        o = torch.empty(4 * blocks, dtype=torch.int32, device="cuda")
        it = [0]

        def step():
            src = srcs[it[0] % sets]
            it[0] += 1
            hswa.stream_probe(src, dst, blocks, out=o)
        us = graph_us(step)
        if best is None or us < best[0]:
            best = (us, 4 * per_cu)
    del srcs, dst
    return {"us": best[0], "waves_per_cu": best[1], "read_bytes": rb, "write_bytes": wb}


GRAPH_TIMING = True   # cleared by --no-graph (profiler runs)


def _graph_entry(step, nbytes, read_bytes, write_bytes):
    if not GRAPH_TIMING:
        return None
    us = graph_us(step)
    bound = small_stream_bound_us(read_bytes, write_bytes)
    return {"us": us, "gbps": nbytes / us / 1e3, "frac_of_hbm_peak": nbytes / us / 1e3 / HBM_PEAK_GBPS,
            "stream_bound_us": bound["us"], "frac_of_stream_bound": bound["us"] / us,
            "note": "64 calls (rotated buffer sets) captured in one HIP graph and replayed: device "
                    "time per call; stream bound: hswa_stream_probe moving the same read and "
                    "written bytes in one launch, timed the same way"}


def _traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary.

    FETCH_SIZE and WRITE_SIZE were each taken in a run of their own and scaled
    by what the same counters read for a plain 1 GiB copy.  The entry records
    the hash of the kernel source it was measured on; once the source has
    changed the figure no longer applies and None is returned."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            entry = json.load(f).get(kernel_key)
        if entry is None:
            return None
        src = os.path.join(ROOT, entry["source"])
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if not digest.startswith(entry["source_sha256_prefix"]):
            return None
        return entry["bytes"]
    except (OSError, ValueError, KeyError):
        return None


def cpu_baseline(x, wl, budget_s):
    """The oracle, untuned, on a time-bounded sample of query rows."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    n, window = wl["n"], wl["window"]
    k = x["k"].double().cpu().numpy()
    v = x["v"].double().cpu().numpy()
    sink = x["sink"].double().cpu().numpy()
    rng = np.random.default_rng(7)
    order = rng.permutation(n)
    done, flops, t0 = 0, 0.0, time.perf_counter()
    chunk = 64
    while True:
        rows = np.sort(order[done:done + chunk])
        qr = x["q"][:, torch.from_numpy(rows).to(x["q"].device)].double().cpu().numpy()
        oracle.prefill_rows(None, k, v, rows, sink=sink, window=window,
                            rope_theta=wl["rope_theta"], rotary_fraction=wl["rotary_fraction"],
                            q_rows=qr)
        flops += float(np.minimum(rows + 1, window).sum()) * wl["hq"] * FLOP_PER_PAIR
        done += len(rows)
        if time.perf_counter() - t0 >= budget_s or done >= n:
            break
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} random query rows of {n} (all 64 heads), fp64 NumPy, {el:.1f} s; "
                      f"useful FLOPs of the sampled rows over wall time"}


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:  # noqa: BLE001
        return 1


def _oracle_entry(value, unit, seconds, sample, gpu_value):
    """One oracle baseline: the untuned oracle's rate on a sample of the
    workload, and the GPU's rate over it."""
    return {"value": value, "unit": unit, "cores": _oracle_threads(), "kind": "oracle",
            "seconds": seconds, "sample": sample,
            "gpu_over_oracle": (gpu_value / value) if value > 0 else None}


def _oracle_rows(run_rows, row_cost, n, budget_s, seed, chunk):
    """Random query rows, `chunk` at a time, until `budget_s` has passed:
    returns (useful work done, rows done, seconds)."""
    rng = np.random.default_rng(seed)
    order = rng.permutation(n)
    done, work, t0 = 0, 0.0, time.perf_counter()
    while done < n:
        rows = np.sort(order[done:done + chunk])
        run_rows(rows)
        work += row_cost(rows)
        done += len(rows)
        if time.perf_counter() - t0 >= budget_s:
            break
    return work, done, time.perf_counter() - t0


def copy_calibration(steps, warmup):
    """A plain device copy of known size: the reference for scaling the
    profiler's HBM byte counters (FETCH_SIZE / WRITE_SIZE)."""
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    _, per = timed(lambda: dst.copy_(src), steps, warmup)
    t = float(np.mean(per)) / 1e3
    return {"copy_bytes_each_way": nbytes, "gbps_read_plus_write": 2 * nbytes / t / 1e9,
            "us": t * 1e6}


def stream_bound(read_bytes, write_bytes, steps=10, warmup=2):
    """The rate at which the chip moves read_bytes in and write_bytes out
    with no arithmetic: hswa_stream_probe (16-byte coalesced accesses, each
    wavefront interleaving its reads and writes in proportion) at 4, 8, 16
    and 32 wavefronts per CU, the best median kept."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    src = torch.empty(read_bytes, dtype=torch.uint8, device="cuda") if read_bytes else None
    dst = torch.empty(write_bytes, dtype=torch.uint8, device="cuda") if write_bytes else None
    total = read_bytes + write_bytes
    by_shape, best = {}, None
    for per_cu in (1, 2, 4, 8):
        blocks = per_cu * cus
        o = torch.empty(4 * blocks, dtype=torch.int32, device="cuda")
        _, per = timed(lambda: hswa.stream_probe(src, dst, blocks, out=o), steps, warmup)
        t = float(np.median(per)) / 1e3
        by_shape[f"{4 * per_cu}_waves_per_cu"] = total / t / 1e9
        if best is None or t < best[0]:
            best = (t, 4 * per_cu)
    del src, dst
    return {"ms": best[0] * 1e3, "gbps": total / best[0] / 1e9, "waves_per_cu": best[1],
            "read_bytes": read_bytes, "write_bytes": write_bytes, "gbps_by_shape": by_shape}


def only(which, steps, warmup):
    if which == "copy":
        return {"copy": copy_calibration(steps, warmup)}
    parts = {"tiny": ["tiny"], "ga": ["ga"], "chunk": ["chunk"], "decode": ["decode"],
             "decode_ring": ["decode_ring"], "decode_ga": ["decode_ga"],
             "decode_mtp": ["decode_mtp"], "decode_fp8": ["decode_fp8"],
             "sparse": ["sparse"], "sparse_fp8": ["sparse_fp8"], "select": ["select"],
             "gather": ["gather"]}[which]
    return secondary(steps, warmup, parts, cpu=False)


def secondary(steps, warmup,
              parts=("tiny", "ga", "chunk", "decode", "decode_mtp", "decode_fp8", "sparse",
                     "gather", "sparse_fp8", "select"), cpu=True, cpu_seconds=4.0):
    out = {}
    dev = "cuda"
    budget = cpu_seconds if cpu else 0.0
    if "tiny" in parts:
        _tiny(out, steps, warmup, dev, budget)
    if "ga" in parts:
        _ga(out, steps, warmup, dev, budget)
    if "chunk" in parts:
        _chunk(out, steps, warmup, dev)
    if "decode" in parts or "decode_ring" in parts or "decode_ga" in parts:
        _decode(out, dev, budget, ring="decode_ga" not in parts, ga="decode_ring" not in parts)
    if "decode_mtp" in parts:
        _decode_mtp(out, dev)
    if "decode_fp8" in parts:
        _decode_fp8(out, dev)
    if "sparse" in parts:
        _sparse(out, dev, budget)
    if "gather" in parts:
        _gather(out, steps, dev)
    if "sparse_fp8" in parts:
        _sparse_fp8(out, dev)
    if "select" in parts:
        _select(out, dev)
    ga_decodes = [k for k in ("decode_ga_contiguous", "decode_mtp_ga_contiguous",
                              "decode_fp8_ga_contiguous") if k in out]
    if ga_decodes:
        # the rate the chip reads a large buffer at (no writes, no arithmetic):
        # the measured bound of the HBM-bound decode kernels
        rb = stream_bound(4 << 30, 0)
        for k in ga_decodes:
            out[k]["frac_of_stream_read_bound"] = out[k]["gbps"] / rb["gbps"]
            out[k]["stream_read_bound_gbps"] = rb["gbps"]
        _log(f"stream read bound {rb['gbps']:.0f} GB/s")
    return out


def measured_peaks(steps, warmup):
    """On-box reference rates next to the spec peaks: a large bf16 GEMM
    (hipBLASLt through torch.matmul; dense, no sparsity) and a plain device
    copy of 1 GiB."""
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    c = torch.empty(8192, 8192, device="cuda", dtype=torch.bfloat16)
    _, per = timed(lambda: torch.matmul(a, b, out=c), steps, warmup)
    t = float(np.median(per)) / 1e3
    gemm = 2 * 8192 ** 3 / t / 1e12
    del a, b, c
    copy = copy_calibration(steps, warmup)
    read_only = stream_bound(4 << 30, 0)
    return {"bf16_gemm_8192_tflops": gemm, "copy_1gib_gbps_read_plus_write": copy["gbps_read_plus_write"],
            "stream_probe_read_4gib_gbps": read_only["gbps"],
            "spec_bf16_tflops": BF16_PEAK_TFLOPS, "spec_hbm_gbps": HBM_PEAK_GBPS}


def _tiny(out, steps, warmup, dev, cpu_budget):
    # Tiny fp32 SWA+sink prefill: n = 512, 2 q / 1 kv heads, no RoPE, in its
    # four variants (sink on / -inf, W = 128 / W = n); launch-latency-bound
    wl = synthetic.WORKLOADS["tiny_fp32_swa_n512"]
    res = {}
    for window in (128, 512):
        for with_sink in (True, False):
            x = synthetic.prefill_inputs(1, wl["n"], wl["hq"], wl["hkv"], 192, 128, "f32",
                                         wl["seed"], dev, wl["sink_range"] if with_sink else None)
            o = torch.empty(1, wl["n"], wl["hq"], 128, dtype=torch.float32, device=dev)
            fn = lambda: hswa.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"],  # noqa: E731
                                               window=window, out=o)
            _, per = timed(fn, max(20, steps), warmup)
            t = float(np.median(per)) / 1e3
            flops = window_pairs(wl["n"], window) * wl["hq"] * FLOP_PER_PAIR
            key = f"W{window}_{'sink' if with_sink else 'nosink'}"
            res[key] = {"us_median": t * 1e6, "us_min": float(np.min(per)) * 1e3,
                        "tflops": flops / t / 1e12}
            if cpu_budget > 0 and window == 128 and with_sink:
                import oracle
                q, k, v = (x[n_].double().cpu().numpy() for n_ in "qkv")
                sk = x["sink"].double().cpu().numpy()
                t0 = time.perf_counter()
                oracle.swa_sink_prefill(q, k, v, sk, window=window)
                el = time.perf_counter() - t0
                res["oracle"] = _oracle_entry(flops / el / 1e9, "GFLOP/s", el,
                                              "the whole workload (512 rows, 2 heads, W = 128, "
                                              "sink), fp64 NumPy", flops / t / 1e9)
    res["note"] = "launch-latency-bound: parity only, no roofline claim"
    out["tiny_fp32_swa_n512"] = res
    _log(f"tiny {res}")


def _ga(out, steps, warmup, dev, cpu_budget=0.0):
    # GA prefill, n = 32768, 64 q / 4 kv heads, full causal
    wl = synthetic.WORKLOADS["ga_prefill_n32768"]
    x = synthetic.prefill_inputs(1, wl["n"], wl["hq"], wl["hkv"], 192, 128, "bf16", wl["seed"], dev,
                                 None)
    ws = torch.empty(hswa.prefill_workspace_size(1, wl["n"], wl["hkv"], 192, wl["rotary_fraction"]),
                     dtype=torch.uint8, device=dev)
    o = torch.empty(1, wl["n"], wl["hq"], 128, dtype=torch.bfloat16, device=dev)
    fn = lambda: hswa.ga_prefill(x["q"], x["k"], x["v"], rope_theta=wl["rope_theta"],  # noqa: E731
                                 rotary_fraction=wl["rotary_fraction"], out=o, workspace=ws)
    _, per = timed(fn, max(3, steps // 4), 1)
    flops = window_pairs(wl["n"], 0) * wl["hq"] * FLOP_PER_PAIR
    t = float(np.mean(per)) / 1e3
    out["ga_prefill_n32768"] = {"tflops": flops / t / 1e12, "ms": t * 1e3,
                                "ms_median": float(np.median(per)), "ms_min": float(np.min(per)),
                                "frac_of_bf16_peak": flops / t / 1e12 / BF16_PEAK_TFLOPS}
    if cpu_budget > 0:
        import oracle
        k = x["k"].double().cpu().numpy()
        v = x["v"].double().cpu().numpy()

        def run(rows):
            qr = x["q"][:, torch.from_numpy(rows).to(dev)].double().cpu().numpy()
            oracle.prefill_rows(None, k, v, rows, sink=None, window=None,
                                rope_theta=wl["rope_theta"], rotary_fraction=wl["rotary_fraction"],
                                q_rows=qr)
        work, done, el = _oracle_rows(run, lambda r: float((r + 1).sum()) * wl["hq"] * FLOP_PER_PAIR,
                                      wl["n"], cpu_budget, 8, 8)
        out["ga_prefill_n32768"]["oracle"] = _oracle_entry(
            work / el / 1e9, "GFLOP/s", el,
            f"{done} random query rows of {wl['n']} (all 64 heads), fp64 NumPy; useful FLOPs of "
            f"the sampled rows over wall time (extrapolated to the workload by FLOP rate)",
            flops / t / 1e9)
    _log(f"GA prefill {out['ga_prefill_n32768']}")


def _chunk(out, steps, warmup, dev):
    # Chunked prefill: one 16384-token chunk behind a cached prefix; the SWA
    # layer's cost does not depend on the prefix, the GA layer's grows with it
    for name in ("swa_chunk_q16384_prefix1048576", "ga_chunk_q16384_prefix114688"):
        wl = synthetic.WORKLOADS[name]
        res = {}
        for prefix in (0, wl["kv_len"] - wl["q_len"]):
            kv = prefix + wl["q_len"]
            x = synthetic.chunk_inputs(1, wl["q_len"], kv, wl["hq"], wl["hkv"], 192, 128, "bf16",
                                       wl["seed"], dev, wl["sink_range"])
            ws = torch.empty(hswa.prefill_workspace_size(1, kv, wl["hkv"], 192,
                                                         wl["rotary_fraction"]),
                             dtype=torch.uint8, device=dev)
            o = torch.empty(1, wl["q_len"], wl["hq"], 128, dtype=torch.bfloat16, device=dev)
            fn = lambda: hswa.swa_sink_prefill_chunk(  # noqa: E731
                x["q"], x["k"], x["v"], x["sink"], window=wl["window"],
                rope_theta=wl["rope_theta"], rotary_fraction=wl["rotary_fraction"], out=o,
                workspace=ws)
            # the same chunk over a cache of already-rotated keys (no key preparation)
            fc = lambda: hswa.swa_sink_prefill_chunk_cached(  # noqa: E731
                x["q"], x["k"], x["v"], x["sink"], window=wl["window"],
                rope_theta=wl["rope_theta"], rotary_fraction=wl["rotary_fraction"], out=o,
                workspace=ws)
            p = np.arange(prefix, kv, dtype=np.int64)
            pairs = int((np.minimum(p + 1, wl["window"]) if wl["window"] > 0 else p + 1).sum())
            flops = pairs * wl["hq"] * FLOP_PER_PAIR
            for key, f in ((f"prefix_{prefix}", fn), (f"prefix_{prefix}_cached_keys", fc)):
                _, per = timed(f, max(3, steps // 4), 1)
                t = float(np.median(per)) / 1e3
                res[key] = {"ms_median": t * 1e3, "tflops": flops / t / 1e12,
                            "tokens_per_s": wl["q_len"] / t}
            del x, ws, o
        lo, hi = res["prefix_0"], res[f"prefix_{wl['kv_len'] - wl['q_len']}"]
        res["tokens_per_s_ratio_long_vs_empty_prefix"] = hi["tokens_per_s"] / lo["tokens_per_s"]
        out[name] = res
        _log(f"{name} {res}")


def _decode(out, dev, cpu_budget=0.0, ring=True, ga=True):
    # Hybrid decode: 64 sequences at p ~ U[131072, 262143]
    wl = synthetic.WORKLOADS["hybrid_decode_b64"]
    pos = synthetic.decode_positions(wl["B"], *wl["pos_range"], wl["seed"])
    maxp = wl["pos_range"][1]
    sw, ga_cfg = wl["swa"], wl["ga"]
    if ring:
        # ring: rotate over 8 buffer sets (> 256 MB) so the cache is not served from the MALL
        sets = [synthetic.ring_decode_inputs(wl["B"], sw["hq"], sw["hkv"], sw["window"], 192, 128,
                                             "bf16", wl["seed"] + 100 * r, pos, dev,
                                             sw["sink_range"])
                for r in range(8)]
        wsr = torch.empty(hswa.decode_workspace_size(hswa.KV_RING, wl["B"], sw["hq"], 128,
                                                     sw["window"], maxp),
                          dtype=torch.uint8, device=dev)
        orr = torch.empty(wl["B"], sw["hq"], 128, dtype=torch.bfloat16, device=dev)
        it = [0]

        def ring_step():
            d = sets[it[0] % len(sets)]
            it[0] += 1
            hswa.swa_sink_decode(d["q"], d["k"], d["v"], d["pos"], maxp, layout=hswa.KV_RING,
                                 sink=d["sink"], window=sw["window"], out=orr, workspace=wsr)
        _, per = timed(ring_step, 40, 8)
        ring_bytes = (wl["B"] * sw["window"] * sw["hkv"] * (192 + 128) * 2 +
                      wl["B"] * sw["hq"] * (192 + 128) * 2)
        t = float(np.mean(per)) / 1e3
        tb = batched_us(ring_step) / 1e6
        out_bytes = wl["B"] * sw["hq"] * 128 * 2
        out["decode_swa_ring"] = {"gbps": ring_bytes / t / 1e9, "us": t * 1e6, "bytes": ring_bytes,
                                  "frac_of_hbm_peak": ring_bytes / t / 1e9 / HBM_PEAK_GBPS,
                                  "us_batched": tb * 1e6, "gbps_batched": ring_bytes / tb / 1e9,
                                  "graph": _graph_entry(ring_step, ring_bytes, ring_bytes, out_bytes),
                                  "note": "8 rotated buffer sets (353 MB) to defeat MALL residency; "
                                          "us: one event pair per call; us_batched: 200 calls "
                                          "between one event pair"}
        if cpu_budget > 0:
            import oracle
            d = sets[0]
            q, k, v = (d[n_].double().cpu().numpy() for n_ in "qkv")
            sk = d["sink"].double().cpu().numpy()
            t0 = time.perf_counter()
            oracle.swa_sink_decode_ring(q, k, v, pos.numpy(), sk)
            el = time.perf_counter() - t0
            out["decode_swa_ring"]["oracle"] = _oracle_entry(
                ring_bytes / el / 1e9, "GB/s", el,
                "the whole step (64 sequences, all heads), fp64 NumPy; algorithmic bytes over "
                "wall time", ring_bytes / t / 1e9)
        _log(f"decode ring {out['decode_swa_ring']}")
        del sets
    if not ga:
        return
    c = synthetic.contiguous_decode_inputs(wl["B"], ga_cfg["hq"], ga_cfg["hkv"], 192, 128, "bf16",
                                           wl["seed"], pos, dev, None)
    wsc = torch.empty(hswa.decode_workspace_size(hswa.KV_CONTIGUOUS, wl["B"], ga_cfg["hq"], 128, 0,
                                                 maxp),
                      dtype=torch.uint8, device=dev)
    oc = torch.empty(wl["B"], ga_cfg["hq"], 128, dtype=torch.bfloat16, device=dev)
    fn = lambda: hswa.swa_sink_decode(c["q"], c["k"], c["v"], c["pos"], maxp,  # noqa: E731
                                      layout=hswa.KV_CONTIGUOUS, seq_offsets=c["seq_offsets"],
                                      window=0, out=oc, workspace=wsc)
    _, per = timed(fn, 10, 2)
    keys = int((pos + 1).sum())
    ga_bytes = keys * ga_cfg["hkv"] * (192 + 128) * 2 + wl["B"] * ga_cfg["hq"] * (192 + 128) * 2
    t = float(np.mean(per)) / 1e3
    out["decode_ga_contiguous"] = {"gbps": ga_bytes / t / 1e9, "ms": t * 1e3, "bytes": ga_bytes,
                                   "frac_of_hbm_peak": ga_bytes / t / 1e9 / HBM_PEAK_GBPS}
    if cpu_budget > 0:
        import oracle
        offs = c["seq_offsets"].cpu().numpy()
        b = int(pos.argmin())   # the shortest sequence: 1 of the 64
        lo, hi = int(offs[b]), int(offs[b + 1])
        kb, vb = c["k"][lo:hi].double().cpu().numpy(), c["v"][lo:hi].double().cpu().numpy()
        q = c["q"].double().cpu().numpy()
        t0 = time.perf_counter()
        oracle.swa_sink_decode_contiguous(q, None, None, offs, pos.numpy(), None, None,
                                          seqs=np.array([b]), kv_loader=lambda _b: (kb, vb))
        el = time.perf_counter() - t0
        sb = (int(pos[b]) + 1) * ga_cfg["hkv"] * (192 + 128) * 2
        out["decode_ga_contiguous"]["oracle"] = _oracle_entry(
            sb / el / 1e9, "GB/s", el,
            f"1 of the 64 sequences (the shortest, {int(pos[b]) + 1} keys, all 64 heads), fp64 "
            f"NumPy; its algorithmic bytes over wall time", ga_bytes / t / 1e9)
    _log(f"decode GA {out['decode_ga_contiguous']}")


def _decode_mtp(out, dev):
    # MTP verification step: 64 sequences x 4 queries (last accepted token + 3 drafts)
    wl = synthetic.WORKLOADS["mtp_decode_b64_t4"]
    T = wl["T"]
    pos = synthetic.decode_positions(wl["B"], *wl["pos_range"], wl["seed"])
    maxp = wl["pos_range"][1] + T - 1
    sw, ga = wl["swa"], wl["ga"]
    sets = [synthetic.multi_ring_inputs(wl["B"], T, sw["hq"], sw["hkv"], sw["slots"], 192, 128,
                                        "bf16", wl["seed"] + 100 * r, pos, dev, sw["sink_range"])
            for r in range(8)]
    wsr = torch.empty(hswa.decode_multi_workspace_size(hswa.KV_RING, wl["B"], T, sw["hq"], 128,
                                                       sw["window"], sw["slots"], maxp),
                      dtype=torch.uint8, device=dev)
    orr = torch.empty(wl["B"], T, sw["hq"], 128, dtype=torch.bfloat16, device=dev)
    it = [0]

    def ring_step():
        d = sets[it[0] % len(sets)]
        it[0] += 1
        hswa.swa_sink_decode_multi(d["q"], d["k"], d["v"], d["pos"], maxp, layout=hswa.KV_RING,
                                   ring_slots=sw["slots"], sink=d["sink"], window=sw["window"],
                                   out=orr, workspace=wsr)
    _, per = timed(ring_step, 40, 8)
    ring_bytes = (wl["B"] * sw["slots"] * sw["hkv"] * (192 + 128) * 2 +
                  wl["B"] * T * sw["hq"] * (192 + 128) * 2)
    t = float(np.median(per)) / 1e3
    tb = batched_us(ring_step) / 1e6
    out["decode_mtp_swa_ring"] = {"gbps": ring_bytes / t / 1e9, "us": t * 1e6, "bytes": ring_bytes,
                                  "queries_per_s": wl["B"] * T / t, "us_batched": tb * 1e6,
                                  "gbps_batched": ring_bytes / tb / 1e9,
                                  "graph": _graph_entry(ring_step, ring_bytes, ring_bytes,
                                                        wl["B"] * T * sw["hq"] * 128 * 2)}
    _log(f"MTP decode ring {out['decode_mtp_swa_ring']}")
    del sets
    c = synthetic.multi_contiguous_inputs(wl["B"], T, ga["hq"], ga["hkv"], 192, 128, "bf16",
                                          wl["seed"], pos, dev, None)
    wsc = torch.empty(hswa.decode_multi_workspace_size(hswa.KV_CONTIGUOUS, wl["B"], T, ga["hq"],
                                                       128, 0, 0, maxp),
                      dtype=torch.uint8, device=dev)
    oc = torch.empty(wl["B"], T, ga["hq"], 128, dtype=torch.bfloat16, device=dev)
    fn = lambda: hswa.swa_sink_decode_multi(c["q"], c["k"], c["v"], c["pos"], maxp,  # noqa: E731
                                            layout=hswa.KV_CONTIGUOUS,
                                            seq_offsets=c["seq_offsets"], window=0, out=oc,
                                            workspace=wsc)
    _, per = timed(fn, 10, 2)
    keys = int((pos + T).sum())
    ga_bytes = keys * ga["hkv"] * (192 + 128) * 2 + wl["B"] * T * ga["hq"] * (192 + 128) * 2
    pairs = int(sum(int(p) + 1 + tt for p in pos for tt in range(T)))
    t = float(np.median(per)) / 1e3
    out["decode_mtp_ga_contiguous"] = {"gbps": ga_bytes / t / 1e9, "ms": t * 1e3, "bytes": ga_bytes,
                                       "frac_of_hbm_peak": ga_bytes / t / 1e9 / HBM_PEAK_GBPS,
                                       "tflops": pairs * ga["hq"] * FLOP_PER_PAIR / t / 1e12,
                                       "queries_per_s": wl["B"] * T / t}
    _log(f"MTP decode GA {out['decode_mtp_ga_contiguous']}")
    # the step's cache append: 64 sequences x 4 new tokens into the GA pool
    kn = synthetic.normal((wl["B"], T, ga["hkv"], 192), 17, dev, "bf16")
    vn = synthetic.normal((wl["B"], T, ga["hkv"], 128), 18, dev, "bf16")
    fa = lambda: hswa.kv_cache_append(kn, vn, c["k"], c["v"], c["pos"], maxp,  # noqa: E731
                                      layout=hswa.KV_CONTIGUOUS, seq_offsets=c["seq_offsets"],
                                      rope_theta=1.0e7, rotary_fraction=0.334)
    _, per = timed(fa, 20, 4)
    app_bytes = 2 * wl["B"] * T * ga["hkv"] * (192 + 128) * 2
    t = float(np.median(per)) / 1e3
    out["kv_append_mtp_ga"] = {"us": t * 1e6, "bytes": app_bytes, "gbps": app_bytes / t / 1e9,
                               "note": "latency-bound: 64 x 4 tokens, 655 KB read + written"}
    _log(f"append {out['kv_append_mtp_ga']}")


def _decode_fp8(out, dev):
    # The hybrid decode step over E4M3 caches (one byte per element)
    wl = synthetic.WORKLOADS["hybrid_decode_fp8_b64"]
    pos = synthetic.decode_positions(wl["B"], *wl["pos_range"], wl["seed"])
    maxp = wl["pos_range"][1]
    sw, ga = wl["swa"], wl["ga"]
    # ring: 16 buffer sets (336 MB) so that the caches are not served from the MALL
    sets = [synthetic.ring_decode_inputs_fp8(wl["B"], sw["hq"], sw["hkv"], sw["window"], 192, 128,
                                             wl["seed"] + 100 * r, pos, dev, sw["sink_range"],
                                             wl["scale_range"])
            for r in range(16)]
    wsr = torch.empty(hswa.decode_workspace_size(hswa.KV_RING, wl["B"], sw["hq"], 128, sw["window"],
                                                 maxp), dtype=torch.uint8, device=dev)
    orr = torch.empty(wl["B"], sw["hq"], 128, dtype=torch.bfloat16, device=dev)
    it = [0]

    def ring_step():
        d = sets[it[0] % len(sets)]
        it[0] += 1
        hswa.swa_sink_decode_fp8(d["q"], d["k"], d["v"], d["k_scale"], d["v_scale"], d["pos"], maxp,
                                 layout=hswa.KV_RING, sink=d["sink"], window=sw["window"], out=orr,
                                 workspace=wsr)
    _, per = timed(ring_step, 40, 8)
    ring_bytes = wl["B"] * sw["window"] * sw["hkv"] * (192 + 128) + wl["B"] * sw["hq"] * (192 + 128) * 2
    t = float(np.median(per)) / 1e3
    tb = batched_us(ring_step) / 1e6
    out["decode_fp8_swa_ring"] = {"gbps": ring_bytes / t / 1e9, "us": t * 1e6, "bytes": ring_bytes,
                                  "frac_of_hbm_peak": ring_bytes / t / 1e9 / HBM_PEAK_GBPS,
                                  "us_batched": tb * 1e6, "gbps_batched": ring_bytes / tb / 1e9,
                                  "graph": _graph_entry(ring_step, ring_bytes, ring_bytes,
                                                        wl["B"] * sw["hq"] * 128 * 2)}
    _log(f"decode fp8 ring {out['decode_fp8_swa_ring']}")
    del sets
    c = synthetic.contiguous_decode_inputs_fp8(wl["B"], ga["hq"], ga["hkv"], 192, 128, wl["seed"],
                                               pos, dev, None, scale_range=wl["scale_range"])
    wsc = torch.empty(hswa.decode_workspace_size(hswa.KV_CONTIGUOUS, wl["B"], ga["hq"], 128, 0, maxp),
                      dtype=torch.uint8, device=dev)
    oc = torch.empty(wl["B"], ga["hq"], 128, dtype=torch.bfloat16, device=dev)
    fn = lambda: hswa.swa_sink_decode_fp8(c["q"], c["k"], c["v"], c["k_scale"],  # noqa: E731
                                          c["v_scale"], c["pos"], maxp, layout=hswa.KV_CONTIGUOUS,
                                          seq_offsets=c["seq_offsets"], window=0, out=oc,
                                          workspace=wsc)
    _, per = timed(fn, 10, 2)
    keys = int((pos + 1).sum())
    ga_bytes = keys * ga["hkv"] * (192 + 128) + wl["B"] * ga["hq"] * (192 + 128) * 2
    t = float(np.median(per)) / 1e3
    out["decode_fp8_ga_contiguous"] = {"gbps": ga_bytes / t / 1e9, "ms": t * 1e3, "bytes": ga_bytes,
                                       "frac_of_hbm_peak": ga_bytes / t / 1e9 / HBM_PEAK_GBPS}
    _log(f"decode fp8 GA {out['decode_fp8_ga_contiguous']}")


def _sparse(out, dev, cpu_budget=0.0):
    # Sparse prefill, n = 65536, 128 recent + <= 1024 selected
    wl = synthetic.WORKLOADS["sparse_prefill_n65536"]
    x = synthetic.sparse_inputs(1, wl["n"], wl["hq"], wl["hkv"], 192, 128, "bf16", wl["seed"],
                                wl["recent"], wl["max_sel"], dev, wl["sink_range"])
    o = torch.empty(1, wl["n"], wl["hq"], 128, dtype=torch.bfloat16, device=dev)
    fn = lambda: hswa.sparse_sink_attn(x["q"], x["k"], x["v"], x["sel_idx"], x["sel_count"],  # noqa: E731
                                       x["sink"], recent_window=wl["recent"], out=o)
    _, per = timed(fn, 5, 1)
    i = np.arange(wl["n"])
    pairs = int((np.minimum(1024, np.maximum(0, i - 128)) + np.minimum(i + 1, 128)).sum()) * wl["hkv"]
    flops = pairs * (wl["hq"] // wl["hkv"]) * FLOP_PER_PAIR
    gathered = pairs * (192 + 128) * 2
    t = float(np.mean(per)) / 1e3
    out["sparse_prefill_n65536"] = {"tflops": flops / t / 1e12, "ms": t * 1e3,
                                    "gathered_kv_gbps": gathered / t / 1e9}
    # The bound of this kernel: its own gathers without its arithmetic.  The
    # probe reads each (query, kv head) list as the kernel does (selected
    # rows, then the recent window; 36 tiles of 32 rows, lists shorter than
    # 1152 padded with repeats of their last row) with the lists handed to
    # workgroups in the kernel's order (consecutive queries of a kv head on
    # one XCD).
    lists = _sparse_lists(x, wl, dev)
    tiles = (wl["max_sel"] + 128) // 32
    o = torch.empty(lists.shape[0] // (tiles * 32), dtype=torch.int32, device=dev)
    kf = x["k"].view(-1, 192)
    vf = x["v"].view(-1, 128)
    _, per = timed(lambda: hswa.gather_probe(kf, vf, lists, tiles, out=o), 5, 1)
    tp = float(np.median(per)) / 1e3
    out["sparse_prefill_n65536"]["gather_bound"] = {
        "probe_ms": tp * 1e3, "probe_gbps": gathered / tp / 1e9,
        "note": "hswa_gather_probe over the workload's own lists in the kernel's workgroup order"}
    out["sparse_prefill_n65536"]["frac_of_measured_gather_peak"] = tp / t
    del lists, o
    if cpu_budget > 0:
        import oracle
        k = x["k"].double().cpu().numpy()
        v = x["v"].double().cpu().numpy()
        sk = x["sink"].double().cpu().numpy()
        G = wl["hq"] // wl["hkv"]

        def run(rows):
            ri = torch.from_numpy(rows).to(dev)
            oracle.sparse_rows(x["q"][:, ri].double().cpu().numpy(), k, v,
                               x["sel_idx"][:, ri].cpu().numpy(), x["sel_count"][:, ri].cpu().numpy(),
                               rows, sk, recent=wl["recent"], restricted=True)

        def cost(rows):
            return float((np.minimum(1024, np.maximum(0, rows - 128)) +
                          np.minimum(rows + 1, 128)).sum()) * wl["hkv"] * G * FLOP_PER_PAIR
        work, done, el = _oracle_rows(run, cost, wl["n"], cpu_budget, 9, 64)
        out["sparse_prefill_n65536"]["oracle"] = _oracle_entry(
            work / el / 1e9, "GFLOP/s", el,
            f"{done} random query rows of {wl['n']} (all 64 heads), fp64 NumPy; useful FLOPs of "
            f"the sampled rows over wall time (extrapolated to the workload by FLOP rate)",
            flops / t / 1e9)
    _log(f"sparse {out['sparse_prefill_n65536']}")


def _sparse_lists(x, wl, dev):
    """Row numbers (token * hkv + g) of every (query, kv head) list of the
    sparse workload (max_sel + 128 entries, padded with repeats of the
    list's last row), lists in the order the sparse kernel's workgroups take
    them: physical workgroup b serves logical list xcd_remap(b) = (g, i) with
    logical index g * n + i."""
    n, hkv = wl["n"], wl["hkv"]
    sel = x["sel_idx"][0].long()                                  # [n, hkv, ms], -1 padded
    cnt = x["sel_count"][0].long()                                # [n, hkv]
    ms = sel.shape[-1]
    width = ms + 128
    i = torch.arange(n, device=dev)
    rec = (i[:, None] - 127 + torch.arange(128, device=dev)[None, :])   # [n, 128]
    full = torch.cat([sel, rec[:, None, :].expand(n, hkv, 128)], dim=2)  # [n, hkv, width]
    # entry t of a list is sel[t] for t < cnt, else the recent window's t - cnt
    t = torch.arange(width, device=dev)[None, None, :]
    src = torch.where(t < cnt[..., None], t, ms + (t - cnt[..., None]))
    lst = torch.gather(full, 2, src.clamp(max=width - 1))
    rec_len = torch.minimum(i + 1, torch.tensor(128, device=dev))
    length = cnt + rec_len[:, None]                                # [n, hkv]
    # the recent window of query i starts at max(0, i - 127)
    first_rec = (i - 127).clamp(min=0)[:, None, None]
    lst = torch.where((t >= cnt[..., None]) & (t < length[..., None]),
                      first_rec + (t - cnt[..., None]), lst)
    last = torch.gather(lst, 2, (length - 1).clamp(min=0)[..., None])
    lst = torch.where(t < length[..., None], lst, last).clamp(min=0)
    rows = lst * hkv + torch.arange(hkv, device=dev)[None, :, None]              # [n, hkv, width]
    logical = rows.permute(1, 0, 2).reshape(hkv * n, width)                       # index g * n + i
    nwg = hkv * n
    b = torch.arange(nwg, device=dev)
    q, rem = nwg >> 3, nwg & 7
    xx, slot = b & 7, b >> 3
    lg = torch.where(xx < rem, xx * (q + 1) + slot, rem * (q + 1) + (xx - rem) * q + slot)
    return logical[lg].reshape(-1).to(torch.int32).contiguous()


def _gather(out, steps, dev):
    # Random-row gather bandwidth with the sparse kernel's access pattern:
    # K rows of 384 B and V rows of 256 B picked uniformly from the sparse
    # workload's cache (65536 tokens x 4 kv heads: 168 MB, resident in the
    # 256 MB last-level cache) and from a cache 16 times larger (2.7 GB, so
    # nearly every row comes from HBM); 36 tiles of 32 rows per wavefront,
    # 32768 wavefronts (37.7 M rows, 24.2 GB per call).
    wl = synthetic.WORKLOADS["sparse_prefill_n65536"]
    nwaves, tiles = 32768, 36
    res = {}
    for label, mult in (("cache_168MB", 1), ("cache_2.7GB", 16)):
        rows = wl["n"] * wl["hkv"] * mult
        k = synthetic.normal((rows, 192), 31, dev, "bf16")
        v = synthetic.normal((rows, 128), 32, dev, "bf16")
        g = torch.Generator(device=dev)
        g.manual_seed(33)
        idx = torch.randint(0, rows, (nwaves * tiles * 32,), generator=g, device=dev,
                            dtype=torch.int32)
        o = torch.empty(nwaves, dtype=torch.int32, device=dev)
        fn = lambda: hswa.gather_probe(k, v, idx, tiles, out=o)  # noqa: E731
        _, per = timed(fn, max(5, steps // 10), 1)
        t = float(np.median(per)) / 1e3
        nbytes = nwaves * tiles * 32 * (192 + 128) * 2
        res[label] = {"gbps": nbytes / t / 1e9, "us": t * 1e6, "bytes": nbytes,
                      "cache_bytes": rows * (192 + 128) * 2}
        del k, v, idx, o
    res["note"] = ("hswa_gather_probe: the sparse kernel's loads (16-byte pieces, 32-row tiles, one "
                   "wavefront per list) of uniformly random rows, no arithmetic")
    out["gather_probe"] = res
    _log(f"gather {res}")


def _sparse_fp8(out, dev):
    # The sparse workload over E4M3 K/V (one byte per gathered element)
    wl = synthetic.WORKLOADS["sparse_prefill_n65536"]
    x = synthetic.sparse_inputs_fp8(1, wl["n"], wl["hq"], wl["hkv"], 192, 128, wl["seed"],
                                    wl["recent"], wl["max_sel"], dev, wl["sink_range"])
    o = torch.empty(1, wl["n"], wl["hq"], 128, dtype=torch.bfloat16, device=dev)
    fn = lambda: hswa.sparse_sink_attn_fp8(x["q"], x["k"], x["v"], x["k_scale"],  # noqa: E731
                                           x["v_scale"], x["sel_idx"], x["sel_count"], x["sink"],
                                           recent_window=wl["recent"], out=o)
    _, per = timed(fn, 5, 1)
    i = np.arange(wl["n"])
    pairs = int((np.minimum(1024, np.maximum(0, i - 128)) + np.minimum(i + 1, 128)).sum()) * wl["hkv"]
    flops = pairs * (wl["hq"] // wl["hkv"]) * FLOP_PER_PAIR
    gathered = pairs * (192 + 128)
    t = float(np.median(per)) / 1e3
    out["sparse_fp8_prefill_n65536"] = {"tflops": flops / t / 1e12, "ms": t * 1e3,
                                        "gathered_kv_gbps": gathered / t / 1e9}
    _log(f"sparse fp8 {out['sparse_fp8_prefill_n65536']}")


def _select(out, dev):
    # Token selection for the sparse workload: n = 65536, 64 q / 4 kv heads,
    # the top 1024 of the candidates outside the 128 recent tokens
    wl = synthetic.WORKLOADS["sparse_prefill_n65536"]
    x = synthetic.prefill_inputs(1, wl["n"], wl["hq"], wl["hkv"], 192, 128, "bf16", wl["seed"], dev,
                                 None)
    idx = torch.empty((1, wl["n"], wl["hkv"], wl["max_sel"]), dtype=torch.int32, device=dev)
    cnt = torch.empty((1, wl["n"], wl["hkv"]), dtype=torch.int32, device=dev)
    fn = lambda: hswa.sparse_select_tokens(x["q"], x["k"], max_sel=wl["max_sel"],  # noqa: E731
                                           recent_window=wl["recent"], out=(idx, cnt))
    _, per = timed(fn, 3, 1)
    t = float(np.median(per)) / 1e3
    i = np.arange(wl["n"], dtype=np.int64)
    causal = int((i + 1).sum())
    cand = int(np.maximum(0, i - wl["recent"] + 1).sum())
    # two passes of score products: log-sum-exp over keys 0 .. i (its own
    # kernel), then the importances of the candidates (read back once)
    flops = (causal + cand) * wl["hq"] * 2 * 192
    out["select_tokens_n65536"] = {"ms": t * 1e3, "qk_tflops": flops / t / 1e12,
                                   "rows_per_s": wl["n"] * wl["hkv"] / t,
                                   "frac_of_bf16_peak": flops / t / 1e12 / BF16_PEAK_TFLOPS}
    _log(f"select {out['select_tokens_n65536']}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replayed decode timings (for profiler runs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", choices=["prefill", "tiny", "ga", "chunk", "decode", "decode_ring",
                                       "decode_ga", "decode_mtp", "decode_fp8", "sparse", "gather",
                                       "sparse_fp8", "select", "copy"], default=None,
                    help="run one workload only (for profiler runs); prints its figures as JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU: this build has no multi-GPU path "
              "(the sharding plan is design only).", file=sys.stderr)
        sys.exit(2)
    _ensure_built()
    global GRAPH_TIMING
    GRAPH_TIMING = not args.no_graph
    dev = "cuda"
    if args.only and args.only != "prefill":
        print(json.dumps(only(args.only, args.steps, args.warmup)), flush=True)
        return
    wl = synthetic.WORKLOADS["swa_prefill_n32768"]
    x = synthetic.prefill_inputs(1, wl["n"], wl["hq"], wl["hkv"], 192, 128, "bf16", wl["seed"], dev,
                                 wl["sink_range"])
    o = torch.empty(1, wl["n"], wl["hq"], 128, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(hswa.prefill_workspace_size(1, wl["n"], wl["hkv"], 192, wl["rotary_fraction"]),
                     dtype=torch.uint8, device=dev)

    def step():
        hswa.swa_sink_prefill(x["q"], x["k"], x["v"], x["sink"], window=wl["window"],
                              rope_theta=wl["rope_theta"], rotary_fraction=wl["rotary_fraction"],
                              out=o, workspace=ws)

    torch.cuda.synchronize()
    wall, per = timed(step, args.steps, args.warmup)
    ms_step = wall * 1e3 / args.steps
    flops = window_pairs(wl["n"], wl["window"]) * wl["hq"] * FLOP_PER_PAIR
    value = flops * args.steps / wall / 1e12
    n, hq, hkv = wl["n"], wl["hq"], wl["hkv"]
    alg_bytes = n * (hq * 192 + hkv * 192 + hkv * 128 + hq * 128) * 2
    kern_s = float(np.mean(per)) / 1e3
    achieved = alg_bytes / kern_s / 1e9
    _log(f"prefill: {ms_step:.3f} ms/step wall, {kern_s * 1e3:.3f} ms/launch (events), "
         f"{value:.1f} TFLOP/s, {achieved:.0f} GB/s")

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "swa_prefill_n32768", "batch": 1, "seq_len": n, "hq": hq,
                   "hkv": hkv, "d_qk": 192, "d_v": 128, "window": wl["window"],
                   "rope_theta": wl["rope_theta"], "rotary_fraction": wl["rotary_fraction"],
                   "sink": "U(-2,2) per head", "useful_gflop_per_step": flops / 1e9},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": _traffic("prefill_seq_kernel:swa_prefill_n32768"),
                     "kernel": "prefill_seq_kernel",
                     "launch_scope": "one swa_sink_prefill call (one kernel: q and K rotated inside it)",
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "launch_ms": kern_s * 1e3,
                     "launch_ms_median": float(np.median(per)),
                     "launch_ms_min": float(np.min(per)),
                     "frac_of_bf16_mfma_peak": value / BF16_PEAK_TFLOPS},
    }
    # the same bytes moved with no arithmetic: the rate this traffic mix allows
    out_bytes = n * hq * 128 * 2
    sb = stream_bound(alg_bytes - out_bytes, out_bytes)
    sb["frac"] = sb["ms"] / (kern_s * 1e3)
    sb["note"] = ("hswa_stream_probe moving the call's algorithmic read and write bytes; frac = "
                  "probe time / prefill call time")
    rec["roofline"]["measured_stream_bound"] = sb
    _log(f"stream bound {sb}")
    if args.only:
        print(json.dumps(rec), flush=True)
        return
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(x, wl, args.cpu_seconds)
        _log(f"cpu baseline {rec['cpu_baseline']}")
    del x, o, ws
    torch.cuda.empty_cache()
    if not args.no_secondary:
        rec["secondary"] = secondary(args.steps, args.warmup, cpu=not args.no_cpu)
        rec["measured_peaks"] = measured_peaks(args.steps, args.warmup)
        _log(f"measured peaks {rec['measured_peaks']}")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
