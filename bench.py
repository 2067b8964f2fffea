"""Throughput of the block-scaled microscaling hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  * the large MoE-expert sweep, bfloat16 [256, 2048, 7168] (about 3.8 G
    parameters, with 0.1% all-zero, bf16-subnormal and +-1e4-spike 32-column
    blocks), processed in 36-expert chunks of about 1 GiB: MXFP4 quantize-pack,
    MXFP4 dequantize to bf16, NVFP4 quantize-pack (per-row scale), NVFP4
    dequantize to bf16, chunk by chunk;
  * the cache quantize/dequantize round trip on KV-cache-shaped bf16 tensors:
    fp8 block 32 [16, 8192, 512], mxfp4 block 32 [16, 8192, 128], nvfp4 block
    16 [16, 2048, 512].
`value` is effective GB/s: algorithmic bytes (every input read once plus every
output written once) of the whole step divided by the step's wall time.  The
timed steps replay the step's launches captured once as a HIP graph (the same
kernels with the same arguments, without host launch gaps between them);
`--eager` times eager launches instead, and `eager_GBps` always reports them.

Prints one JSON line.  Also reports, per operation, its average launch
duration from a HIP graph of its launches replayed back to back (the sweep's
eight chunk launches; eight rotating buffer sets for the cache round trips, so
that no launch finds its input in the 256 MB last-level cache), timed with HIP
events on the launch stream; the roofline of the dominant kernel against
MI355X's 8 TB/s HBM peak and against a plain copy of the same size (the
practical ceiling, from the reference kernels of libmxq_roofline); and the CPU
oracle timed on a bounded sample of the same workload, on one thread and on all
the host's threads.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
CALIBRATION_BYTES = 36 * 2048 * 7168 * 2
METRIC = "effective GB/s (in+out) for FP4 quant-pack & dequant; % of MI355X HBM peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU-oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--experts", type=int, default=256,
                    help="experts of the sweep (256 is the full workload)")
    ap.add_argument("--no-gemm", action="store_true",
                    help="skip the grouped-GEMM measurement (not part of `value`)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the MXFP8 / static FP4 / KV-cache measurements (not part of `value`)")
    ap.add_argument("--eager", action="store_true",
                    help="time the steps as eager launches instead of HIP graph replays")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run the reference copy kernel over one 36-expert "
                         "chunk (reads and writes CALIBRATION_BYTES) for HBM counter calibration")
    ap.add_argument("--no-ref", action="store_true",
                    help="skip the copy / read / write reference kernels")
    ap.add_argument("--by-predecessor", action="store_true",
                    help="also time the dominant operation's graph straight after each sweep "
                         "operation's graph (roofline.avg_launch_us_after); off by default, so "
                         "that a kernel trace of the default run holds the step's launches and "
                         "the per-operation graphs only")
    return ap.parse_args()


def bytes_mx(n_elem: int) -> int:
    # bf16 in (2 B) + packed (1/2 B) + one e8m0 byte per 32
    return 2 * n_elem + n_elem // 2 + n_elem // 32


def bytes_nv(n_elem: int, rows: int) -> int:
    # bf16 in + packed + one e4m3 byte per 16 + one float32 per row
    return 2 * n_elem + n_elem // 2 + n_elem // 16 + 4 * rows


def measured_traffic(kernel: str, src_hash: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"^source_hash:\s*(\S+)", txt, re.M)
    if not m or m.group(1) != src_hash:
        return None
    m = re.search(rf"^{re.escape(kernel)}\s+traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt, re.M)
    return float(m.group(1)) if m else None


def progress(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_quantize_pack_amd as mxq
    from fp8_quantize_pack_amd.profiling import kernel_source_hash
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---------------- inputs (generated once, resident in HBM) ----------------
    E, N, K = synth.SHAPES["c5"]
    E = args.experts
    chunks = synth.c5_chunks(E)
    x = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
    for cid, e0, ne in chunks:
        x[e0:e0 + ne] = synth.c5_chunk(cid, ne, device=dev)
    mx_p = torch.empty((E, N, K // 2), dtype=torch.int8, device=dev)
    mx_s = torch.empty((E, N, K // 32), dtype=torch.uint8, device=dev)
    nv_p = torch.empty((E, N, K // 2), dtype=torch.uint8, device=dev)
    nv_s = torch.empty((E, N, K // 16), dtype=torch.uint8, device=dev)
    nv_g = torch.empty((E, N), dtype=torch.float32, device=dev)
    y = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
    cache_cases = [("c4a", "fp8", 32), ("c4b", "mxfp4", 32), ("c4c", "nvfp4", 16)]
    cache_in = {c: synth.kv_cache(synth.SHAPES[c], seed=synth.SEEDS[c], device=dev) for c, _, _ in cache_cases}
    cache_out = {c: torch.empty_like(v) for c, v in cache_in.items()}
    torch.cuda.synchronize()
    progress("inputs resident:", E, "experts")

    # ---------------- one step: list of (op name, bytes, callable) ----------------
    plan = []
    for cid, e0, ne in chunks:
        sl = slice(e0, e0 + ne)
        n = ne * N * K
        xs, ys = x[sl], y[sl]
        mp, ms, np_, ns, ng = mx_p[sl], mx_s[sl], nv_p[sl], nv_s[sl], nv_g[sl]
        plan.append(("mxfp4_quant", bytes_mx(n), lambda xs=xs, mp=mp, ms=ms: mxq.mxq_quantize_mxfp4(xs, mp, ms)))
        plan.append(("mxfp4_dequant", bytes_mx(n), lambda mp=mp, ms=ms, ys=ys: mxq.mxq_dequantize_mxfp4(mp, ms, ys)))
        plan.append(("nvfp4_quant", bytes_nv(n, ne * N),
                     lambda xs=xs, np_=np_, ns=ns, ng=ng: mxq.mxq_quantize_nvfp4(xs, np_, ns, ng)))
        plan.append(("nvfp4_dequant", bytes_nv(n, ne * N),
                     lambda np_=np_, ns=ns, ng=ng, ys=ys: mxq.mxq_dequantize_nvfp4(np_, ns, ng, ys)))
    for c, fmt, B in cache_cases:
        xi, yo = cache_in[c], cache_out[c]
        plan.append((f"cache_{fmt}", 4 * xi.numel(),
                     lambda xi=xi, yo=yo, fmt=fmt, B=B: mxq.mxq_quantize_cache(xi, yo, fmt, B)))
    step_bytes = sum(b for _, b, _ in plan)

    def run_step(events=None):
        for i, (_, _, fn) in enumerate(plan):
            if events is not None:
                events[i][0].record(stream)
            fn()
            if events is not None:
                events[i][1].record(stream)

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # per-launch durations: K eager steps with HIP events around every launch
    # (on the stream the kernels run on)
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in plan] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        run_step(ev[s])
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t0
    progress(f"{args.steps} eager steps with per-launch events: {eager_wall:.3f} s")

    # the step as one HIP graph: the same launches with the same arguments,
    # replayed without host launch gaps between them
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_step()
        graph.replay()
        torch.cuda.synchronize()

    # timed region: exactly K steps, synchronized on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            run_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    progress(f"{args.steps} timed steps ({'graph replays' if graph is not None else 'eager'}): {wall:.3f} s")

    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (wall / args.steps) / 1e9

    # per-launch durations from HIP event pairs around every eager launch
    ev_ops = {}
    for st in range(args.steps):
        for i, (name, b, _) in enumerate(plan):
            o = ev_ops.setdefault(name, [0, 0.0])
            o[0] += 1
            o[1] += ev[st][i][0].elapsed_time(ev[st][i][1])

    # per-operation durations from graphs of back-to-back launches: the
    # sweep's chunk launches of one operation, or the cache round trip over
    # CACHE_SETS rotating buffer sets (the sets of one case together exceed
    # the 256 MB last-level cache, so every launch reads cold input, as in the
    # step, where 7 GB of sweep traffic runs between two uses)
    cache_sets = {c: [(cache_in[c], cache_out[c])] + [
        (synth.kv_cache(synth.SHAPES[c], seed=synth.SEEDS[c] * 100 + i, device=dev),
         torch.empty_like(cache_in[c])) for i in range(1, CACHE_SETS)] for c, _, _ in cache_cases}
    op_launches = {}
    for name, b, fn in plan:
        if not name.startswith("cache"):
            op_launches.setdefault(name, []).append((b, fn))
    for c, fmt, B in cache_cases:
        op_launches[f"cache_{fmt}"] = [
            (4 * xi.numel(), lambda xi=xi, yo=yo, fmt=fmt, B=B: mxq.mxq_quantize_cache(xi, yo, fmt, B))
            for _ in range(CACHE_CYCLES) for xi, yo in cache_sets[c]]
    reps = max(args.steps, 5)
    ops = {}
    op_graphs = capture_graphs(torch, {n: [fn for _, fn in l] for n, l in op_launches.items()})
    op_times = time_graphs_interleaved(torch, op_graphs, reps)
    for name, launches in op_launches.items():
        t = op_times[name]
        nb = sum(b for b, _ in launches)
        n_ev, ms_ev = ev_ops[name]
        per_step_launches = sum(1 for n, _, _ in plan if n == name)
        ops[name] = {"launches_per_graph": len(launches), "graph_replays": reps,
                     "bytes_per_launch": nb // len(launches),
                     "avg_launch_us": round(t / len(launches) * 1e6, 2),
                     "GBps": round(nb / t / 1e9, 1), "frac_of_peak": round(nb / t / 1e9 / PEAK_HBM_GBPS, 4),
                     "event_pair_avg_us": round(ms_ev * 1e3 / n_ev, 2),
                     "step_us": round(t / len(launches) * per_step_launches * 1e6, 1)}
    fp4 = [n for n in ops if not n.startswith("cache")]
    fp4_bytes = sum(b for n, b, _ in plan if n in fp4)
    fp4_s = sum(ops[n]["step_us"] for n in fp4) * 1e-6
    dom = max(ops, key=lambda n: ops[n]["step_us"])
    # on request, the dominant operation's launch time straight after each
    # sweep operation (it depends on the predecessor), and the shader clock
    # read right after each of them
    by_pred = None
    if args.by_predecessor:
        after = time_after(torch, op_graphs, dom, fp4, reps)
        by_pred = {p: round(t / len(op_launches[dom]) * 1e6, 2) for p, t in after.items()}
        clock_after = shader_clock_after(torch, op_graphs, fp4, reps, dev)
    del op_graphs, cache_sets
    progress("per-operation graphs timed")
    src_hash = kernel_source_hash()
    traffic = measured_traffic(dom, src_hash)

    ref = None if args.no_ref else reference_rates(torch, dev, x, y, reps)
    progress("reference copy / read / write measured" if ref else "reference kernels skipped")
    achieved = ops[dom]["GBps"]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": traffic,
                "algorithmic_bytes_per_launch": ops[dom]["bytes_per_launch"],
                "avg_launch_us": ops[dom]["avg_launch_us"]}
    if by_pred is not None:
        roofline["avg_launch_us_after"] = by_pred
        roofline["shader_clock_MHz_after"] = clock_after
    if ref:
        cp = ref["copy"]["sweep_chunk"]
        roofline["copy_GBps"] = cp["GBps"]
        roofline["copy_bytes_per_launch"] = cp["bytes_per_launch"]
        roofline["frac_of_copy"] = round(achieved / cp["GBps"], 4)
        for n, o in ops.items():
            size = "sweep_chunk" if not n.startswith("cache") else (
                "cache_256MiB" if n == "cache_fp8" else "cache_64MiB")
            o["frac_of_same_size_copy"] = round(o["GBps"] / ref["copy"][size]["GBps"], 4)

    gemm = None if args.no_gemm else grouped_gemm(torch, mxq, dev, max(args.steps, 1))
    progress("grouped GEMM measured" if gemm else "grouped GEMM skipped")
    extra = None if args.no_extra else extra_ops(torch, mxq, synth, dev, x, y, max(args.steps, 1),
                                                 (mx_p, mx_s, nv_p, nv_s, nv_g))
    progress("extra ops measured" if extra else "extra ops skipped")

    if args.calibrate_copy:
        # a plain copy kernel of known traffic, outside the timed region
        from fp8_quantize_pack_amd import roofline as rl
        xs, ys = x[:synth.C5_CHUNK_EXPERTS], y[:synth.C5_CHUNK_EXPERTS]
        assert xs.numel() * xs.element_size() == CALIBRATION_BYTES
        for _ in range(3):
            rl.copy(xs, ys, unroll=2)
        torch.cuda.synchronize()

    # ---------------- CPU baseline: the oracle on a bounded sample ----------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, args.cpu_seconds)
        progress("CPU oracle baseline measured")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "MoE expert sweep bf16 [%d,2048,7168] in 36-expert chunks: MXFP4 + NVFP4 "
                               "quantize-pack and dequantize to bf16; plus cache QDQ fp8/b32 [16,8192,512], "
                               "mxfp4/b32 [16,8192,128], nvfp4/b16 [16,2048,512]" % E,
                   "parallelism": "single GPU", "chunks": len(chunks), "step_bytes": step_bytes,
                   "launch": "eager" if graph is None else "hip_graph (one step captured, replayed K times)"},
        "eager_GBps": round(step_bytes * args.steps / eager_wall / 1e9, 1),
        "frac_of_peak": round(value / PEAK_HBM_GBPS, 4),
        "fp4_sweep_GBps": round(fp4_bytes / fp4_s / 1e9, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "reference_kernels": ref,
        "grouped_gemm": gemm,
        "extra_ops": extra,
        "ops": ops,
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(out), flush=True)


CACHE_SETS = 8
CACHE_CYCLES = 4     # passes over the rotating sets in one timed graph


def capture_graphs(torch, fns_by_name):
    """Each list of launches captured once as a HIP graph (after one eager
    pass) and replayed once."""
    graphs = {}
    for name, fns in fns_by_name.items():
        for f in fns:
            f()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in fns:
                f()
        g.replay()
        graphs[name] = g
    torch.cuda.synchronize()
    return graphs


def time_graphs_interleaved(torch, graphs, reps):
    """Seconds for one replay of each graph: the graphs are replayed in turn,
    `reps` rounds, each replay between two HIP events on the launch stream (so
    every operation is timed among the others, as in the step, rather than
    after a long run of itself); the mean over the rounds."""
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)] for n in graphs}
    for r in range(reps):
        for n, g in graphs.items():
            ev[n][r][0].record()
            g.replay()
            ev[n][r][1].record()
    torch.cuda.synchronize()
    return {n: sum(a.elapsed_time(b) for a, b in ev[n]) * 1e-3 / reps for n in graphs}


def time_after(torch, graphs, target, preds, reps):
    """Seconds for one replay of graphs[target] started straight after a
    replay of graphs[p], for each p in preds (no synchronization in between;
    `reps` pairs each, the mean)."""
    out = {}
    for p in preds:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            graphs[p].replay()
            a.record()
            graphs[target].replay()
            b.record()
        torch.cuda.synchronize()
        out[p] = sum(a.elapsed_time(b) for a, b in ev) * 1e-3 / reps
    return out


def shader_clock_after(torch, graphs, preds, reps, dev):
    """Mean shader clock (MHz) read by the clock probe of libmxq_roofline
    launched straight after a replay of graphs[p], for each p in preds
    (`reps` pairs each)."""
    from fp8_quantize_pack_amd import roofline as rl
    out = torch.zeros(2 * 256, dtype=torch.int64, device=dev)
    res = {}
    for p in preds:
        vals = []
        for _ in range(reps):
            graphs[p].replay()
            rl.clock(out, iters=4096)
            torch.cuda.synchronize()
            vals.append(rl.clock_mhz(out))
        res[p] = round(sum(vals) / len(vals), 1)
    return res


def time_graph(torch, fns, reps):
    """Seconds for one pass over `fns` (kernel launches on the current
    stream), captured once as a HIP graph and replayed `reps` times back to
    back between two HIP events on that stream."""
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) * 1e-3 / reps
    del g
    return t


def reference_rates(torch, dev, x, y, reps):
    """The practical HBM ceiling: the plain copy, read-only and write-only
    reference kernels (libmxq_roofline; same 16-byte non-temporal accesses and
    wave tiles as the codec kernels, no arithmetic), each at the best of
    unroll 1, 2 and 4, timed as graphs of back-to-back launches.  Sizes: one
    sweep chunk (1.06 GB read + 1.06 GB written for the copy), and copies
    that move 256 MiB and 64 MiB (the cache round trips' sizes) over eight
    rotating sets, so that none is served from the last-level cache.  The
    buffers are disjoint slices of the sweep's input and output tensors."""
    from fp8_quantize_pack_amd import roofline as rl
    xb, yb = x.view(-1).view(torch.uint8), y.view(-1).view(torch.uint8)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {"copy": {}, "read": {}, "write": {}}

    def best(kind, name, moved, fns_for):
        res = None
        for u in (1, 2, 4):
            fns = fns_for(u)
            t = time_graph(torch, fns, reps) / len(fns)
            r = {"bytes_per_launch": moved, "avg_launch_us": round(t * 1e6, 2),
                 "GBps": round(moved / t / 1e9, 1), "unroll": u}
            if res is None or r["GBps"] > res["GBps"]:
                res = r
        res["frac_of_peak"] = round(res["GBps"] / PEAK_HBM_GBPS, 4)
        out[kind][name] = res

    n = CALIBRATION_BYTES
    best("copy", "sweep_chunk", 2 * n, lambda u: [lambda: rl.copy(xb[:n], yb[:n], u)])
    for name, half in (("cache_256MiB", 128 << 20), ("cache_64MiB", 32 << 20)):
        sets = [(xb[i * half:(i + 1) * half], yb[i * half:(i + 1) * half]) for i in range(CACHE_SETS)]
        best("copy", name, 2 * half,
             lambda u, sets=sets: [lambda s=s, d=d: rl.copy(s, d, u) for s, d in sets])
    best("read", "sweep_chunk", n, lambda u: [lambda: rl.read(xb[:n], sink, u)])
    best("write", "sweep_chunk", n, lambda u: [lambda: rl.fill(yb[:n], 0, u)])
    return out


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def grouped_gemm(torch, mxq, dev, reps):
    """The consumer of the codec: grouped GEMMs over packed expert weights,
    dequantized on the fly, forward (x @ W_e^T) and backward (x @ W_e), on the
    per-expert shapes of the MXFP4 MoE config (32 x [4096, 2048], 512 tokens
    per expert) and the NVFP4 gate/up config (64 x [3072, 4096], 256 tokens
    per expert); synthetic random codes and scales.  Timed with HIP events
    around `reps` launches each; not part of `value`.  For context each entry
    also times torch.bmm on the same per-expert products with dense bfloat16
    weights (the vendor BLAS, nothing to dequantize): a practical MFMA rate
    for these shapes, not a result of this library; and the pages' own
    unfused design: this library's dequantization of every expert's weights
    to bfloat16 [E, N, K], then that dense product.  In the backward product
    (x @ W_e) the dequantized tensor is the right operand as it is.  The
    forward product (x @ W_e^T) would read it through a transposed view,
    which torch's bfloat16 bmm has faulted on with this software stack, so the
    composition there multiplies by the same buffer viewed as [E, K, N]: the
    same GEMM shape and bytes on a contiguous operand, timed for cost only."""
    g = torch.Generator(device=dev).manual_seed(11)
    out = {"peak_TFLOPs": PEAK_BF16_TFLOPS, "bound": "mfma", "dtype": "bf16"}
    for fmt, E, N, K, per in (("mxfp4", 32, 4096, 2048, 512), ("nvfp4", 64, 3072, 4096, 256)):
        T = E * per
        offs = torch.arange(1, E + 1, device=dev, dtype=torch.int32) * per
        packed = torch.randint(0, 256, (E, N, K // 2), device=dev, dtype=torch.uint8, generator=g)
        if fmt == "mxfp4":
            scales = torch.randint(118, 126, (E, N, K // 32), device=dev, dtype=torch.uint8, generator=g)
        else:
            scales = torch.randint(0x30, 0x60, (E, N, K // 16), device=dev, dtype=torch.uint8, generator=g)
            rs = torch.full((E, N), 1e-2, device=dev)
        for tr in (False, True):
            x = torch.randn(T, N if tr else K, device=dev, generator=g).to(torch.bfloat16)
            y = torch.empty(T, K if tr else N, device=dev, dtype=torch.bfloat16)
            if fmt == "mxfp4":
                fn = lambda: mxq.mxq_grouped_mm_mxfp4(x, packed.view(torch.int8), scales, offs, y, tr)
            else:
                fn = lambda: mxq.mxq_grouped_mm_nvfp4(x, packed, scales, rs, offs, y, tr)
            for _ in range(GEMM_WARMUP):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / reps * 1e-3
            tf = 2.0 * T * N * K / t / 1e12
            # dense reference: [E, per, R] @ [E, R, C], both contiguous
            xd = x.view(E, per, N if tr else K)
            wd = torch.randn(E, N if tr else K, K if tr else N, device=dev, generator=g).to(torch.bfloat16)
            for _ in range(GEMM_WARMUP):
                yd = torch.bmm(xd, wd)
            torch.cuda.synchronize()
            a.record()
            for _ in range(reps):
                torch.bmm(xd, wd, out=yd)
            b.record()
            torch.cuda.synchronize()
            td = a.elapsed_time(b) / reps * 1e-3
            tfd = 2.0 * T * N * K / td / 1e12
            del wd
            # the unfused design: dequantize all weights, then the dense product
            wq = torch.empty(E, N, K, device=dev, dtype=torch.bfloat16)
            if fmt == "mxfp4":
                deq = lambda: mxq.mxq_dequantize_mxfp4(packed.view(torch.int8), scales, wq)
            else:
                deq = lambda: mxq.mxq_dequantize_nvfp4(packed, scales, rs, wq)
            wr = wq if tr else wq.view(E, K, N)
            comp = lambda: (deq(), torch.bmm(xd, wr, out=yd))
            for _ in range(GEMM_WARMUP - 1):      # _time_launches adds one more
                deq()
            t_deq = _time_launches(torch, deq, reps)
            for _ in range(GEMM_WARMUP - 1):
                comp()
            t_comp = _time_launches(torch, comp, reps)
            del wq, wr, yd
            out[f"{fmt}_{'backward' if tr else 'forward'}"] = {
                "experts": E, "N": N, "K": K, "tokens": T, "avg_launch_us": round(t * 1e6, 1),
                "TFLOPs": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                "torch_bmm_dense_bf16_TFLOPs": round(tfd, 1),
                "torch_bmm_dense_us": round(td * 1e6, 1),
                "vs_torch_bmm_dense": round(tf / tfd, 3),
                "dequant_us": round(t_deq * 1e6, 1),
                "dequant_then_bmm_us": round(t_comp * 1e6, 1),
                "speedup_vs_dequant_then_bmm": round(t_comp / t, 3)}
    return out


KV_SETS = 8
# launches of each product before its timed burst: the first launches after
# other work run at a lower clock (up to 20% slower in a burst of GEMMs)
GEMM_WARMUP = 3


def _time_launches(torch, fn, reps):
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e-3


def extra_ops(torch, mxq, synth, dev, x, y, reps, sweep_codes):
    """The other calls of the library, each timed with HIP events around
    `reps` launches on resident inputs, with its algorithmic bytes (inputs
    read once, outputs written once) and its fraction of the HBM peak; not
    part of `value`.
      * MXFP8 quantize / dequantize, MXFP4 and NVFP4 dequantize to
        float16, the static two-level FP4 round trip (block 16, calibrated
        block amax) and per-tensor NVFP4 quantize (a whole-tensor amax pass,
        then the quantize pass) on one 36-expert chunk of the sweep, bf16
        [36, 2048, 7168];
      * the NVFP4 KV cache: per-head quantization with k_smooth of K
        [32768, 12, 128] bf16 (two kernels: the per-head amax pass and the
        quantize pass; its bytes count K read once), and the paged
        dequantization of 32 cache blocks of 1024 tokens into
        [32768, 12, 128] bf16."""
    out = {"peak_GBps": PEAK_HBM_GBPS, "bound": "hbm"}

    def record(name, nbytes, t, **kw):
        gbps = nbytes / t / 1e9
        out[name] = dict(kw, bytes_per_launch=int(nbytes), avg_launch_us=round(t * 1e6, 1),
                         GBps=round(gbps, 1), frac=round(gbps / PEAK_HBM_GBPS, 4))

    ne = synth.C5_CHUNK_EXPERTS
    xs, ys = x[:ne], y[:ne]
    n = xs.numel()
    K = xs.shape[-1]
    codes = torch.empty(xs.shape, dtype=torch.uint8, device=dev)
    sc8 = torch.empty((*xs.shape[:-1], K // 32), dtype=torch.uint8, device=dev)
    b8 = 2 * n + n + n // 32
    record("mxfp8_quant", b8, _time_launches(torch, lambda: mxq.mxq_quantize_mxfp8(xs, codes, sc8), reps),
           shape=list(xs.shape))
    record("mxfp8_dequant", b8, _time_launches(torch, lambda: mxq.mxq_dequantize_mxfp8(codes, sc8, ys), reps),
           shape=list(xs.shape))
    del codes, sc8
    # float16 outputs of the two fp4 dequantizers on the same chunk, from the
    # codes the sweep left for it (the sweep times the bf16 outputs)
    mp, ms, np_, ns, ng = (t[:ne] for t in sweep_codes)
    yh = torch.empty(xs.shape, dtype=torch.float16, device=dev)
    record("mxfp4_dequant_f16", bytes_mx(n),
           _time_launches(torch, lambda: mxq.mxq_dequantize_mxfp4(mp, ms, yh), reps), shape=list(xs.shape))
    record("nvfp4_dequant_f16", bytes_nv(n, n // K),
           _time_launches(torch, lambda: mxq.mxq_dequantize_nvfp4(np_, ns, ng, yh), reps), shape=list(xs.shape))
    del yh
    amax = xs.abs().reshape(-1, K // 16, 16).amax(-1).float()    # calibrated block amax
    gam = xs.abs().max().float().reshape(1)
    bst = 2 * n + 2 * n + 4 * (n // 16) + 4
    record("fp4_static_qdq", bst,
           _time_launches(torch, lambda: mxq.mxq_fake_quantize_fp4_static(xs, amax, gam, ys, 16), reps),
           shape=list(xs.shape), block=16)
    del amax
    # per-tensor NVFP4 (one amax for the whole tensor: a read pass, then the
    # quantize pass); bytes count the input once.  One scale for the whole
    # tensor makes the row length irrelevant to the result (16-value blocks
    # are the same), so the chunk is viewed as rows of 4096: the row kernel
    # instantiation differs from the sweep's, which keeps the two apart in
    # per-kernel profiles.
    xt = xs.reshape(-1, 4096)
    rows = xt.shape[0]
    tp = torch.empty((rows, 4096 // 2), dtype=torch.uint8, device=dev)
    ts = torch.empty((rows, 4096 // 16), dtype=torch.uint8, device=dev)
    tg = torch.empty(rows, dtype=torch.float32, device=dev)
    scr = torch.zeros(1, dtype=torch.float32, device=dev)
    t = _time_launches(torch, lambda: mxq.mxq_quantize_nvfp4(xt, tp, ts, tg, mode="tensor", scratch=scr), reps)
    record("nvfp4_quant_tensor_mode", bytes_nv(n, rows), t, shape=[rows, 4096],
           GBps_with_second_read=round((bytes_nv(n, rows) + 2 * n) / t / 1e9, 1))
    del tp, ts, tg
    # The KV tensors (about 0.1 GB) would stay in the 256 MB last-level cache
    # across back-to-back launches, so the launches cycle through KV_SETS
    # independent sets (about 1 GB in all): each launch reads data that no
    # launch of the previous KV_SETS - 1 has touched.
    S, H, D, bt = 32768, 12, 128, 1024
    nk = S * H * D
    sets = []
    for i in range(KV_SETS):
        sets.append(dict(k=synth.kv_cache((S, H, D), seed=5 + i, device=dev),
                         p=torch.empty((S, H, D // 2), dtype=torch.uint8, device=dev),
                         s=torch.empty((S, H, D // 16), dtype=torch.uint8, device=dev),
                         g=torch.empty((S, H), dtype=torch.float32, device=dev),
                         ha=torch.empty(H * mxq.KV_AMAX_SLOTS, dtype=torch.float32, device=dev)))
    turn = [0]

    def kv_quant():
        c = sets[turn[0] % KV_SETS]
        turn[0] += 1
        mxq.mxq_quantize_kv_nvfp4(c["k"], c["ha"], c["p"], c["s"], c["g"], True)

    bkv = 2 * nk + nk // 2 + nk // 16 + 4 * S * H
    t = _time_launches(torch, kv_quant, reps)
    record("kv_quantize_smooth", bkv, t, shape=[S, H, D], rotating_sets=KV_SETS,
           GBps_with_second_read=round((bkv + 2 * nk) / t / 1e9, 1))
    nb = S // bt
    for c in sets:
        blocks = [(c["p"].reshape(nb, bt * H, D // 2)[b].clone(), c["s"].reshape(nb, bt * H, D // 16)[b].clone(),
                   c["ha"][:H].max().reshape(1).clone()) for b in range(nb)]
        tab = lambda i: torch.tensor([blk[i].data_ptr() for blk in blocks], dtype=torch.int64).to(dev)
        c.update(blocks=blocks, vt=tab(0), st=tab(1), at=tab(2))
        del c["k"], c["p"], c["s"], c["g"]
        c["y"] = torch.empty((S, H, D), dtype=torch.bfloat16, device=dev)

    def kv_pages():
        c = sets[turn[0] % KV_SETS]
        turn[0] += 1
        mxq.mxq_dequantize_kv_pages_nvfp4(c["vt"], c["st"], c["at"], bt, c["y"])

    bpg = nk // 2 + nk // 16 + 4 * nb + 2 * nk
    record("kv_pages_dequant", bpg, _time_launches(torch, kv_pages, reps),
           blocks=nb, block_tokens=bt, heads=H, head_dim=D, rotating_sets=KV_SETS)
    return out


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x_gpu, budget_s: float):
    """The CPU oracle, as it is, on a bounded sample of the same sweep: every
    16th batch of 256 rows, gathered until about `budget_s` seconds of
    single-thread work (estimated from the first batch), all four weight
    operations.  Timed twice on the same sample: on one thread, and on every
    thread the oracle's OpenMP row loops get on this host (OMP_NUM_THREADS, or
    all CPUs the process may run on).  `value` is the all-thread rate."""
    import torch
    import oracle
    K = x_gpu.shape[-1]
    rows = x_gpu.reshape(-1, K)
    batch = 256

    def run(xs):
        t = time.perf_counter()
        p, s = oracle.quantize_mxfp4(xs)
        oracle.dequantize_mxfp4(p, s, torch.bfloat16)
        p, s, g = oracle.quantize_nvfp4(xs)
        oracle.dequantize_nvfp4(p, s, g, torch.bfloat16)
        return time.perf_counter() - t

    all_threads = oracle.max_threads()
    oracle.set_threads(1)
    first = rows[:batch].cpu()
    t1 = run(first)
    nb = max(1, min(int(budget_s / max(t1, 1e-6)), rows.shape[0] // (batch * 16)))
    idx = torch.cat([torch.arange(b * batch * 16, b * batch * 16 + batch) for b in range(nb)])
    xs = rows[idx.to(rows.device)].cpu()
    n = xs.numel()
    nbytes = 2 * bytes_mx(n) + 2 * bytes_nv(n, xs.shape[0])
    secs1 = run(xs)
    oracle.set_threads(all_threads)
    secsn = run(xs)
    return {"value": round(nbytes / secsn / 1e9, 4), "unit": "GB/s", "cores": all_threads,
            "kind": "oracle",
            "sample": f"{xs.shape[0]} rows x {K} of the sweep (every 16th 256-row batch), MXFP4 and "
                      f"NVFP4 quantize and dequantize, {nbytes} algorithmic bytes: "
                      f"{secsn:.2f} s on {all_threads} threads, {secs1:.1f} s on 1 thread",
            "single_thread_value": round(nbytes / secs1 / 1e9, 4),
            "threads": all_threads, "host_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": _cpu_model()}


if __name__ == "__main__":
    main()
