#!/usr/bin/env python3
"""Decode-step benchmark of the INT4 KV-cache path on one MI355X.

Workload (the headline): Llama-3-8B-shaped decode, 32 layers, 32 query heads over 8 KV
heads (GQA 4:1), head_dim 128, batch 8, 8192 cached positions per sequence.  One step =
for every layer, kvq_append_decode_attn: quantize the new token's K/V into slot 8192 and
attend over the 8193 positions (one kernel per layer on this shape; --unfused runs
kvq_append then kvq_decode_attn instead).  The 32 layers have distinct caches (2.36 GB
of packed K/V in total), so the 256 MB Infinity Cache cannot serve a step.  Inputs are
seeded synthetic fp16 N(0,1) K/V with 3 of 128 channels x20 (synth.py), quantized into
the caches before timing.

Prints ONE JSON line: effective KV GB/s (algorithmic bytes per step / step time), the
roofline of the dominant kernel, and the CPU oracle timed on a bounded sample.

--workload selects one of the other workloads instead (each prints its own JSON line of
the same form; the default run is the headline above):
  mha7b-prefill  kvq_quantize_prefill of one MHA-7B-shaped layer (B 8, 32 heads x 128,
                 20480 positions): pure streaming, 3.42 GB per layer
  mha7b-decode   32 layers of decode over 20480 positions, one query head per KV head
  ctx128k-int4   32 layers of batch-1 decode over 131072 positions, INT4 K g64 / V g128
  ctx128k-int8   the same with the INT8 per-token format
  gemma-codec    Gemma-3-4B-shaped step of the WHT + Lloyd-Max codec: 34 layers (29 with a
                 1024-row window ring, 5 global), append at position 4096 then attend
  llama8b-sinks  the headline shape with every layer windowed: a 4096-row ring plus 4
                 attention-sink positions, append at position 8192 then attend 4100 rows
  gemma-codec3   the gemma-codec step with the 3-bit codec
  llama8b-int4h  the headline step on INT4 with fp16 scales (split-K kernel)
  llama8b-recent the headline step with the last 128 positions also kept, and read, in
                 fp16 (8065 rows from the INT4 codes, 128 from the fp16 rings)
  llama8b-paged  the headline step on the paged layout: pages of 16 positions, each
                 sequence's pages shuffled over the pool by a seeded block table
  dequant        kvq_dequant of K and V of 8 Llama-3-8B-shaped layer caches to fp32
  llama8b-prefill-chunk  chunked prefill on the Llama-3-8B shape: per layer, quantize a
                 512-token chunk into positions 7680 .. 8191 and attend it causally
                 (kvq_prefill_attn); TFLOP/s against the fp16 matrix-core peak
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
MFMA_F16_PEAK_TFS = 2500.0   # MI355X dense fp16 matrix-core peak, published
# Sources of the dominant kernel (and its build flags): HBM-traffic counters recorded in
# profiles/ are reported only while these files hash to the value recorded with them.
_COMMON = ["int4_quantized_kv_amd/csrc/kvq_device.h", "int4_quantized_kv_amd/csrc/kvq_internal.h",
           "int4_quantized_kv_amd/csrc/kvq_arith.h", "int4_quantized_kv_amd/build.py"]
KERNEL_SOURCES = ["int4_quantized_kv_amd/csrc/decode_mfma.hip"] + _COMMON
TRAFFIC_FILE = "profiles/decode_int4_mfma_llama8b_ctx8k_b8_traffic.md"
# the other workloads: (traffic record, sources of the kernels it covers)
OTHER_TRAFFIC = {
    "mha7b-prefill": ("profiles/quant_int4_mha7b_ctx20k_b8_traffic.md",
                      ["int4_quantized_kv_amd/csrc/quant.hip"] + _COMMON),
    "dequant": ("profiles/dequant_int4_llama8b_ctx8k_b8_traffic.md",
                ["int4_quantized_kv_amd/csrc/quant.hip"] + _COMMON),
    "mha7b-decode": ("profiles/decode_int4_mfma_mha7b_ctx20k_b8_traffic.md", KERNEL_SOURCES),
    "ctx128k-int4": ("profiles/decode_int4_mfma_ctx128k_b1_traffic.md", KERNEL_SOURCES),
    "ctx128k-int8": ("profiles/decode_mfma_int8_ctx128k_b1_traffic.md", KERNEL_SOURCES),
    "gemma-codec": ("profiles/decode_splitk_codec_gemma3_4b_b4_traffic.md",
                    ["int4_quantized_kv_amd/csrc/decode.hip"] + _COMMON),
    "llama8b-sinks": ("profiles/decode_int4_mfma_llama8b_window4k_sinks4_traffic.md", KERNEL_SOURCES),
    "llama8b-recent": ("profiles/decode_int4_mfma_llama8b_ctx8k_recent128_traffic.md", KERNEL_SOURCES),
    "gemma-codec3": ("profiles/decode_splitk_codec3_gemma3_4b_b4_traffic.md",
                     ["int4_quantized_kv_amd/csrc/decode.hip"] + _COMMON),
    "llama8b-int4h": ("profiles/decode_int4_mfma_int4h_llama8b_ctx8k_b8_traffic.md", KERNEL_SOURCES),
    "llama8b-paged": ("profiles/decode_int4_mfma_llama8b_ctx8k_paged16_traffic.md", KERNEL_SOURCES),
    "llama8b-prefill-chunk": ("profiles/prefill_int4_mfma_llama8b_chunk512_ctx8k_traffic.md", KERNEL_SOURCES),
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--workload", default="llama8b",
                   choices=["llama8b", "mha7b-prefill", "mha7b-decode", "ctx128k-int4",
                            "ctx128k-int8", "gemma-codec", "gemma-codec3", "llama8b-sinks", "llama8b-recent",
                            "llama8b-int4h", "llama8b-paged", "llama8b-prefill-chunk",
                            "dequant"])
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=None, help="override the layer count (debug only)")
    p.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    p.add_argument("--unfused", action="store_true",
                   help="kvq_append + kvq_decode_attn per layer instead of kvq_append_decode_attn")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="timed CPU work of the oracle baseline (whole (batch, kv head) units)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="time a plain 1 GiB device copy and a 1 GiB read-only reduction instead "
                        "(the known-size reference for the HBM counters)")
    p.add_argument("--calibrate-read", action="store_true",
                   help="sweep the streaming-read kernel (libkvq_bench.so) over launch shapes on "
                        "4 GiB and print the table (the attainable read rate every line reports)")
    p.add_argument("--timeline", action="store_true",
                   help="phase timeline of the headline step's kernel from the probe build "
                        "libkvq_timeline.so (python -m int4_quantized_kv_amd.build --timeline)")
    p.add_argument("--no-attainable", action="store_true",
                   help="leave out the attainable-read measurement of the line")
    p.add_argument("--cpu-workers", type=int, default=None,
                   help="processes of the all-core oracle leg (default: the affinity set, at most 16)")
    return p.parse_args()


class Layer:
    pass


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the decode path has no multi-GPU implementation.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy(args)
        return
    if args.calibrate_read:
        calibrate_read(args)
        return
    if args.timeline:
        timeline(args)
        return
    import int4_quantized_kv_amd as kvq
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.workload != "llama8b":
        line = OTHER[args.workload](args)
        if args.workload in OTHER_TRAFFIC:
            line["roofline"]["traffic"] = recorded_traffic(*OTHER_TRAFFIC[args.workload])
        add_attainable(args, line)
        print(json.dumps(line), flush=True)
        return
    w = synth.WORKLOADS[2]
    nl = args.layers or w.layers
    B, Hq, Hkv, D, S = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.context
    L = S + 1
    desc = kvq.make_desc("int4", B, Hkv, D, L, w.group_k, w.group_v)
    dref = ctypes.byref(desc)

    layers = []
    for li in range(nl):
        k, v, q, kn, vn = synth.layer_inputs(w, li, dev)
        lay = Layer()
        lay.dc = kvq.DeviceCache(desc, dev)
        kvq.kvq_quantize_prefill(desc, lay.dc.c, k, v, 0, S)
        del k, v
        lay.q, lay.kn, lay.vn = q, kn, vn
        lay.out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        lay.cref = ctypes.byref(lay.dc.c)
        layers.append(lay)
    torch.cuda.synchronize()

    lens = (ctypes.c_int32 * B)(*([L] * B))
    pos = (ctypes.c_int32 * B)(*([S] * B))
    ws = kvq.decode_workspace(desc, Hq, L, device=dev)
    ws_bytes = ws.numel() * 4
    nsplit = kvq.kvq_plan_splits(desc, Hq, L)
    LIB = kvq.LIB

    def step(stream, append=True, attend=True):
        sp = ctypes.c_void_p(stream)
        for lay in layers:
            if not args.unfused:
                st = LIB.kvq_append_decode_attn(dref, lay.cref, lay.kn.data_ptr(), lay.vn.data_ptr(),
                                                lay.q.data_ptr(), Hq, lens, 0, 0.0, 0,
                                                lay.out.data_ptr(), ws.data_ptr(), ws_bytes, sp)
                if st:
                    raise kvq.KvqError(st, "kvq_append_decode_attn")
                continue
            if append:
                st = LIB.kvq_append(dref, lay.cref, lay.kn.data_ptr(), lay.vn.data_ptr(), pos, sp)
                if st:
                    raise kvq.KvqError(st, "kvq_append")
            if attend:
                st = LIB.kvq_decode_attn(dref, lay.cref, lay.q.data_ptr(), Hq, lens, 0, 0.0, 0,
                                         lay.out.data_ptr(), ws.data_ptr(), ws_bytes, sp)
                if st:
                    raise kvq.KvqError(st, "kvq_decode_attn")

    # eager warm-up (also the reference result of a graph replay)
    cur = torch.cuda.current_stream()
    for _ in range(max(1, args.warmup)):
        step(cur.cuda_stream)
    torch.cuda.synchronize()
    eager_out = layers[-1].out.clone()

    def capture(**kw):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=s):
            step(torch.cuda.current_stream().cuda_stream, **kw)
        torch.cuda.synchronize()
        return g

    if args.eager:
        run = lambda: step(torch.cuda.current_stream().cuda_stream)  # noqa: E731
    else:
        g_step = capture()
        run = g_step.replay
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        # (tiles are shared out dynamically, so the fp32 sums may differ in their last
        # bits from run to run; anything beyond rounding is an error)
        if not torch.allclose(layers[-1].out, eager_out, rtol=1e-4, atol=1e-5):
            raise RuntimeError("graph replay differs from the eager result")

    # ---- timed region: exactly K steps, synchronized on both sides; the events are
    # recorded on the stream the kernels run on (the graph replays on the current stream)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        run()
    ev1.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps

    if args.unfused:
        # dominant kernel: kvq_decode_attn alone, all layers, timed in its own pass
        if args.eager:
            attn_run = lambda: step(torch.cuda.current_stream().cuda_stream, append=False)  # noqa: E731
        else:
            g_attn = capture(append=False)
            attn_run = g_attn.replay
        attn_run()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            attn_run()
        e1.record()
        torch.cuda.synchronize()
        kern_ms = e0.elapsed_time(e1) / (args.steps * nl)
        kern_name = "kvq_decode_attn (decode_int4_mfma_kernel, splits merged in-kernel)"
    else:
        # one kernel per layer: the timed region is that kernel's launches back to back
        kern_ms = ms_step / nl
        kern_name = "kvq_append_decode_attn (decode_int4_mfma_kernel with the append fused)"

    # ---- algorithmic bytes of one layer's step: read the 8192 cached rows, write the
    # new row (codes + scales), read its fp16 K/V, read q, write the fp32 output
    row_bytes = (D // 2 + 4 * (D // w.group_k)) + (D // 2 + 4 * (D // w.group_v))  # K + V, 140 B
    layer_bytes = (B * Hkv * S * row_bytes + B * Hkv * row_bytes + B * Hkv * D * 2 * 2
                   + B * Hq * D * 2 + B * Hq * D * 4)
    step_bytes = nl * layer_bytes
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    if args.unfused:   # the attention kernel alone also reads the appended row back
        kern_bytes = B * Hkv * L * row_bytes + B * Hq * D * 2 + B * Hq * D * 4
    else:
        kern_bytes = layer_bytes
    kern_gbs = kern_bytes / (kern_ms * 1e-3) / 1e9

    result = {
        "metric": "INT4-KV decode attn: effective KV GB/s, % HBM peak, tok/s (8B-shape, 8K ctx)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": nl, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "context": L, "format": "int4 K g64 / V g128, fp32 scales",
                   "launch": "eager" if args.eager else "hip-graph", "num_splits": nsplit,
                   "entry": "kvq_append + kvq_decode_attn" if args.unfused else "kvq_append_decode_attn"},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tok_per_s": round(B / (ms_step * 1e-3), 1),
        "bytes_per_step": step_bytes,
        "wall_s_timed": round(wall_s, 4),
        "roofline": {
            "kernel": kern_name,
            "bound": "hbm",
            "achieved": round(kern_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(),
            "bytes_per_launch": kern_bytes,
            "avg_launch_us": round(kern_ms * 1e3, 2),
        },
        "cpu_baseline": None,
    }

    # ---- after the timed region: the step's access pattern alone, on the same caches
    if not args.no_attainable:
        pat_gbs, pat_us = tile_pattern_rate(args, [lay.dc for lay in layers], B * Hkv, L,
                                            4 * (D // w.group_k), nsplit, S)
        result["pattern_read_GBps"] = round(pat_gbs, 1)
        result["pattern_read_config"] = {
            "kernel": "libkvq_bench.so: tile_pattern_kernel", "launches": nl,
            "bytes_per_launch": B * Hkv * S * row_bytes, "avg_launch_us": round(pat_us, 2)}
        result["roofline"]["frac_of_pattern"] = round(kern_gbs / pat_gbs, 4)
    del layers, ws
    add_attainable(args, result)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, L, args.cpu_workers)

    print(json.dumps(result), flush=True)


def tile_pattern_rate(args, caches, units, cap, kscale_bytes, nsplit, rows):
    """The decode step's transfers with no arithmetic (libkvq_bench.so kvqb_tile_pattern):
    each cache's first `rows` rows per (b, kv head) unit, in the decode kernel's 32-row
    tiles, split plan and per-wave ring, one launch per cache replayed as a HIP graph like
    the timed step.  Returns (GB/s of the tile bytes, microseconds per launch)."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "int4_quantized_kv_amd", "libkvq_bench.so"))
    fn = lib.kvqb_tile_pattern
    fn.restype = ctypes.c_int32
    fn.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int32] * 5 + [ctypes.c_void_p]
    tps = rows // (32 * nsplit)

    def step(stream):
        for c in caches:
            st = fn(c.k_codes.data_ptr(), c.k_scales.data_ptr(), c.v_codes.data_ptr(),
                    c.v_scales.data_ptr(), units, cap, kscale_bytes, nsplit, tps,
                    ctypes.c_void_p(stream))
            if st:
                raise RuntimeError(f"kvqb_tile_pattern failed ({st})")

    run = _runner(args, step)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (args.steps * len(caches))
    tile_bytes = units * nsplit * tps * 32 * (128 + kscale_bytes + 4)
    return tile_bytes / (us * 1e-6) / 1e9, us


def kernel_source_hash(sources=None):
    import hashlib
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(traffic_file=None, sources=None):
    """HBM bytes per launch of the dominant kernel from the rocprofv3 FETCH_SIZE and
    WRITE_SIZE passes recorded in the traffic file (each scaled by the factor the same
    counter shows on a copy of known size), or None if there is no record or the kernel
    has changed since it was taken."""
    path = os.path.join(ROOT, traffic_file or TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        line = line.strip().strip("`")
        if ":" in line and line.split(":", 1)[0] in ("source_sha256", "traffic_bytes_per_launch"):
            k, v = line.split(":", 1)
            rec[k] = v.strip()
    if rec.get("source_sha256") != kernel_source_hash(sources) or "traffic_bytes_per_launch" not in rec:
        return None
    return int(rec["traffic_bytes_per_launch"])


def calibrate_copy(args):
    """A plain device copy of 1 GiB (1 GiB read + 1 GiB written per launch) and a
    read-only sum over 1 GiB, timed with events; one JSON line."""
    import torch
    n = 1 << 28                                   # fp32 elements = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    acc = torch.empty((), dtype=torch.float32, device="cuda:0")
    res = {}
    for name, fn in (("copy", lambda: dst.copy_(src)), ("sum", lambda: torch.sum(src, 0, out=acc))):
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        moved = (2 if name == "copy" else 1) * n * 4
        res[name] = {"bytes_read": n * 4, "bytes_written": n * 4 if name == "copy" else 4,
                     "ms": round(ms, 4), "GBps": round(moved / (ms * 1e-3) / 1e9, 1)}
    print(json.dumps({"calibration": res, "steps": args.steps}), flush=True)


# ---------------------------------------------------------------------------------------
# Attainable read rate: the hand-written streaming-read kernel of libkvq_bench.so
# (csrc/stream_read.hip) over 4 GiB, 16-byte loads, `unroll` in flight per lane.

READ_BYTES = 4 << 30
# launch shapes every line tries (workgroups of 256 lanes, loads in flight per lane,
# non-temporal): the five fastest of the 48-shape sweep of --calibrate-read (1K-32K
# workgroups, 2-16 loads in flight, plain and non-temporal; all five non-temporal).
# The best median of them is the line's attainable read rate.
READ_CONFIGS = [(32768, 16, 1), (32768, 8, 1), (16384, 16, 1), (1024, 2, 1), (16384, 8, 1)]


def _bench_lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "int4_quantized_kv_amd", "libkvq_bench.so"))
    fn = lib.kvqb_stream_read
    fn.restype = ctypes.c_int32
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    return fn


def _read_rate(fn, buf, sink, grid, unroll, nt, reps):
    """Median GB/s of `reps` event-timed launches of the streaming read."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream

    def launch():
        st = fn(buf.data_ptr(), READ_BYTES, grid, unroll, nt, sink.data_ptr(), ctypes.c_void_p(stream))
        if st:
            raise RuntimeError(f"kvqb_stream_read failed ({st})")

    launch()
    torch.cuda.synchronize()
    rates = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        launch()
        e1.record()
        torch.cuda.synchronize()
        rates.append(READ_BYTES / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    rates.sort()
    return rates[len(rates) // 2]


def attainable_read(configs=READ_CONFIGS, reps=7):
    """(best median GB/s, its config) of the streaming read over a 4 GiB buffer."""
    import torch
    fn = _bench_lib()
    buf = torch.ones(READ_BYTES // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.empty(max(c[0] for c in configs), dtype=torch.int32, device="cuda:0")
    best = (0.0, None)
    table = []
    for grid, unroll, nt in configs:
        r = _read_rate(fn, buf, sink, grid, unroll, nt, reps)
        table.append({"workgroups": grid, "loads_in_flight": unroll, "nontemporal": bool(nt),
                      "GBps": round(r, 1)})
        if r > best[0]:
            best = (r, table[-1])
    del buf, sink
    torch.cuda.empty_cache()
    return best[0], best[1], table


def add_attainable(args, line):
    """Put the attainable read rate into the line, and the roofline kernel's share of it."""
    if args.no_attainable:
        return
    rate, cfg, _ = attainable_read()
    line["attainable_read_GBps"] = round(rate, 1)
    line["attainable_read_config"] = dict(cfg, bytes=READ_BYTES,
                                          kernel="libkvq_bench.so: stream_read_kernel")
    roof = line.get("roofline")
    if roof and roof.get("unit") == "GB/s":
        roof["frac_of_attainable"] = round(roof["achieved"] / rate, 4)


def calibrate_read(args):
    configs = [(g, u, nt) for g in (1024, 2048, 4096, 8192, 16384, 32768)
               for u in (2, 4, 8, 16) for nt in (0, 1)]
    rate, cfg, table = attainable_read(configs, reps=max(5, args.steps // 2))
    print(json.dumps({"stream_read": table, "best": cfg, "bytes": READ_BYTES}), flush=True)


def timeline(args):
    """Per-phase timeline of the headline step's matrix-core kernel, from the probe build
    (libkvq_timeline.so: the same sources with -DKVQ_TIMELINE, each workgroup recording
    the 100 MHz real-time counter at its phase points).  The 32 layers of the step run
    from a HIP graph as in the timed bench; the stamps of the last replay are read back.
    Prints one JSON line: per phase, the median over layers of (min, median, max) over
    the layer's workgroups (waves for loop ends), in microseconds from the layer's first
    workgroup entry, plus the gap from each layer's last exit to the next layer's first
    entry and the loop-end medians per XCD."""
    import numpy as np
    import torch
    import int4_quantized_kv_amd as kvq
    from int4_quantized_kv_amd import _binding
    import synth
    lib = _binding._load(os.path.join(ROOT, "int4_quantized_kv_amd", "libkvq_timeline.so"))
    dev = "cuda:0"
    w = synth.WORKLOADS[2]
    nl = args.layers or w.layers
    B, Hq, Hkv, D, S = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.context
    L = S + 1
    desc = kvq.make_desc("int4", B, Hkv, D, L, w.group_k, w.group_v)
    ns = kvq.kvq_plan_splits(desc, Hq, L)
    need = kvq.kvq_decode_workspace_bytes(desc, Hq, L)
    nwg = ns * Hkv * B
    tl_off = (need + 255) // 256 * 256
    layers = []
    for li in range(nl):
        k, v, q, kn, vn = synth.layer_inputs(w, li, dev)
        lay = Layer()
        lay.dc = kvq.DeviceCache(desc, dev)
        kvq.kvq_quantize_prefill(desc, lay.dc.c, k, v, 0, S)
        del k, v
        lay.q, lay.kn, lay.vn = q, kn, vn
        lay.out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        lay.ws = torch.zeros((tl_off + nwg * 256) // 4, dtype=torch.float32, device=dev)
        lay.cref = ctypes.byref(lay.dc.c)
        layers.append(lay)
    torch.cuda.synchronize()
    lens = (ctypes.c_int32 * B)(*([L] * B))
    dref = ctypes.byref(desc)

    def step(stream):
        sp = ctypes.c_void_p(stream)
        for lay in layers:
            st = lib.kvq_append_decode_attn(dref, lay.cref, lay.kn.data_ptr(), lay.vn.data_ptr(),
                                            lay.q.data_ptr(), Hq, lens, 0, 0.0, 0, lay.out.data_ptr(),
                                            lay.ws.data_ptr(), lay.ws.numel() * 4, sp)
            if st:
                raise kvq.KvqError(st, "kvq_append_decode_attn (timeline build)")

    run = _runner(args, step)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    stamps = [lay.ws.view(torch.int64)[tl_off // 8: tl_off // 8 + nwg * 32].cpu().numpy()
              .reshape(nwg, 32).astype(np.int64) for lay in layers]
    us = lambda t: t / 100.0   # noqa: E731  (100 MHz counter)
    per = {k: [] for k in ("entry", "kernel_args", "q_in_lds", "first_tile", "loop_start", "loop_end",
                           "published", "arrived", "exit")}
    gaps, xcc_end, tiles = [], {}, []
    for li, st in enumerate(stamps):
        t0 = st[:, 0].min()
        rel = lambda col: us(st[:, col] - t0)   # noqa: E731
        per["entry"].append(np.percentile(rel(0), [0, 50, 100]))
        per["kernel_args"].append(np.percentile(rel(16), [0, 50, 100]))
        per["q_in_lds"].append(np.percentile(rel(2), [0, 50, 100]))
        per["first_tile"].append(np.percentile(rel(17), [0, 50, 100]))
        per["loop_start"].append(np.percentile(rel(3), [0, 50, 100]))
        ends = us(st[:, 4:12] - t0).ravel()
        per["loop_end"].append(np.percentile(ends, [0, 50, 100]))
        per["published"].append(np.percentile(rel(12), [0, 50, 100]))
        per["arrived"].append(np.percentile(rel(13), [0, 50, 100]))
        per["exit"].append(np.percentile(rel(14), [0, 50, 100]))
        if li + 1 < len(stamps):
            gaps.append(us(stamps[li + 1][:, 0].min() - st[:, 14].max()))
        xcc = (st[:, 1] >> 32) & 0xF
        for x in np.unique(xcc):
            xcc_end.setdefault(int(x), []).append(float(np.median(us(st[xcc == x][:, 4:12] - t0))))
        t = st[:, 15]
        tiles.extend(((t >> (8 * wv)) & 255).tolist() for wv in range(8))
    tl = np.array(tiles).ravel()
    # where the loop-end spread comes from: per workgroup, its last wave's loop end
    # (relative to the layer's first entry), by split index; the spread inside a
    # workgroup; and whether late workgroups started late
    by_sp, intra, corr = {}, [], []
    for st in stamps:
        t0 = st[:, 0].min()
        wg_end = us(st[:, 4:12].max(1) - t0)
        intra.extend(us(st[:, 4:12].max(1) - st[:, 4:12].min(1)).tolist())
        for sp in range(ns):
            by_sp.setdefault(sp, []).extend(wg_end[sp::ns].tolist())
        corr.append(float(np.corrcoef(us(st[:, 0] - t0), wg_end)[0, 1]))
    # what makes a workgroup late: its first tile's arrival, its compute unit (the same
    # CU late in every layer), or its (b, kv head) unit's data (the unit's other splits
    # late with it); lateness = last loop end minus the layer's median
    corr_first, corr_unit, late_by_cu, unit_bound = [], [], {}, []
    for st in stamps:
        t0 = st[:, 0].min()
        wg_end = us(st[:, 4:12].max(1) - t0)
        late = wg_end - np.median(wg_end)
        # the last loop end if each (b, kv head) unit's splits shared its tiles perfectly
        # (every split ending at the mean of their ends), against the actual last one
        unit_bound.append((float(wg_end.mean()), float(wg_end.reshape(-1, ns).mean(1).max()),
                           *np.percentile(wg_end, [50, 90, 99, 100]).tolist()))
        corr_first.append(float(np.corrcoef(us(st[:, 17] - t0), wg_end)[0, 1]))
        per_unit = late.reshape(-1, ns)
        others = (per_unit.sum(1, keepdims=True) - per_unit) / max(ns - 1, 1)
        if ns > 1:
            corr_unit.append(float(np.corrcoef(per_unit.ravel(), others.ravel())[0, 1]))
        cu = ((st[:, 1] >> 32) & 0xF) * 256 + ((st[:, 1] >> 8) & 0xFF)
        for c, x in zip(cu.tolist(), late.tolist()):
            late_by_cu.setdefault(c, []).append(x)
    cu_mean = np.array([np.mean(v) for v in late_by_cu.values() if len(v) > 1])
    all_late = np.concatenate([np.array(v) for v in late_by_cu.values()])
    out_extra = {"wg_last_loop_end_by_split_us": {sp: [round(float(x), 2) for x in np.percentile(v, [0, 50, 100])]
                                                 for sp, v in by_sp.items()},
                 "loop_end_spread_inside_wg_us": [round(float(x), 2) for x in np.percentile(intra, [0, 50, 90, 100])],
                 "corr_entry_vs_wg_end": round(float(np.median(corr)), 3),
                 "corr_first_tile_vs_wg_end": round(float(np.median(corr_first)), 3),
                 "corr_wg_vs_unit_siblings_lateness": round(float(np.median(corr_unit)), 3) if corr_unit else None,
                 # (mean over all workgroups, max over units of their mean, percentiles
                 # 50 / 90 / 99 / 100 over workgroups)
                 "wg_last_loop_end_mean_unitmax_p50_p90_p99_max_us": [round(float(x), 2)
                                                               for x in np.median(np.array(unit_bound), axis=0)],
                 "compute_units_seen": len(late_by_cu),
                 "lateness_sd_us": round(float(all_late.std()), 3),
                 "per_cu_mean_lateness_sd_us": round(float(cu_mean.std()), 3) if cu_mean.size else None,
                 "per_cu_mean_lateness_max_us": round(float(cu_mean.max()), 3) if cu_mean.size else None}
    out = {"timeline_us": {k: [round(float(x), 2) for x in np.median(np.array(v), axis=0)]
                           for k, v in per.items()},
           **out_extra,
           "columns": ["min", "median", "max"],
           "gap_to_next_layer_us": [round(float(x), 2) for x in np.percentile(gaps, [0, 50, 100])] if gaps else None,
           "loop_end_median_by_xcc_us": {k: round(float(np.median(v)), 2) for k, v in sorted(xcc_end.items())},
           "tiles_per_wave": [int(tl.min()), float(np.median(tl)), int(tl.max())],
           "workgroups": nwg, "layers": nl, "num_splits": ns,
           "workload": w.name, "entry": "kvq_append_decode_attn (timeline probe build)"}
    print(json.dumps(out), flush=True)


def _blas_threads():
    from threadpoolctl import threadpool_info
    return max((i.get("num_threads", 0) for i in threadpool_info()), default=0)


def _cpu_meta(workers_used):
    return {"os_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas_threads_default": _blas_threads(), "blas_threads_used": 1,
            "threads_used": workers_used}


def _allcore_unit(task):
    """One worker of the all-core leg: `reps` headline units (append the new row,
    exact dequantization of 8193 rows, fp64 attention for the unit's query heads) over
    the unit's arrays, on one core; returns (start, end) wall times of its timed work."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attention, quant
    k, v, kn, vn, qq, L, reps = task
    (ck, sk), (cv, sv) = quant.quantize_int4(k, 64), quant.quantize_int4(v, 128)
    with threadpool_limits(1):
        t0 = time.time()
        for _ in range(reps):
            nk, nsk = quant.quantize_int4(kn[None], 64)
            nv, nsv = quant.quantize_int4(vn[None], 128)
            kh = quant.dequantize_int4_exact(np.concatenate([ck, nk]), np.concatenate([sk, nsk]), 64)
            vh = quant.dequantize_int4_exact(np.concatenate([cv, nv]), np.concatenate([sv, nsv]), 128)
            attention.decode_attention(qq[None], kh[None, None], vh[None, None], [L])
        t1 = time.time()
    return t0, t1


def cpu_baseline(w, seconds, L, workers=None):
    """The oracle (never tuned) timed on host cores, one (batch, kv head) unit of a layer
    at a time, layer after layer, until `seconds` of timed work: quantize the new row,
    dequantize the cache exactly, fp64 softmax attention for the unit's G query heads.
    The cache state a unit starts from (the prefill) is built outside the timer.
    Single-threaded BLAS."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import synth
    from oracle import attention, quant

    G = w.q_heads // w.kv_heads
    units = 0
    dt = 0.0
    layer = 0
    while dt < seconds and layer < w.layers:
        k, v, q, kn, vn = (t.cpu().numpy() for t in synth.layer_inputs(w, layer, "cuda:0"))
        for b in range(w.batch):
            for h in range(w.kv_heads):
                if dt >= seconds:
                    break
                (ck, sk), (cv, sv) = quant.quantize_int4(k[b, h], 64), quant.quantize_int4(v[b, h], 128)
                qq = q[b, h * G:(h + 1) * G]
                with threadpool_limits(1):
                    t0 = time.perf_counter()
                    nk, nsk = quant.quantize_int4(kn[b, h][None], 64)     # append the new row
                    nv, nsv = quant.quantize_int4(vn[b, h][None], 128)
                    ck2 = np.concatenate([ck, nk]); sk2 = np.concatenate([sk, nsk])
                    cv2 = np.concatenate([cv, nv]); sv2 = np.concatenate([sv, nsv])
                    kh = quant.dequantize_int4_exact(ck2, sk2, 64)
                    vh = quant.dequantize_int4_exact(cv2, sv2, 128)
                    attention.decode_attention(qq[None], kh[None, None], vh[None, None], [L])
                    dt += time.perf_counter() - t0
                units += 1
        layer += 1
        del k, v
    S = L - 1
    row = 140
    unit_bytes = S * row + row + 2 * 128 * 2 + G * 128 * 2 + G * 128 * 4
    full = w.batch * w.kv_heads * w.layers
    res = {"value": round(units * unit_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
           "kind": "oracle",
           "sample": f"{units} of the step's {full} (layer, batch, kv head) units "
                     f"(append + exact dequant + fp64 attention over {L} positions), "
                     f"{dt:.2f} s timed on one core; a full step extrapolates to "
                     f"{dt * full / units:.1f} s"}
    res.update(_cpu_meta(1))
    # ---- all-core leg: one process per core of the affinity set (at most 16), each
    # running whole units of the first layer over its own arrays for ~seconds / 2
    import multiprocessing as mp
    nw = workers or min(16, len(os.sched_getaffinity(0)))
    reps = max(1, int(0.5 * seconds / (dt / units)))
    k, v, q, kn, vn = (t.cpu().numpy() for t in synth.layer_inputs(w, 0, "cuda:0"))
    tasks = []
    for i in range(nw):
        b, h = divmod(i % (w.batch * w.kv_heads), w.kv_heads)
        tasks.append((k[b, h], v[b, h], kn[b, h], vn[b, h], q[b, h * G:(h + 1) * G], L, reps))
    del k, v
    with mp.get_context("spawn").Pool(nw) as pool:
        spans = pool.map(_allcore_unit, tasks)
    wall = max(e for _, e in spans) - min(b0 for b0, _ in spans)
    res["all_cores"] = {"value": round(nw * reps * unit_bytes / wall / 1e9, 4), "unit": "GB/s",
                        "cores": nw, "processes": nw,
                        "sample": f"{nw} processes x {reps} units each (append + exact dequant + "
                                  f"fp64 attention over {L} positions), {wall:.2f} s wall, one "
                                  f"BLAS thread per process"}
    return res


# ---------------------------------------------------------------------------------------
# The other workloads (--workload).  Each returns the JSON object of its line.

def row_bytes(fmt, D, gk, gv):
    """Bytes of K + V codes and scales per (position, kv head)."""
    if fmt in ("int4", "int4h"):
        sb = 4 if fmt == "int4" else 2
        return (D // 2 + sb * (D // gk)) + (D // 2 + sb * (D // gv))
    if fmt == "int8":
        return 2 * (D + 4)
    if fmt == "codec3":
        return 2 * (3 * D // 8 + 4)                       # three bit-planes + one scale
    return 2 * (D // 2 + 4)                               # codec: indices + one scale


def _timed(run, steps):
    """ms per call of `run` over exactly `steps` calls, events on the current stream
    (torch.cuda.synchronize on both sides), and the wall seconds of the region."""
    import torch
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, time.perf_counter() - t0


def _runner(args, fn):
    """A HIP-graph replay of fn(stream) (or eager calls with --eager), warmed up."""
    import torch
    cur = torch.cuda.current_stream()
    for _ in range(max(1, args.warmup)):
        fn(cur.cuda_stream)
    torch.cuda.synchronize()
    if args.eager:
        return lambda: fn(torch.cuda.current_stream().cuda_stream)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        fn(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    return g.replay


def _line(args, metric, value, ms, config, roofline, cpu, extra, dtype="f32"):
    out = {"metric": metric, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
           "data": "synthetic", "config": config, "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2)}
    out.update(extra)
    out["roofline"] = roofline
    out["cpu_baseline"] = cpu
    return out


def _roofline(kernel, nbytes, us):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
            "bytes_per_launch": int(nbytes), "avg_launch_us": round(us, 2)}


DECODE_MODES = {   # workload id, cache format
    "mha7b-decode": (3, "int4"),
    "ctx128k-int4": (5, "int4"),
    "ctx128k-int8": (5, "int8"),
    "gemma-codec": (4, "codec"),
    "gemma-codec3": (8, "codec3"),
    "llama8b-int4h": (9, "int4h"),
    "llama8b-sinks": (6, "int4"),
    "llama8b-recent": (7, "int4"),
    "llama8b-paged": (10, "int4"),
}


def attended_rows(L, W, sinks):
    """Rows a decode step of length L attends: all of them, or the window's W and the
    sink positions that lie before it."""
    if not W or W >= L:
        return L
    return W + min(sinks, L - W)


def bench_decode(args):
    """One decode step over every layer of a workload: for appending workloads
    kvq_append_decode_attn per layer (append at position `context`, attend over
    context + 1), otherwise kvq_decode_attn.  Window layers keep a ring of `window` rows
    (after `sinks` slots for the first positions when the workload keeps sinks)."""
    import torch
    import int4_quantized_kv_amd as kvq
    import synth
    wid, fmt = DECODE_MODES[args.workload]
    w = synth.WORKLOADS[wid]
    dev = "cuda:0"
    nl = args.layers or w.layers
    B, Hq, Hkv, D, S = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.context
    L = S + 1 if w.append else S
    rb = row_bytes(fmt, D, w.group_k, w.group_v)
    LIB = kvq.LIB
    layers, ws_need = [], 0
    attend_bytes = step_bytes = 0
    for li in range(nl):
        lay = Layer()
        lay.W = w.layer_window(li)
        ns = w.sinks if lay.W else 0
        cap = lay.W + ns if lay.W else L
        if w.page_size:   # paged layout: shuffled pages from a pool of exactly enough
            P = w.page_size
            cap = (L + P - 1) // P * P
            table, npages = synth.block_table(B, cap, P, synth.seed_of(w.wid, li, 5))
            lay.desc = kvq.make_desc(fmt, B, Hkv, D, cap, w.group_k, w.group_v, page_size=P,
                                     num_pages=npages)
            lay.table = table.to(dev)
        else:
            lay.desc = kvq.make_desc(fmt, B, Hkv, D, cap, w.group_k, w.group_v, sinks=ns, recent=w.recent)
            lay.table = None
        k, v, q, kn, vn = synth.layer_inputs(w, li, dev)
        lay.dc = kvq.DeviceCache(lay.desc, dev, block_table=lay.table)
        if ns:                        # the sink positions, in their own slots
            kvq.kvq_quantize_prefill(lay.desc, lay.dc.c, k[:, :, :ns].contiguous(),
                                     v[:, :, :ns].contiguous(), 0, ns)
        lo = max(ns, S - (cap - ns))  # the rows a ring of cap - ns slots still holds
        kvq.kvq_quantize_prefill(lay.desc, lay.dc.c, k[:, :, lo:].contiguous(),
                                 v[:, :, lo:].contiguous(), lo, S - lo)
        del k, v
        lay.q, lay.kn, lay.vn = q, kn, vn
        lay.out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        lay.dref, lay.cref = ctypes.byref(lay.desc), ctypes.byref(lay.dc.c)
        ws_need = max(ws_need, kvq.kvq_decode_workspace_bytes(lay.desc, Hq, L, lay.W))
        # the step reads the cached rows of the horizon (all but the new one when it
        # appends), the new row's fp16 K/V, q; writes the new row's codes and the output.
        # The attention call alone (for the roofline) reads every row of the horizon.
        rows = attended_rows(L, lay.W, ns)
        qo = B * Hq * D * 2 + B * Hq * D * 4
        # rows read in fp16 (recent) cost 2 * D * 2 bytes each instead of rb; the
        # appended row is quantized (rb written) and, with recent rows, also written in
        # fp16 to its ring row
        nr = min(rows, w.recent)
        f16row = 2 * D * 2
        attend_bytes += B * Hkv * ((rows - nr) * rb + nr * f16row) + qo
        if w.append and nr:   # nr - 1 ring rows and the new row read; rb + f16row written
            step_bytes += B * Hkv * ((rows - nr) * rb + nr * f16row + rb + f16row) + qo
        elif w.append:        # rows - 1 cached rows and the new row read; rb written
            step_bytes += B * Hkv * ((rows - 1) * rb + f16row + rb) + qo
        else:
            step_bytes += B * Hkv * ((rows - nr) * rb + nr * f16row) + qo
        layers.append(lay)
    torch.cuda.synchronize()
    ws = torch.zeros(ws_need // 4 + 4, dtype=torch.float32, device=dev)
    ws_bytes = ws.numel() * 4
    lens = (ctypes.c_int32 * B)(*([L] * B))

    def step(stream, attend_only=False):
        sp = ctypes.c_void_p(stream)
        for lay in layers:
            if w.append and not attend_only:
                st = LIB.kvq_append_decode_attn(lay.dref, lay.cref, lay.kn.data_ptr(), lay.vn.data_ptr(),
                                                lay.q.data_ptr(), Hq, lens, lay.W, 0.0, 0,
                                                lay.out.data_ptr(), ws.data_ptr(), ws_bytes, sp)
            else:
                st = LIB.kvq_decode_attn(lay.dref, lay.cref, lay.q.data_ptr(), Hq, lens, lay.W, 0.0, 0,
                                         lay.out.data_ptr(), ws.data_ptr(), ws_bytes, sp)
            if st:
                raise kvq.KvqError(st, "decode step")

    run = _runner(args, step)
    ms_step, wall = _timed(run, args.steps)
    if w.append:     # the attention calls alone, in their own pass
        attn = _runner(args, lambda st: step(st, attend_only=True))
        attn_ms, _ = _timed(attn, args.steps)
    else:
        attn_ms = ms_step
    if fmt in ("int4", "int4h") and D == 128 and w.group_v == 128:
        kern = "kvq_decode_attn: decode_int4_mfma_kernel (splits merged in-kernel)"
        if fmt == "int4h":
            kern = ("kvq_decode_attn: decode_int4_mfma_kernel, fp16-scale instance (splits merged "
                    "in-kernel)")
        if w.page_size:
            kern = (f"kvq_decode_attn: decode_int4_mfma_kernel, paged instance (pages of "
                    f"{w.page_size}, splits merged in-kernel)")
        if w.sinks and w.window_layers:
            kern = "kvq_decode_attn: decode_int4_mfma_kernel, sink instance (splits merged in-kernel)"
        if w.recent:
            kern = ("kvq_decode_attn: decode_int4_mfma_kernel, recent-row instance (splits and the "
                    "fp16-row workgroup merged in-kernel)")
    elif fmt == "int8" and D == 128:
        kern = "kvq_decode_attn: decode_int4_mfma_kernel, INT8 tiles (splits merged in-kernel)"
    else:
        kern = f"kvq_decode_attn: decode_splitk_kernel<{D}, {Hq // Hkv}, {fmt}> + merge_kernel"
    roof = _roofline(kern, attend_bytes / nl, attn_ms * 1e3 / nl)
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    cfg = {"workload": w.name, "format": fmt, "layers": nl, "batch": B, "q_heads": Hq,
           "kv_heads": Hkv, "head_dim": D, "context": L, "append": w.append,
           "window_layers": min(nl, w.window_layers), "window": w.window, "sinks": w.sinks,
           "recent_fp16": w.recent, "page_size": w.page_size,
           "launch": "eager" if args.eager else "hip-graph",
           "num_splits": kvq.kvq_plan_splits(layers[-1].desc, Hq,
                                             attended_rows(L, layers[-1].W, layers[-1].desc.sinks))}
    extra = {}
    if fmt in ("codec", "codec3"):
        extra["row_cosine"] = codec_row_cosine(w, fmt, layers, nl, dev)
    cpu = None if args.no_cpu_baseline else cpu_baseline_decode(w, fmt, args.cpu_seconds, L)
    names = {"mha7b-decode": "MHA-7B shape, 20K ctx, B 8", "ctx128k-int4": "128K ctx, B 1, INT4",
             "ctx128k-int8": "128K ctx, B 1, INT8 per-token",
             "gemma-codec": "Gemma-3-4B shape, WHT+Lloyd-Max codec, window 1024 x29 + global x5",
             "gemma-codec3": "Gemma-3-4B shape, WHT+Lloyd-Max 3-bit codec, window 1024 x29 + global x5",
             "llama8b-int4h": "Llama-3-8B shape, 8K ctx, B 8, INT4 with fp16 scales",
             "llama8b-sinks": "Llama-3-8B shape, 8K ctx, B 8, window 4096 + 4 sinks",
             "llama8b-recent": "Llama-3-8B shape, 8K ctx, B 8, last 128 positions in fp16",
             "llama8b-paged": "Llama-3-8B shape, 8K ctx, B 8, pages of 16 positions, shuffled block table"}
    return _line(args, f"decode step: effective KV GB/s ({names[args.workload]})", gbs, ms_step, cfg,
                 roof, cpu, dict({"tok_per_s": round(B / (ms_step * 1e-3), 1), "bytes_per_step": step_bytes,
                                  "wall_s_timed": round(wall, 4)}, **extra))


def codec_row_cosine(w, fmt, layers, nl, dev):
    """Cosine between each fp16 source row and its codec reconstruction (kvq_dequant of
    the cached codes), over the prefilled rows a window layer's ring and a global layer
    hold: layers 0 and nl - 1, K and V, every (batch, kv head)."""
    import torch
    import int4_quantized_kv_amd as kvq
    import synth
    cos = []
    for li in sorted({0, nl - 1}):
        lay = layers[li]
        k, v, _, _, _ = synth.layer_inputs(w, li, dev)
        S = w.context
        cap = lay.desc.capacity
        # (a window layer's ring slot of position S - cap now holds the appended row S)
        lo = max(0, S - cap + 1) if lay.W else 0
        for kv, src in ((0, k), (1, v)):
            out = torch.empty((w.batch, w.kv_heads, S - lo, w.head_dim), dtype=torch.float32, device=dev)
            kvq.kvq_dequant(lay.desc, lay.dc.c, kv, lo, S - lo, out)
            x = src[:, :, lo:S].double()
            y = out.double()
            cos.append(((x * y).sum(-1) / (x.norm(dim=-1) * y.norm(dim=-1))).flatten())
        del k, v
    c = torch.cat(cos)
    return {"mean": round(float(c.mean()), 5), "min": round(float(c.min()), 5), "rows": int(c.numel()),
            "layers": sorted({0, nl - 1}), "page_figure_4bit": 0.9954,
            "what": "cosine of fp16 source row vs its dequantized codec row (kvq_dequant)"}


def bench_prefill(args):
    """kvq_quantize_prefill of one MHA-7B-shaped layer (K and V [8, 32, 20480, 128] fp16
    into the INT4 cache), the same call repeated; the inputs (2.68 GB) do not fit the
    Infinity Cache, so every call streams from HBM."""
    import torch
    import int4_quantized_kv_amd as kvq
    import synth
    w = synth.WORKLOADS[3]
    dev = "cuda:0"
    B, Hkv, D, S = w.batch, w.kv_heads, w.head_dim, w.context
    desc = kvq.make_desc("int4", B, Hkv, D, S, w.group_k, w.group_v)
    dc = kvq.DeviceCache(desc, dev)
    k, v, _, _, _ = synth.layer_inputs(w, 0, dev)
    dref, cref = ctypes.byref(desc), ctypes.byref(dc.c)

    def step(stream):
        st = kvq.LIB.kvq_quantize_prefill(dref, cref, k.data_ptr(), v.data_ptr(), 0, S,
                                          ctypes.c_void_p(stream))
        if st:
            raise kvq.KvqError(st, "kvq_quantize_prefill")

    run = _runner(args, step)
    ms, wall = _timed(run, args.steps)
    rb = row_bytes("int4", D, w.group_k, w.group_v)
    nbytes = B * Hkv * S * (2 * D * 2 + rb)
    gbs = nbytes / (ms * 1e-3) / 1e9
    cfg = {"workload": w.name + "-prefill", "format": "int4", "layers_timed": 1, "batch": B,
           "kv_heads": Hkv, "head_dim": D, "positions": S, "launch": "eager" if args.eager else "hip-graph"}
    cpu = None if args.no_cpu_baseline else cpu_baseline_prefill(w, args.cpu_seconds)
    return _line(args, "prefill quantize: effective GB/s (fp16 read + codes/scales written, MHA-7B shape, 20K ctx)",
                 gbs, ms, cfg, _roofline("kvq_quantize_prefill: quant_int4_kernel", nbytes, ms * 1e3), cpu,
                 {"bytes_per_layer": nbytes, "ms_32_layers": round(32 * ms, 3), "wall_s_timed": round(wall, 4)})


def bench_dequant(args):
    """kvq_dequant of K and V (all 8192 positions) of 8 distinct Llama-3-8B-shaped layer
    caches into one fp32 buffer: 16 calls per step."""
    import torch
    import int4_quantized_kv_amd as kvq
    import synth
    w = synth.WORKLOADS[2]
    dev = "cuda:0"
    nl = args.layers or 8
    B, Hkv, D, S = w.batch, w.kv_heads, w.head_dim, w.context
    desc = kvq.make_desc("int4", B, Hkv, D, S, w.group_k, w.group_v)
    caches = []
    for li in range(nl):
        k, v, _, _, _ = synth.layer_inputs(w, li, dev)
        dc = kvq.DeviceCache(desc, dev)
        kvq.kvq_quantize_prefill(desc, dc.c, k, v, 0, S)
        del k, v
        caches.append(dc)
    out = torch.empty((B, Hkv, S, D), dtype=torch.float32, device=dev)
    dref = ctypes.byref(desc)
    crefs = [ctypes.byref(dc.c) for dc in caches]

    def step(stream):
        for cref in crefs:
            for kv in (0, 1):
                st = kvq.LIB.kvq_dequant(dref, cref, kv, 0, S, out.data_ptr(), ctypes.c_void_p(stream))
                if st:
                    raise kvq.KvqError(st, "kvq_dequant")

    run = _runner(args, step)
    ms, wall = _timed(run, args.steps)
    per_k = B * Hkv * S * (D // 2 + 4 * (D // w.group_k) + 4 * D)
    per_v = B * Hkv * S * (D // 2 + 4 * (D // w.group_v) + 4 * D)
    nbytes = nl * (per_k + per_v)
    gbs = nbytes / (ms * 1e-3) / 1e9
    cfg = {"workload": w.name + "-dequant", "format": "int4", "layer_caches": nl, "batch": B,
           "kv_heads": Hkv, "head_dim": D, "positions": S, "launch": "eager" if args.eager else "hip-graph"}
    cpu = None if args.no_cpu_baseline else cpu_baseline_dequant(w, args.cpu_seconds)
    return _line(args, "dequant: effective GB/s (codes + scales read, fp32 written; Llama-3-8B shape, 8K)",
                 gbs, ms, cfg, _roofline("kvq_dequant: dequant_int4_kernel", nbytes / (2 * nl),
                                         ms * 1e3 / (2 * nl)), cpu,
                 {"bytes_per_step": nbytes, "wall_s_timed": round(wall, 4)})


def bench_prefill_chunk(args):
    """Chunked prefill on the Llama-3-8B shape: the last 512 tokens of an 8192-token prompt
    as one chunk per layer.  A step = for each of the 32 layers (distinct caches holding
    positions 0 .. 7679), kvq_quantize_prefill of the chunk's K/V into positions
    7680 .. 8191, then kvq_prefill_attn of its 512 queries (causal).  The attention is a
    dense contraction (G * 512 query rows per cached row), so its roofline is the matrix
    cores' fp16 peak; flops are the algorithmic 4 * head_dim per (query row, attended
    position) (q.K and P.V, 2 flops per multiply-add)."""
    import torch
    import int4_quantized_kv_amd as kvq
    import synth
    w = synth.WORKLOADS[2]
    dev = "cuda:0"
    nl = args.layers or w.layers
    B, Hq, Hkv, D = w.batch, w.q_heads, w.kv_heads, w.head_dim
    NQ, L = 512, w.context
    P0 = L - NQ
    desc = kvq.make_desc("int4", B, Hkv, D, L, w.group_k, w.group_v)
    dref = ctypes.byref(desc)
    LIB = kvq.LIB
    layers = []
    for li in range(nl):
        k, v, _, _, _ = synth.layer_inputs(w, li, dev)
        lay = Layer()
        lay.dc = kvq.DeviceCache(desc, dev)
        kvq.kvq_quantize_prefill(desc, lay.dc.c, k[:, :, :P0].contiguous(), v[:, :, :P0].contiguous(), 0, P0)
        lay.kc, lay.vc = k[:, :, P0:].contiguous(), v[:, :, P0:].contiguous()
        del k, v
        lay.q = synth.query((B, Hq, NQ, D), synth.seed_of(w.wid, li, 6), dev)
        lay.out = torch.empty((B, Hq, NQ, D), dtype=torch.float32, device=dev)
        lay.cref = ctypes.byref(lay.dc.c)
        layers.append(lay)
    torch.cuda.synchronize()
    lens = (ctypes.c_int32 * B)(*([L] * B))

    def step(stream, attend_only=False):
        sp = ctypes.c_void_p(stream)
        for lay in layers:
            if not attend_only:
                st = LIB.kvq_quantize_prefill(dref, lay.cref, lay.kc.data_ptr(), lay.vc.data_ptr(), P0, NQ, sp)
                if st:
                    raise kvq.KvqError(st, "kvq_quantize_prefill")
            st = LIB.kvq_prefill_attn(dref, lay.cref, lay.q.data_ptr(), Hq, NQ, lens, 0, 0.0,
                                      lay.out.data_ptr(), sp)
            if st:
                raise kvq.KvqError(st, "kvq_prefill_attn")

    run = _runner(args, step)
    ms_step, wall = _timed(run, args.steps)
    attn = _runner(args, lambda st: step(st, attend_only=True))
    attn_ms, _ = _timed(attn, args.steps)
    pairs = B * Hq * (NQ * P0 + NQ * (NQ + 1) // 2)   # (query row, attended position) pairs
    flops = 4 * D * pairs                              # per layer
    tfs = nl * flops / (ms_step * 1e-3) / 1e12
    kern_tfs = flops / (attn_ms * 1e-3 / nl) / 1e12
    roof = {"kernel": "kvq_prefill_attn: prefill_int4_mfma_kernel", "bound": "mfma",
            "achieved": round(kern_tfs, 1), "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
            "frac": round(kern_tfs / MFMA_F16_PEAK_TFS, 4), "traffic": None,
            "flops_per_launch": flops, "avg_launch_us": round(attn_ms * 1e3 / nl, 2)}
    cfg = {"workload": w.name + "-prefill-chunk512", "format": "int4", "layers": nl, "batch": B,
           "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "chunk": NQ, "chunk_start": P0,
           "context": L, "launch": "eager" if args.eager else "hip-graph"}
    cpu = None if args.no_cpu_baseline else cpu_baseline_prefill_chunk(w, args.cpu_seconds, NQ, L)
    out = {"metric": "chunked prefill attention over the INT4 cache: TFLOP/s (Llama-3-8B shape, "
                     "512-token chunk at 8K)",
           "value": round(tfs, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f16 MFMA, f32 accumulate",
           "data": "synthetic", "config": cfg,
           "prefill_tok_per_s": round(B * NQ / (ms_step * 1e-3), 1),
           "flops_per_step": nl * flops, "wall_s_timed": round(wall, 4)}
    out["roofline"] = roof
    out["cpu_baseline"] = cpu
    return out


def cpu_baseline_prefill_chunk(w, seconds, NQ, L):
    """The oracle's prefill attention (never tuned) on one host core: one (batch, kv
    head) unit of layer 0 at a time (the G query heads' 512 chunk queries over their
    causal horizons, exact dequantization included) until `seconds` of timed work."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import synth
    from oracle import attention, quant
    G = w.q_heads // w.kv_heads
    D = w.head_dim
    k, v, _, _, _ = synth.layer_inputs(w, 0, "cuda:0")
    k, v = k.cpu().numpy(), v.cpu().numpy()
    units, dt, pairs = 0, 0.0, 0
    for b in range(w.batch):
        for h in range(w.kv_heads):
            if dt >= seconds:
                break
            q = synth.query((1, G, NQ, D), synth.seed_of(w.wid, 0, 6) + units, "cpu").numpy()
            with threadpool_limits(1):
                t0 = time.perf_counter()
                qk, sk = quant.quantize_int4(k[b, h][None, None], 64)
                qv, sv = quant.quantize_int4(v[b, h][None, None], 128)
                kh = quant.dequantize_int4_exact(qk, sk, 64)
                vh = quant.dequantize_int4_exact(qv, sv, 128)
                attention.prefill_attention(q, kh, vh, [L])
                dt += time.perf_counter() - t0
            units += 1
            pairs += G * (NQ * (L - NQ) + NQ * (NQ + 1) // 2)
    return dict({"value": round(4 * D * pairs / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                 "kind": "oracle",
                 "sample": f"{units} of layer 0's {w.batch * w.kv_heads} (batch, kv head) units "
                           f"({G} heads x {NQ} chunk queries, fp64), {dt:.2f} s timed"}, **_cpu_meta(1))


OTHER = {"mha7b-prefill": bench_prefill, "llama8b-prefill-chunk": bench_prefill_chunk, "mha7b-decode": bench_decode, "ctx128k-int4": bench_decode,
         "ctx128k-int8": bench_decode, "gemma-codec": bench_decode, "llama8b-sinks": bench_decode,
         "llama8b-recent": bench_decode, "gemma-codec3": bench_decode, "llama8b-int4h": bench_decode,
         "llama8b-paged": bench_decode,
         "dequant": bench_dequant}


def _oracle_rows(fmt, x16, gk, gv, kv):
    """Oracle quantization of rows [N, D] and their exact dequantization (fp64)."""
    from oracle import codec, quant
    if fmt in ("int4", "int4h"):
        g = gk if kv == 0 else gv
        c, s = (quant.quantize_int4 if fmt == "int4" else quant.quantize_int4_fp16_scale)(x16, g)
        return (c, s), lambda cs: quant.dequantize_int4_exact(cs[0], cs[1], g)
    if fmt == "int8":
        return quant.quantize_int8(x16), lambda cs: quant.dequantize_int8_exact(cs[0], cs[1])
    bits = 3 if fmt == "codec3" else 4
    idx, s, _ = codec.encode(x16, bits=bits)
    return (idx, s), lambda cs: codec.decode(cs[0], cs[1], bits=bits)


def cpu_baseline_decode(w, fmt, seconds, L):
    """The oracle (never tuned) on one host core, one (layer, batch, kv head) unit at a
    time until `seconds` of timed work: (append the new row,) exact dequantization of
    the attended rows, fp64 attention for the unit's query heads.  The unit's cache (the
    prefill) is quantized outside the timer."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import synth
    from oracle import attention
    G = w.q_heads // w.kv_heads
    D = w.head_dim
    rb = row_bytes(fmt, D, w.group_k, w.group_v)
    units = 0
    nbytes = 0
    dt = 0.0
    layer = 0
    while dt < seconds and layer < w.layers:
        W = w.layer_window(layer)
        ns = w.sinks if W else 0
        rows = attended_rows(L, W, ns)
        k, v, q, kn, vn = (None if t is None else t.cpu().numpy()
                           for t in synth.layer_inputs(w, layer, "cuda:0"))
        nsink = rows - min(L, W) if W else 0            # sink positions before the window
        lo = L - (rows - nsink)                         # first attended window position
        for b in range(w.batch):
            for h in range(w.kv_heads):
                if dt >= seconds:
                    break
                kr = np.concatenate([k[b, h, :nsink], k[b, h, lo:]])
                vr = np.concatenate([v[b, h, :nsink], v[b, h, lo:]])
                (kc, kdq), (vc, vdq) = _oracle_rows(fmt, kr, w.group_k, w.group_v, 0), \
                    _oracle_rows(fmt, vr, w.group_k, w.group_v, 1)
                qq = q[b, h * G:(h + 1) * G]
                with threadpool_limits(1):
                    t0 = time.perf_counter()
                    kh, vh = kdq(kc), vdq(vc)
                    if w.append:
                        (nkc, nkdq), (nvc, nvdq) = _oracle_rows(fmt, kn[b, h][None], w.group_k, w.group_v, 0), \
                            _oracle_rows(fmt, vn[b, h][None], w.group_k, w.group_v, 1)
                        kh = np.concatenate([kh, nkdq(nkc)])
                        vh = np.concatenate([vh, nvdq(nvc)])
                    if w.recent:   # the last positions are read at their fp16 values
                        k16 = np.concatenate([kr, kn[b, h][None]]) if w.append else kr
                        v16 = np.concatenate([vr, vn[b, h][None]]) if w.append else vr
                        kh = attention.recent_fp16_rows(kh[None, None], k16[None, None], [kh.shape[0]], w.recent)[0, 0]
                        vh = attention.recent_fp16_rows(vh[None, None], v16[None, None], [vh.shape[0]], w.recent)[0, 0]
                    attention.decode_attention(qq[None], kh[None, None], vh[None, None], [kh.shape[0]])
                    dt += time.perf_counter() - t0
                units += 1
                nr = min(rows, w.recent)     # rows read in fp16 (4 D bytes each)
                if w.append and nr:
                    nbytes += (rows - nr) * rb + nr * 4 * D + rb + 4 * D + G * D * 6
                else:
                    nbytes += rows * rb + G * D * 6 + (4 * D if w.append else 0)
        layer += 1
        del k, v
    full = w.batch * w.kv_heads * w.layers
    return dict({"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{units} of the step's {full} (layer, batch, kv head) units "
                      f"({'append + ' if w.append else ''}exact dequant + fp64 attention), "
                      f"{dt:.2f} s timed"}, **_cpu_meta(1))


def cpu_baseline_prefill(w, seconds):
    """The oracle's INT4 quantization of the K and V rows of one (batch, kv head) at a
    time, on one host core, until `seconds` of timed work."""
    import synth
    from threadpoolctl import threadpool_limits
    from oracle import quant
    D, S = w.head_dim, w.context
    k, v, _, _, _ = synth.layer_inputs(w, 0, "cuda:0")
    units, dt = 0, 0.0
    for b in range(w.batch):
        for h in range(w.kv_heads):
            if dt >= seconds:
                break
            kr, vr = k[b, h].cpu().numpy(), v[b, h].cpu().numpy()
            with threadpool_limits(1):
                t0 = time.perf_counter()
                quant.quantize_int4(kr, w.group_k)
                quant.quantize_int4(vr, w.group_v)
                dt += time.perf_counter() - t0
            units += 1
    nbytes = units * S * (2 * D * 2 + row_bytes("int4", D, w.group_k, w.group_v))
    return dict({"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{units} of the layer's {w.batch * w.kv_heads} (batch, kv head) units "
                      f"({S} K and V rows each), {dt:.2f} s timed"}, **_cpu_meta(1))


def cpu_baseline_dequant(w, seconds):
    """The oracle's fp32 dequantization of the K and V rows of one (batch, kv head) at a
    time, on one host core, until `seconds` of timed work."""
    import synth
    from threadpoolctl import threadpool_limits
    from oracle import quant
    D, S = w.head_dim, w.context
    k, v, _, _, _ = synth.layer_inputs(w, 0, "cuda:0")
    units, dt = 0, 0.0
    for b in range(w.batch):
        for h in range(w.kv_heads):
            if dt >= seconds:
                break
            kc, ks = quant.quantize_int4(k[b, h].cpu().numpy(), w.group_k)
            vc, vs = quant.quantize_int4(v[b, h].cpu().numpy(), w.group_v)
            with threadpool_limits(1):
                t0 = time.perf_counter()
                quant.dequantize_int4(kc, ks, w.group_k)
                quant.dequantize_int4(vc, vs, w.group_v)
                dt += time.perf_counter() - t0
            units += 1
    per = S * ((D // 2 + 4 * (D // w.group_k) + 4 * D) + (D // 2 + 4 * (D // w.group_v) + 4 * D))
    return dict({"value": round(units * per / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{units} of a layer's {w.batch * w.kv_heads} (batch, kv head) units "
                      f"({S} K and V rows each), {dt:.2f} s timed"}, **_cpu_meta(1))


if __name__ == "__main__":
    main()
