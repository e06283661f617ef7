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
# Sources of the dominant kernel (and its build flags): HBM-traffic counters recorded in
# profiles/ are reported only while these files hash to the value recorded with them.
KERNEL_SOURCES = ["int4_quantized_kv_amd/csrc/decode_mfma.hip", "int4_quantized_kv_amd/csrc/kvq_device.h",
                  "int4_quantized_kv_amd/csrc/kvq_internal.h", "int4_quantized_kv_amd/csrc/kvq_arith.h",
                  "int4_quantized_kv_amd/build.py"]
TRAFFIC_FILE = "profiles/decode_int4_mfma_llama8b_ctx8k_b8_traffic.md"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
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
                        "(attainable bandwidth; the known-size reference for the HBM counters)")
    return p.parse_args()


class Layer:
    pass


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy(args)
        return
    import int4_quantized_kv_amd as kvq
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
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

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, L)

    print(json.dumps(result), flush=True)


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the dominant kernel from the rocprofv3 FETCH_SIZE and
    WRITE_SIZE passes recorded in TRAFFIC_FILE (each scaled by the factor the same
    counter shows on a copy of known size), or None if there is no record or the kernel
    has changed since it was taken."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        line = line.strip().strip("`")
        if ":" in line and line.split(":", 1)[0] in ("source_sha256", "traffic_bytes_per_launch"):
            k, v = line.split(":", 1)
            rec[k] = v.strip()
    if rec.get("source_sha256") != kernel_source_hash() or "traffic_bytes_per_launch" not in rec:
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


def cpu_baseline(w, seconds, L):
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
    return {"value": round(units * unit_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{units} of the step's {full} (layer, batch, kv head) units "
                      f"(append + exact dequant + fp64 attention over {L} positions), "
                      f"{dt:.2f} s timed; a full step extrapolates to {dt * full / units:.1f} s"}


if __name__ == "__main__":
    main()
