#!/usr/bin/env python3
"""Decode-step benchmark of the INT4 KV-cache path on one MI355X.

Workload (the headline): Llama-3-8B-shaped decode, 32 layers, 32 query heads over 8 KV
heads (GQA 4:1), head_dim 128, batch 8, 8192 cached positions per sequence.  One step =
for every layer: kvq_append (quantize the new token's K/V into slot 8192) then
kvq_decode_attn over the 8193 positions (split-K kernel + merge kernel).  The 32 layers
have distinct caches (2.36 GB of packed K/V in total), so the 256 MB Infinity Cache
cannot serve a step.  Inputs are seeded synthetic fp16 N(0,1) K/V with 3 of 128
channels x20 (synth.py), quantized into the caches before timing.

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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=None, help="override the layer count (debug only)")
    p.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-units", type=int, default=8,
                   help="(batch, kv head) units of one layer the CPU oracle is timed on")
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
    ws_bytes = kvq.kvq_decode_workspace_bytes(desc, Hq, L)
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device=dev)
    nsplit = kvq.kvq_plan_splits(desc, Hq, L)
    LIB = kvq.LIB

    def step(stream, append=True, attend=True):
        sp = ctypes.c_void_p(stream)
        for lay in layers:
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
        if not torch.equal(layers[-1].out, eager_out):
            raise RuntimeError("graph replay differs from the eager result")

    # ---- timed region: exactly K steps, synchronized on both sides
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

    # ---- dominant kernel: kvq_decode_attn alone (split-K + merge), all layers, graph
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
    attn_ms = e0.elapsed_time(e1) / (args.steps * nl)

    # ---- algorithmic bytes
    row_bytes = (D // 2 + 4 * (D // w.group_k)) + (D // 2 + 4 * (D // w.group_v))  # K + V, 140 B
    cache_read = B * Hkv * L * row_bytes
    q_bytes = B * Hq * D * 2
    out_bytes = B * Hq * D * 4
    append_bytes = B * Hkv * D * 2 * 2 + B * Hkv * row_bytes
    attn_bytes = cache_read + q_bytes + out_bytes
    step_bytes = nl * (attn_bytes + append_bytes)
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    attn_gbs = attn_bytes / (attn_ms * 1e-3) / 1e9

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
                   "launch": "eager" if args.eager else "hip-graph", "num_splits": nsplit},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tok_per_s": round(B / (ms_step * 1e-3), 1),
        "bytes_per_step": step_bytes,
        "wall_s_timed": round(wall_s, 4),
        "roofline": {
            "kernel": "kvq_decode_attn (decode_splitk_kernel + merge_kernel)",
            "bound": "hbm",
            "achieved": round(attn_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
            "traffic": None,
            "bytes_per_launch": attn_bytes,
            "avg_launch_us": round(attn_ms * 1e3, 2),
        },
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, layers[0], desc, args.cpu_units, L)

    print(json.dumps(result), flush=True)


def cpu_baseline(w, lay, desc, units, L):
    """The oracle (never tuned) timed on host cores for `units` (batch, kv head) pairs of
    one layer's decode step: quantize the new row, dequantize the cache exactly, fp64
    softmax attention for the pair's G query heads.  Single-threaded BLAS."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import synth
    from oracle import attention, quant

    S = w.context
    G = w.q_heads // w.kv_heads
    k, v, q, kn, vn = synth.layer_inputs(w, 0, "cuda:0")
    pairs = [(b, h) for b in range(w.batch) for h in range(w.kv_heads)][:units]
    kk = [k[b, h].cpu().numpy() for b, h in pairs]
    vv = [v[b, h].cpu().numpy() for b, h in pairs]
    qq = [q[b, h * G:(h + 1) * G].cpu().numpy() for b, h in pairs]
    kr = [kn[b, h].cpu().numpy() for b, h in pairs]
    vr = [vn[b, h].cpu().numpy() for b, h in pairs]
    del k, v
    # the cache state the step starts from (prefill, not timed)
    pre = [(quant.quantize_int4(a, 64), quant.quantize_int4(b_, 128)) for a, b_ in zip(kk, vv)]
    with threadpool_limits(1):
        t0 = time.perf_counter()
        for i in range(len(pairs)):
            (ck, sk), (cv, sv) = pre[i]
            nk, nsk = quant.quantize_int4(kr[i][None], 64)         # append the new row
            nv, nsv = quant.quantize_int4(vr[i][None], 128)
            ck = np.concatenate([ck, nk]); sk = np.concatenate([sk, nsk])
            cv = np.concatenate([cv, nv]); sv = np.concatenate([sv, nsv])
            kh = quant.dequantize_int4_exact(ck, sk, 64)
            vh = quant.dequantize_int4_exact(cv, sv, 128)
            attention.decode_attention(qq[i][None], kh[None, None], vh[None, None], [L])
        dt = time.perf_counter() - t0
    row = 140
    bytes_sample = len(pairs) * (L * row + G * 128 * 2 + G * 128 * 4)
    return {"value": round(bytes_sample / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(pairs)} of {w.batch * w.kv_heads} (batch, kv head) units of 1 of "
                      f"{w.layers} layers (append + exact dequant + fp64 attention), "
                      f"{dt:.2f} s; full step extrapolates to {dt * w.batch * w.kv_heads / len(pairs) * w.layers:.1f} s"}


if __name__ == "__main__":
    main()
