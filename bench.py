"""Benchmark of the fused MXFP4 MoE decode layer on one MI355X.

One step = one call of fused_moe_mxfp4_decode (router, top-k, MXFP4 routed
experts, MXFP8 shared expert and combine in one launch) on the 1-row decode
workload: T=1, H=3072, 128 experts top-4, I=1024, shared expert I_s=1024.
Weights rotate over --rotate distinct layer instances (full expert sets, each
653 MB) and every step reads a different input row, so the routed weights a
step touches are not served from the 256 MB last-level cache.  The 16-row
workload is measured the same way and reported beside it.

Prints one JSON line.  `value` is the device time per launch over the timed
region: K launches issued back to back on one stream (as a decode step issues
its layers), bracketed by a synchronize and HIP events recorded on that
stream, divided by K; `ms_per_step` is the wall-clock time per step over the
same region.  Every rotated layer instance is launched once before the timed
region (plus the requested warm-up launches), so no timed launch is the first
on its weights.  The same launches timed one at a time (an event pair around
each, so every launch starts on an idle GPU) are reported beside it as
`us_isolated_*`.  Beside the 1-row line: the 16-row workload, the 8-layer
4-row chain replayed from a captured HIP graph (us per layer), and the
8192-row grouped path with each launch step timed by events (routed FP4
GEMMs against the FP4 matrix peak, shared FP8 GEMMs against the FP8 peak).
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP4_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 matrix peak (published)


def layer_bytes(H, I, E, Is, D, T, residual=False, folded=False):
    """Algorithmic HBM bytes of one layer call: router weights, D routed
    experts (W13 + W2 codes and scales), the shared expert (MXFP8; folded: one
    more MXFP4 expert of the table), x, y (+ residual)."""
    routed = 3 * I * H * 17 // 32
    shared = routed if folded else 3 * Is * H * 33 // 32
    return E * H * 4 + D * routed + shared + (3 if residual else 2) * T * H * 2


def kernel_source_hash():
    h = hashlib.sha256()
    for name in ("decode.hip", "mx_device.h"):
        with open(os.path.join(ROOT, "mxfp4_moe_decode_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    entry = rec.get(workload)
    if not entry or entry.get("kernel_hash") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def build_layers(binding, synth, name, count, fold=False):
    import torch
    cfg = synth.workload(name)
    layers = []
    for li in range(count):
        layers.append(binding.MoELayer.from_fp32(
            cfg["H"], cfg["I"], cfg["E"], cfg["k"], cfg["I_s"], synth.router_weights(cfg, li),
            synth.router_bias(cfg, li), lambda e, li=li: synth.device_expert_w13(cfg, li, e),
            lambda e, li=li: synth.device_expert_w2(cfg, li, e),
            synth.device_shared_w13(cfg, li), synth.device_shared_w2(cfg, li), fold_shared=fold))
    torch.cuda.synchronize()
    return cfg, layers


def time_decode(binding, synth, name, rotate, steps, warmup, pool=64, isolated=True, fold=False, norm=False,
                rows=None, grouped=False):
    """Fused launches of the workload (``rows`` overrides its row count); with
    ``grouped``, the grouped path on the same layers and inputs instead."""
    import torch
    cfg, layers = build_layers(binding, synth, name, rotate, fold)
    if rows is not None:
        cfg = dict(cfg, T=rows)
    if norm:  # the pre-router RMSNorm fused in: the input is the residual stream
        gamma = torch.from_numpy(synth.norm_weight(cfg)).cuda()
        layers = [L.with_norm(gamma) for L in layers]
    T = cfg["T"]
    xs = [torch.from_numpy(synth.activations(cfg, T=T, index=j).view(np.int16)).cuda().view(torch.bfloat16)
          for j in range(pool)]
    ws = binding.decode_workspace(layers[0])
    ys = [torch.empty_like(xs[0]) for _ in range(4)]
    ids = torch.empty(steps, T, cfg["k"], dtype=torch.int32, device="cuda")
    w = torch.empty(steps, T, cfg["k"], dtype=torch.float32, device="cuda")
    lib = binding.load()
    stream = torch.cuda.current_stream()
    sp = binding.ctypes.c_void_p(stream.cuda_stream)

    gws = binding.grouped_workspace(layers[0], T) if grouped else None

    def launch(i, rec_ids=None, rec_w=None):
        L = layers[i % rotate]
        if grouped:
            st = lib.fused_moe_mxfp4_grouped(L.c, binding._ptr(xs[i % pool]), T, None, binding._ptr(ys[i % 4]),
                                             binding._ptr(gws), gws.numel(), sp)
        else:
            st = lib.fused_moe_mxfp4_decode(L.c, binding._ptr(xs[i % pool]), T, None, binding._ptr(ys[i % 4]),
                                            binding._ptr(ws), ws.numel(), binding._ptr(rec_ids),
                                            binding._ptr(rec_w), sp)
        if st != 0:
            raise binding.MoeError("layer call", st)

    # every rotated instance is touched once before timing (its first launch
    # pays first-touch costs the steady state does not), then `warmup` more
    for i in range(rotate):
        launch(i)
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    # timed region: `steps` launches back to back, bracketed by synchronize
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    b0.record(stream)
    for i in range(steps):
        launch(warmup + i, ids[i], w[i])
    b1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us_launch = b0.elapsed_time(b1) * 1e3 / steps
    # the same kind of launches one at a time: an event pair around each
    iso = np.full(1, np.nan)
    if isolated:
        ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            ev0[i].record(stream)
            launch(warmup + steps + i)
            ev1[i].record(stream)
        torch.cuda.synchronize()
        iso = np.array([a.elapsed_time(b) for a, b in zip(ev0, ev1)]) * 1e3
    if binding.moe_decode_status(ws) != 0:
        raise RuntimeError("a device-side wait timed out during the benchmark")
    if grouped:  # the routing of the timed steps, for the byte count (outside the timed region)
        for i in range(steps):
            L, xi = layers[(warmup + i) % rotate], xs[(warmup + i) % pool]
            if lib.moe_router_topk(L.c, binding._ptr(xi), T, None, binding._ptr(ids[i]), binding._ptr(w[i]), sp):
                raise binding.MoeError("moe_router_topk", -4)
        torch.cuda.synchronize()
    ids_np = ids.cpu().numpy()
    D = np.array([len(np.unique(ids_np[i])) for i in range(steps)])
    nbytes = np.array([layer_bytes(cfg["H"], cfg["I"], cfg["E"], cfg["I_s"], d, T, folded=fold) +
                       (cfg["H"] * 4 if norm else 0) for d in D])
    del layers
    torch.cuda.empty_cache()
    return {
        "cfg": cfg, "us_launch": float(us_launch), "wall_ms_per_step": wall / steps * 1e3,
        "bytes_mean": float(nbytes.mean()), "gbs": float(nbytes.mean() / (us_launch * 1e-6) / 1e9),
        "distinct_experts_mean": float(D.mean()),
        "us_isolated_mean": float(iso.mean()), "us_isolated_median": float(np.median(iso)),
        "us_isolated_p10": float(np.percentile(iso, 10)), "us_isolated_p90": float(np.percentile(iso, 90)),
    }


def prefill_flops(T, H, I, E, k, Is):
    """Algorithmic FLOPs of the 8192-row layer: routed gate/up + down (MXFP4),
    shared gate/up + down (MXFP8), router (fp32)."""
    routed = 2 * T * k * 3 * I * H
    shared = 2 * T * 3 * Is * H
    router = 2 * T * E * H
    return routed, shared, router


FP8_PEAK_TFLOPS = 5000.0   # MI355X dense MXFP8 matrix peak (published)
FP32_PEAK_TFLOPS = 157.3   # MI355X fp32 vector peak (published)


def time_grouped(binding, synth, steps=10, warmup=30):
    """The grouped path on the 8192-row prefill workload: whole-layer time of
    the plain call (the quantization and the shared gate/up on the library's
    side stream), and each launch step timed with HIP events recorded between
    the steps of the timed call, which runs them all in order on one stream."""
    import torch
    cfg, layers = build_layers(binding, synth, "prefill", 1)
    L = layers[0]
    x = torch.from_numpy(synth.activations(cfg).view(np.int16)).cuda().view(torch.bfloat16)
    y = torch.empty_like(x)
    ws = binding.grouped_workspace(L, cfg["T"])
    # the first ~20 calls after the layer's set-up run up to 10% slower (the
    # GPU leaving its idle clocks): 30 untimed calls first
    for _ in range(warmup):
        binding.fused_moe_mxfp4_grouped(L, x, out=y, workspace=ws)
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record()
    for i in range(steps):
        binding.fused_moe_mxfp4_grouped(L, x, out=y, workspace=ws)
        marks[i + 1].record()
    torch.cuda.synchronize()
    us = np.array([marks[i].elapsed_time(marks[i + 1]) * 1e3 for i in range(steps)])
    runs = []
    for _ in range(steps):
        _, ev = binding.fused_moe_mxfp4_grouped_timed(L, x, out=y, workspace=ws)
        runs.append(ev)
    torch.cuda.synchronize()
    step_us = np.array([[ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(len(ev) - 1)] for ev in runs])
    us_serial = np.array([ev[0].elapsed_time(ev[-1]) * 1e3 for ev in runs])
    routed, shared, router = prefill_flops(cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["k"], cfg["I_s"])
    del layers, L, ws
    torch.cuda.empty_cache()
    st = dict(zip(binding.GROUPED_STEPS, step_us.mean(axis=0)))
    gu, dn = st["routed_gate_up"], st["routed_down"]
    sgu, sdn = st["shared_gate_up"], st["shared_down_combine"]
    # routed: gate/up is 2/3 of the FLOPs, down 1/3 (2 I H and I H per slot)
    return {"us_mean": float(us.mean()), "us_median": float(np.median(us)),
            "us_mean_one_stream": float(us_serial.mean()),
            "step_us": {k: round(float(v), 2) for k, v in st.items()},
            "routed_fp4": {"us": round(gu + dn, 2), "tflops": routed / ((gu + dn) * 1e-6) / 1e12,
                           "gate_up_tflops": routed * 2 / 3 / (gu * 1e-6) / 1e12,
                           "down_tflops": routed / 3 / (dn * 1e-6) / 1e12},
            "shared_fp8": {"us": round(sgu + sdn, 2), "tflops": shared / ((sgu + sdn) * 1e-6) / 1e12},
            "router_fp32": {"us": round(st["router"], 2), "tflops": router / (st["router"] * 1e-6) / 1e12},
            "gflop_routed": routed / 1e9, "gflop_shared": shared / 1e9, "gflop_router": router / 1e9}


def time_chain(binding, synth, replays=20):
    """The 8-layer decode chain (4 rows, Zipf-biased routers, residual):
    8 fused launches, each reading the previous layer's output, captured once
    into a HIP graph and replayed.  Each replay starts on a new input row set
    (copied into the graph's input buffer before its start event)."""
    import torch
    cfg = synth.workload("chain8")
    nl, T = cfg["layers"], cfg["T"]
    layers = [binding.MoELayer.from_fp32(
        cfg["H"], cfg["I"], cfg["E"], cfg["k"], cfg["I_s"], synth.router_weights(cfg, li),
        synth.router_bias(cfg, li), lambda e, li=li: synth.device_expert_w13(cfg, li, e),
        lambda e, li=li: synth.device_expert_w2(cfg, li, e),
        synth.device_shared_w13(cfg, li), synth.device_shared_w2(cfg, li)) for li in range(nl)]
    xs = [torch.from_numpy(synth.activations(cfg, index=j).view(np.int16)).cuda().view(torch.bfloat16)
          for j in range(replays + 1)]
    ws = binding.decode_workspace(layers[0])
    bufs = [torch.empty_like(xs[0]) for _ in range(nl + 1)]
    ids = [torch.empty(T, cfg["k"], dtype=torch.int32, device="cuda") for _ in range(nl)]
    wts = [torch.empty(T, cfg["k"], dtype=torch.float32, device="cuda") for _ in range(nl)]
    lib = binding.load()

    def chain():
        sp = binding._stream()
        for li in range(nl):
            st = lib.fused_moe_mxfp4_decode(layers[li].c, binding._ptr(bufs[li]), T, binding._ptr(bufs[li]),
                                            binding._ptr(bufs[li + 1]), binding._ptr(ws), ws.numel(),
                                            binding._ptr(ids[li]), binding._ptr(wts[li]), sp)
            if st != 0:
                raise binding.MoeError("fused_moe_mxfp4_decode", st)

    bufs[0].copy_(xs[-1])
    chain()  # eager once: first touch of every layer
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain()
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    D = np.zeros((replays, nl))
    for r in range(replays):
        bufs[0].copy_(xs[r])
        ev[r][0].record(stream)
        graph.replay()
        ev[r][1].record(stream)
        torch.cuda.synchronize()
        D[r] = [len(np.unique(i.cpu().numpy())) for i in ids]
    us = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
    if binding.moe_decode_status(ws) != 0:
        raise RuntimeError("a device-side wait timed out during the chain benchmark")
    nbytes = np.array([[layer_bytes(cfg["H"], cfg["I"], cfg["E"], cfg["I_s"], d, T, residual=True) for d in row]
                       for row in D])
    del layers, graph
    torch.cuda.empty_cache()
    per_layer = float(np.median(us)) / nl
    gbs = float(nbytes.sum(axis=1).mean()) / (np.median(us) * 1e-6) / 1e9
    return {"us_per_layer": per_layer, "us_replay_median": float(np.median(us)),
            "us_replay_p10": float(np.percentile(us, 10)), "us_replay_p90": float(np.percentile(us, 90)),
            "distinct_experts_per_layer": [round(float(v), 2) for v in D.mean(axis=0)],
            "bytes_per_layer_mean": float(nbytes.mean()), "gbs": gbs}


def cpu_baseline(synth, seconds=15.0):
    """The oracle, as it stands, on a bounded sample of the 1-row workload."""
    import torch
    from oracle import moe, mx
    from threadpoolctl import threadpool_info

    cfg = synth.workload("decode1")
    layer = 0
    x_all = [synth.activations(cfg, T=1, index=j) for j in range(64)]
    wr = synth.router_weights(cfg, layer)
    # quantize (outside the timed region) the experts the sample rows use
    cache13, cache2 = {}, {}

    def q13(e):
        if e not in cache13:
            cache13[e] = mx.mx_quantize(synth.device_expert_w13(cfg, layer, e).cpu().numpy().astype(np.float64), "fp4")
        return cache13[e]

    def q2(e):
        if e not in cache2:
            cache2[e] = mx.mx_quantize(synth.device_expert_w2(cfg, layer, e).cpu().numpy().astype(np.float64), "fp4")
        return cache2[e]

    class P:
        def __init__(self, f, i):
            self.f, self.i = f, i

        def __getitem__(self, e):
            return self.f(int(e))[self.i]

    sc13, ss13 = mx.mx_quantize(synth.device_shared_w13(cfg, layer).cpu().numpy().astype(np.float64), "fp8")
    sc2, ss2 = mx.mx_quantize(synth.device_shared_w2(cfg, layer).cpu().numpy().astype(np.float64), "fp8")
    L = moe.Layer(cfg["H"], cfg["I"], cfg["E"], cfg["k"], cfg["I_s"], wr, None,
                  P(q13, 0), P(q13, 1), P(q2, 0), P(q2, 1), sc13, ss13, sc2, ss2)
    n_rows = 0
    # warm the expert cache for the rows the sample will use
    for x in x_all[:8]:
        ids, _ = moe.select_topk(moe.router_logits(mx.bf16_bits_to_f64(x), wr), cfg["k"])
        for e in ids.reshape(-1):
            q13(int(e)), q2(int(e))
    t0 = time.perf_counter()
    while True:
        moe.moe_layer(x_all[n_rows % 8], L)
        n_rows += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": el / n_rows * 1e6, "unit": "us", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_rows} calls of the fp64 oracle layer on the 1-row workload "
                      f"(T=1, H=3072, 128 experts top-4, I=1024, MXFP8 shared I_s=1024), "
                      f"8 distinct input rows, weights pre-quantized"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=16, help="distinct layer instances cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-16", action="store_true", help="skip the 16-row measurement")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 8192-row grouped measurement")
    ap.add_argument("--no-chain", action="store_true", help="skip the 8-layer graph-replayed chain")
    ap.add_argument("--no-folded", action="store_true",
                    help="skip the layers with the shared expert folded into the table as an MXFP4 expert")
    ap.add_argument("--no-norm", action="store_true", help="skip the layers with the pre-router RMSNorm fused in")
    ap.add_argument("--no-wide", action="store_true", help="skip the 64-row step (wide fused launch vs grouped)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-isolated", action="store_true",
                    help="skip the one-launch-at-a-time timing (profiler runs: only back-to-back launches)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the measurement, run 5 plain elementwise copies (torch.neg, fp32) of this "
                         "many MiB: a kernel of known traffic that calibrates the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is built and measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch
    from mxfp4_moe_decode_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load()
    r1 = time_decode(binding, synth, "decode1", args.rotate, args.steps, args.warmup,
                     isolated=not args.no_isolated)
    print(f"[bench] 1 row: {r1['us_launch']:.2f} us per launch back to back ({r1['gbs']:.0f} GB/s); "
          f"isolated launches {r1['us_isolated_mean']:.2f} us mean", file=sys.stderr, flush=True)
    r16 = None
    if not args.no_16:
        r16 = time_decode(binding, synth, "decode16", max(4, args.rotate // 2), args.steps, args.warmup,
                          isolated=not args.no_isolated)
        print(f"[bench] 16 rows: {r16['us_launch']:.2f} us per launch back to back, {r16['gbs']:.0f} GB/s, "
              f"D={r16['distinct_experts_mean']:.1f}; isolated {r16['us_isolated_mean']:.2f} us",
              file=sys.stderr, flush=True)
    rf = {}
    if not args.no_folded:
        for name, label in (("decode1", "1 row"), ("decode16", "16 rows")):
            if name == "decode16" and args.no_16:
                continue
            rf[name] = time_decode(binding, synth, name, max(4, args.rotate // 2), args.steps, args.warmup,
                                   isolated=False, fold=True)
            print(f"[bench] {label}, shared expert folded (MXFP4 expert 128): {rf[name]['us_launch']:.2f} us per "
                  f"launch, {rf[name]['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    rn = {}
    if not args.no_norm:
        for name, label in (("decode1", "1 row"), ("decode16", "16 rows")):
            if name == "decode16" and args.no_16:
                continue
            rn[name] = time_decode(binding, synth, name, max(4, args.rotate // 2), args.steps, args.warmup,
                                   isolated=False, norm=True)
            print(f"[bench] {label}, pre-router RMSNorm fused in: {rn[name]['us_launch']:.2f} us per launch, "
                  f"{rn[name]['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    rw = {}
    if not args.no_wide:
        for kind in ("fused", "grouped"):
            rw[kind] = time_decode(binding, synth, "decode16", max(4, args.rotate // 2), max(20, args.steps // 4),
                                   args.warmup, isolated=False, rows=64, grouped=kind == "grouped")
            print(f"[bench] 64 rows, {kind}: {rw[kind]['us_launch']:.2f} us per step, {rw[kind]['gbs']:.0f} GB/s, "
                  f"D={rw[kind]['distinct_experts_mean']:.1f}", file=sys.stderr, flush=True)
    rc = None
    if not args.no_chain:
        rc = time_chain(binding, synth)
        print(f"[bench] 8-layer chain, 4 rows, graph replay: {rc['us_per_layer']:.2f} us per layer, "
              f"{rc['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    rp = None
    if not args.no_prefill:
        rp = time_grouped(binding, synth)
        print(f"[bench] prefill 8192 rows (grouped path): {rp['us_mean']:.1f} us per layer "
              f"({rp['us_mean_one_stream']:.1f} us with every step on one stream); routed FP4 GEMMs "
              f"{rp['routed_fp4']['us']:.1f} us ({rp['routed_fp4']['tflops']:.0f} TFLOP/s), shared FP8 "
              f"{rp['shared_fp8']['us']:.1f} us", file=sys.stderr, flush=True)
    if args.copy_mib:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 5 x torch.neg over {args.copy_mib} MiB fp32 "
              f"(each reads and writes {args.copy_mib << 20} bytes)", file=sys.stderr, flush=True)
        del src, dst
    cpu = None if args.no_cpu_baseline else cpu_baseline(synth, args.cpu_seconds)

    traffic = load_traffic("decode1")
    out = {
        "metric": "fused MXFP4 MoE layer us at 1/16 rows; achieved HBM GB/s and % roofline",
        "value": round(r1["us_launch"], 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r1["wall_ms_per_step"], 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 (E2M1 x E8M0 routed, E4M3 x E8M0 shared, fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": "decode1: 1 bf16 row, hidden 3072, 128 MXFP4 experts top-4, "
                               "intermediate 1024, MXFP8 shared expert 1024, one launch per layer",
                   "rows": 1, "hidden": 3072, "experts": 128, "top_k": 4, "inter": 1024,
                   "shared_inter": 1024, "rotated_layer_instances": args.rotate},
        "us_isolated_mean": round(r1["us_isolated_mean"], 3),
        "us_isolated_median": round(r1["us_isolated_median"], 3),
        "us_isolated_p10": round(r1["us_isolated_p10"], 3),
        "us_isolated_p90": round(r1["us_isolated_p90"], 3),
        "roofline": {"bound": "hbm", "achieved": round(r1["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(r1["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(r1["bytes_mean"])},
    }
    if r16:
        out["rows16"] = {"us_per_launch": round(r16["us_launch"], 3),
                         "gbs": round(r16["gbs"], 1), "frac": round(r16["gbs"] / HBM_PEAK_GBS, 4),
                         "traffic": load_traffic("decode16"),
                         "distinct_experts_mean": round(r16["distinct_experts_mean"], 2),
                         "us_isolated_mean": round(r16["us_isolated_mean"], 3),
                         "algorithmic_bytes_per_launch": int(r16["bytes_mean"]),
                         "ms_per_step": round(r16["wall_ms_per_step"], 5)}
    if rf:
        out["folded_shared"] = {
            "workload": "the same layers with the MXFP8 shared expert re-quantized to MXFP4 and folded into the "
                        "expert table as expert 128 (every row selects it with weight 1)",
            **{("rows1" if n == "decode1" else "rows16"): {
                "us_per_launch": round(r["us_launch"], 3), "gbs": round(r["gbs"], 1),
                "frac": round(r["gbs"] / HBM_PEAK_GBS, 4), "distinct_routed_experts_mean":
                round(r["distinct_experts_mean"], 2), "algorithmic_bytes_per_launch": int(r["bytes_mean"])}
               for n, r in rf.items()}}
    if rn:
        out["fused_norm"] = {
            "workload": "the same layers with the pre-router RMSNorm fused into the launch (input = residual "
                        "stream h, MoE on RMSNorm(h), h added back)",
            **{("rows1" if n == "decode1" else "rows16"): {
                "us_per_launch": round(r["us_launch"], 3), "gbs": round(r["gbs"], 1),
                "frac": round(r["gbs"] / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": int(r["bytes_mean"])}
               for n, r in rn.items()}}
    if rw:
        out["rows64"] = {
            "workload": "a 64-row step on the 16-row workload's layer (speculative decoding at 8-16 users): one "
                        "wide fused launch, against the grouped path's launches (the timing of the latter "
                        "includes a router call to record the routing)",
            **{kind: {"us_per_step": round(r["us_launch"], 3), "gbs": round(r["gbs"], 1),
                      "frac": round(r["gbs"] / HBM_PEAK_GBS, 4),
                      "distinct_experts_mean": round(r["distinct_experts_mean"], 2),
                      "algorithmic_bytes_per_step": int(r["bytes_mean"])} for kind, r in rw.items()}}
    if rc:
        out["chain8"] = {
            "workload": "8 distinct layers (hidden 3072, 128 experts top-4, I 1024, MXFP8 shared 1024), 4 rows, "
                        "Zipf(1.2)-biased routers, fused residual; one launch per layer, 8 launches captured "
                        "in a HIP graph and replayed",
            "us_per_layer": round(rc["us_per_layer"], 3), "us_replay_median": round(rc["us_replay_median"], 2),
            "us_replay_p10": round(rc["us_replay_p10"], 2), "us_replay_p90": round(rc["us_replay_p90"], 2),
            "distinct_experts_per_layer": rc["distinct_experts_per_layer"],
            "algorithmic_bytes_per_layer": int(rc["bytes_per_layer_mean"]),
            "gbs": round(rc["gbs"], 1), "frac": round(rc["gbs"] / HBM_PEAK_GBS, 4)}
    if rp:
        out["prefill8192"] = {
            "workload": "8192 bf16 rows through the same layer on the grouped path (router, sort, MX quant, "
                        "grouped FP4 GEMMs, MXFP8 shared expert, combine)",
            "us_mean": round(rp["us_mean"], 2), "us_median": round(rp["us_median"], 2),
            "us_mean_one_stream": round(rp["us_mean_one_stream"], 2),
            "step_us": rp["step_us"],
            "gflop": {"routed_fp4": round(rp["gflop_routed"], 1), "shared_fp8": round(rp["gflop_shared"], 1),
                      "router_fp32": round(rp["gflop_router"], 2)},
            "routed_fp4_gemms": {"us": rp["routed_fp4"]["us"], "tflops": round(rp["routed_fp4"]["tflops"], 1),
                                 "peak_tflops": FP4_PEAK_TFLOPS,
                                 "frac": round(rp["routed_fp4"]["tflops"] / FP4_PEAK_TFLOPS, 4),
                                 "gate_up_frac": round(rp["routed_fp4"]["gate_up_tflops"] / FP4_PEAK_TFLOPS, 4),
                                 "down_frac": round(rp["routed_fp4"]["down_tflops"] / FP4_PEAK_TFLOPS, 4)},
            "shared_fp8_gemms": {"us": rp["shared_fp8"]["us"], "tflops": round(rp["shared_fp8"]["tflops"], 1),
                                 "peak_tflops": FP8_PEAK_TFLOPS,
                                 "frac": round(rp["shared_fp8"]["tflops"] / FP8_PEAK_TFLOPS, 4)},
            "router_fp32": {"us": rp["router_fp32"]["us"], "tflops": round(rp["router_fp32"]["tflops"], 2),
                            "peak_tflops": FP32_PEAK_TFLOPS,
                            "frac": round(rp["router_fp32"]["tflops"] / FP32_PEAK_TFLOPS, 4)}}
    out["cpu_baseline"] = cpu
    print(json.dumps(out))


if __name__ == "__main__":
    main()
