#!/usr/bin/env python3
"""Benchmark of the routed-expert MXFP4 MoE FFN hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
resident in HBM: per-32 int8 activation quantisation, top-k routing + expert
grouping, gate/up projection + SwiGLU + requant, down projection, weighted
combine.  Layer weight sets are rotated per step so the MALL (256 MB) cannot
hold them.  Prints one JSON line.

Workloads (--workload):
  decode        DS-V4 layer (256 experts, top-6 + shared, D 4096, F 2048),
                1 token per step, 8 layer sets (27.5 GB)            [default]
  decode-batch  same layer, --rows 2/4/8/16 tokens per step (--hot: +2.0 logit
                bias on 16 experts)
  prefill       same layer, --rows 512 or 4096 tokens per step, 2 layer sets
  matvec        MXFP4 matvec 14336x4096, --rows K resident rows, 16 copies
  copy          calibration only: a plain 1 GiB device-to-device copy (torch),
                the known-size reference for HBM byte counters
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-FFN tokens/s + achieved HBM GB/s (decode 1-16 rows), TFLOP/s (prefill)"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0

# HBM bytes per launch of each workload's dominant kernel, from rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) on the native counters driver
# replaying this benchmark's own inputs (profiles/hbm_traffic_counters.md),
# scaled by the plain-copy calibration: read = 2 x FETCH_SIZE, written =
# WRITE_SIZE.  Valid only for the kernel sources they were taken with (hash
# below, over the device code in csrc/): after any change to it the benchmark
# reports traffic as null.
TRAFFIC_SRC = "2d236613a72e4058"
TRAFFIC = {  # (workload, rows[, variant]): (read bytes, written bytes)
    ("decode", 1): (2 * 30777.0 * 1024, 48.6 * 1024),
    ("decode-batch", 16): (2 * 349734.1 * 1024, 687.7 * 1024),
    ("decode-batch", 16, "hot"): (2 * 171023.99 * 1024, 676.9 * 1024),
    ("prefill", 4096): (2 * 1346555.0 * 1024, 146336.0 * 1024),
    ("prefill", 512): (2 * 1179207.25 * 1024, 15348.6 * 1024),
    ("matvec", 5): (2 * 15404.8 * 1024, 280.0 * 1024),
}


def kernel_sources_hash():
    """Hash of the device code (csrc/*.hip and *.h; host-only .cpp excluded)."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mxfp4_routed_expert_e2m1_amd",
                     "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if not f.endswith((".hip", ".h")):
            continue
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(key):
    """Counted HBM bytes per launch for this workload, or None (not counted,
    or the kernels changed since)."""
    if key not in TRAFFIC or kernel_sources_hash() != TRAFFIC_SRC:
        return None
    r, w = TRAFFIC[key]
    return int(r + w)
I8_MFMA_PEAK_TOPS = 5000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "decode-batch", "prefill", "matvec", "copy"])
    ap.add_argument("--rows", type=int, default=None)
    ap.add_argument("--hot", action="store_true")
    ap.add_argument("--shard", choices=["tp8"], default=None,
                    help="one GPU's share of a tensor-parallel layer: d_ff split 8 ways "
                         "(256 features per expert), the same experts and routes")
    ap.add_argument("--router", action="store_true",
                    help="start each step from the hidden state: the router projection "
                         "(BF16 weights) computes the logits inside the step")
    ap.add_argument("--sets", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=None)
    ap.add_argument("--out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--dump-inputs", default=None, metavar="DIR",
                    help="write the input of the kernel-timing step (x.f32, logits.f32) "
                         "for the native counters driver, then exit")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step eagerly instead of replaying HIP graphs (for "
                         "counter profilers that cannot follow graph launches); the timings "
                         "then include host launch gaps")
    return ap.parse_args()


def main():
    args = parse()
    global EAGER
    EAGER = args.eager
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the routed-expert path here has no "
              "multi-GPU execution (no collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mxfp4_routed_expert_e2m1_amd as m
    import synth

    m.lib()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    wl = args.workload
    if wl == "matvec":
        return bench_matvec(args, m, synth, np, torch, dev)
    if wl == "copy":
        return bench_copy(args, torch, dev)

    L = synth.DSV4_LAYER
    if args.shard == "tp8":
        L = synth.Layer(n_experts=L.n_experts, top_k=L.top_k, d_model=L.d_model,
                        d_ff=L.d_ff // 8, has_shared=L.has_shared)
    if wl == "decode":
        T, seed, sets = 1, synth.DECODE["seed"], 8
    elif wl == "decode-batch":
        T, seed, sets = (args.rows or 16), synth.DECODE_BATCH["seed"], 8
    else:
        T, seed, sets = (args.rows or 4096), synth.PREFILL["seed"], 2
    sets = args.sets or sets
    prefill = wl == "prefill"
    steps = args.steps or (200 if prefill else 1000)
    warmup = args.warmup if args.warmup is not None else (20 if prefill else 50)
    n_inputs = 4 if prefill else 16
    hot = 2.0 if args.hot else 0.0

    t0 = time.time()
    layers = []
    for s in range(sets):
        fn = lambda e, s=s: synth.expert_weights(seed, s, e, L.d_model, L.d_ff, device=dev)
        layers.append(m.pack_layer(L.d_model, L.d_ff, L.n_experts, L.top_k, fn, True, dev))
    base_layers = layers
    wrs = []
    if args.router:
        wrs = [torch.from_numpy(synth.router_weights(seed, s, L.n_experts, L.d_model)
                                .view(np.int16)).to(dev) for s in range(sets)]
        layers = [lay.variant(router=wr) for lay, wr in zip(base_layers, wrs)]
    torch.cuda.synchronize()
    print(f"[bench] packed {sets} layer sets in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)

    xs = [torch.from_numpy(synth.activations(seed, i, T, L.d_model)).to(dev)
          for i in range(n_inputs)]
    lgs = [torch.from_numpy(synth.router_logits(seed, i, T, L.n_experts, hot_bias=hot)).to(dev)
           for i in range(n_inputs)]
    lg_out = torch.empty((T, L.n_experts), dtype=torch.float32, device=dev)
    if args.router:   # the logits come from the router instead; routes from those
        lgs = [m.moe_router_logits(xs[i], wrs[i % sets]) for i in range(n_inputs)]
    q = torch.empty((T, L.d_model), dtype=torch.int8, device=dev)
    qs = torch.empty((T, L.d_model // 32), dtype=torch.float32, device=dev)
    route_out = (torch.empty((T, L.top_k), dtype=torch.int32, device=dev),
                 torch.empty((T, L.top_k), dtype=torch.float32, device=dev),
                 torch.empty(L.n_experts, dtype=torch.int32, device=dev),
                 torch.empty(L.n_experts + 1, dtype=torch.int32, device=dev),
                 torch.empty(T * L.top_k, dtype=torch.int32, device=dev))
    y = torch.empty((T, L.d_model), dtype=torch.float32, device=dev)
    ws = torch.empty(m.moe_ffn_workspace_bytes(layers[0], T), dtype=torch.uint8, device=dev)
    ffn = m.moe_ffn_prefill if prefill else m.moe_ffn_decode

    def step(i):
        lg = lgs[i % n_inputs]
        if prefill:
            m.moe_quant_act_q8(xs[i % n_inputs], q=q, scales=qs)
            if args.router:
                lg = m.moe_router_logits(xs[i % n_inputs], wrs[i % sets], logits=lg_out)
            m.moe_route_group(lg, L.top_k, out=route_out)
            ids, w, counts, offsets, srt = route_out
            ffn(layers[i % sets], q, qs, ids, w, offsets, srt, y=y, ws=ws)
        else:  # decode: the whole step from the layer input in one call
            m.moe_ffn_decode_step(layers[i % sets], xs[i % n_inputs],
                                  lg_out if args.router else lg, q=q, scales=qs,
                                  route_out=route_out, y=y, ws=ws)

    # touched experts per input (bytes are counted from the actual routes)
    touched = []
    for i in range(n_inputs):
        m.moe_route_group(lgs[i], L.top_k, out=route_out)
        counts = route_out[2].cpu().numpy()
        touched.append(int(np.count_nonzero(counts)) + 1)  # + shared expert

    # eager warmup; eager reference of the last timed step
    cycle = int(np.lcm(sets, n_inputs))
    reps, rem = divmod(steps, cycle)
    last = (steps - 1) % cycle
    if args.dump_inputs:
        os.makedirs(args.dump_inputs, exist_ok=True)
        xs[last % n_inputs].cpu().numpy().tofile(os.path.join(args.dump_inputs, "x.f32"))
        lgs[last % n_inputs].cpu().numpy().tofile(os.path.join(args.dump_inputs, "logits.f32"))
        print(json.dumps({"dumped": args.dump_inputs, "workload": wl, "rows": T,
                          "experts_touched": touched[last % n_inputs]}))
        return
    for i in range(max(warmup, cycle)):
        step(i)
    torch.cuda.synchronize()
    t_e = time.perf_counter()
    for i in range(cycle):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t_e) * 1e3 / cycle
    step(last)
    torch.cuda.synchronize()
    y_eager = y.clone()

    # HIP graphs: one holds a whole rotation cycle of steps, one the remainder,
    # so exactly `steps` steps run with no host work between them
    g_step = capture(torch, lambda: [step(i) for i in range(cycle)])
    g_rem = capture(torch, lambda: [step(i) for i in range(rem)]) if rem else None
    g_step.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # an event between replays (no synchronisation) gives each cycle's time
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev0.record(stream)
    for i in range(reps):
        marks[i].record(stream)
        g_step.replay()
    marks[reps].record(stream)
    if g_rem is not None:
        g_rem.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    if not torch.equal(y, y_eager):
        raise SystemExit("graph replay differs from the eager step")
    cycle_ms = [marks[i].elapsed_time(marks[i + 1]) / cycle for i in range(reps)]
    step_pct = ([round(float(v), 5) for v in np.percentile(cycle_ms, [10, 50, 90])]
                if cycle_ms else None)
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / steps
    tok_s = T * steps / (ms_total / 1e3)

    gu_bytes = 2 * L.d_ff * L.d_model // 2 + 2 * L.d_ff * L.d_model // 32
    dn_bytes = L.d_model * L.d_ff // 2 + L.d_model * L.d_ff // 32
    A = T * L.top_k + T
    act_bytes = T * (L.d_model * 4 + L.d_model + L.d_model // 8)  # x read, q + scales written
    mean_touched = float(np.mean(touched))
    step_bytes = mean_touched * (gu_bytes + dn_bytes) + act_bytes + T * L.d_model * 4
    if args.router:
        step_bytes += L.n_experts * L.d_model * 2 + T * L.n_experts * 4

    # dominant kernel, alone over the rotated sets in a graph: the gate/up
    # projection (decode) or the gate/up GEMM (prefill)
    ids, w, counts, offsets, srt = route_out   # routes of input `last`
    n_k = sets * max(1, 64 // sets)
    fused1 = not prefill and T == 1   # one row: quantiser + router + gate/up, one kernel
    if fused1:
        kcall = lambda i: m.moe_ffn_decode_step(
            base_layers[i % sets], xs[last % n_inputs], lgs[last % n_inputs], q=q, scales=qs,
            route_out=route_out, y=y, ws=ws, stage_mask=m.MOE_STAGE_GATE_UP)
    else:
        kcall = lambda i: m.moe_ffn_stages(base_layers[i % sets], int(prefill), m.MOE_STAGE_GATE_UP,
                                           q, qs, ids, w, offsets, srt, y, ws)
    g_k = capture(torch, lambda: [kcall(i) for i in range(n_k)])
    g_k.replay()
    torch.cuda.synchronize()
    kreps = max(2, (200 if prefill else 2000) // n_k)
    ev0.record(stream)
    for _ in range(kreps):
        g_k.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    k_us = ev0.elapsed_time(ev1) * 1e3 / (kreps * n_k)
    last_touched = touched[last % n_inputs]
    if prefill:
        k_flops = 2.0 * A * (2 * L.d_ff) * L.d_model
        achieved = k_flops / (k_us * 1e-6) / 1e12
        # hidden codes are written as bf16 (2 bytes) with fp32 scales; the GEMM
        # reads every hidden row's activations as gathered bf16 codes + scales
        hidden_bytes = A * (2 * L.d_ff + L.d_ff // 32 * 4)
        k_bytes = last_touched * gu_bytes + A * (2 * L.d_model + L.d_model // 8) + hidden_bytes
        hbm_gbs = k_bytes / (k_us * 1e-6) / 1e9
        # the bound is the one the kernel's arithmetic intensity selects: below
        # the ridge (peak flops / peak bytes) the weights' stream bounds it
        ridge = BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        intensity = k_flops / k_bytes
        common = dict(traffic=traffic_for((wl, T) if not args.router and not args.shard else None),
                      kernel="gemm_kernel<gate/up>", avg_us=round(k_us, 3),
                      flop_per_byte=round(intensity, 1), ridge_flop_per_byte=round(ridge, 1))
        if intensity >= ridge:
            roof = dict(bound="mfma", achieved=round(achieved, 2), peak=BF16_MFMA_PEAK_TFLOPS,
                        unit="TFLOP/s", frac=round(achieved / BF16_MFMA_PEAK_TFLOPS, 4), **common,
                        i8_peak_frac=round(achieved / I8_MFMA_PEAK_TOPS, 4),
                        hbm_gbs=round(hbm_gbs, 1))
        else:
            roof = dict(bound="hbm", achieved=round(hbm_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(hbm_gbs / HBM_PEAK_GBS, 4), **common,
                        tflops=round(achieved, 2),
                        mfma_frac=round(achieved / BF16_MFMA_PEAK_TFLOPS, 4))
    else:
        # gate/up weights of the touched experts, activations, hidden codes out
        # (one row: the fp32 row and the logits in, its codes and routes out)
        k_bytes = (last_touched * gu_bytes + T * (L.d_model + L.d_model // 8)
                   + A * (2 * L.d_ff + L.d_ff // 32 * 4))
        kname = "stream_kernel<gate/up>"
        if fused1:
            k_bytes += T * (L.d_model * 4 + L.n_experts * 4)
            kname = "stream_step1_kernel<quantise + route + gate/up>"
        achieved = k_bytes / (k_us * 1e-6) / 1e9
        # the counted routes are the benchmark's own (hot-expert and router runs
        # route differently, except for the one-row step's 7 experts)
        tkey = ((wl, T) + (("hot",) if hot else ())
                if not args.shard and (not args.router or (T == 1 and not hot)) else None)
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic_for(tkey),
                    kernel=kname, avg_us=round(k_us, 3),
                    bytes_per_launch=int(k_bytes), experts_touched=last_touched)

    router = None
    if args.router:   # the router projection alone, over the rotated weights
        rcall = lambda i: m.moe_router_logits(xs[last % n_inputs], wrs[i % sets], logits=lg_out)
        g_r = capture(torch, lambda: [rcall(i) for i in range(n_k)])
        g_r.replay()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(kreps):
            g_r.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        r_us = ev0.elapsed_time(ev1) * 1e3 / (kreps * n_k)
        r_bytes = L.n_experts * L.d_model * 2 + T * L.d_model * 4 + T * L.n_experts * 4
        r_flops = 2.0 * T * L.n_experts * L.d_model
        router = dict(kernel="router_kernel", avg_us=round(r_us, 3), bytes_per_launch=r_bytes,
                      hbm_gbs=round(r_bytes / (r_us * 1e-6) / 1e9, 1),
                      fp32_fma_tflops=round(r_flops / (r_us * 1e-6) / 1e12, 2))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, L, seed, T, m, synth, np, torch, dev, prefill)

    line = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4(e2m1+e8m0) x int8 -> exact block dots, f32 accumulate",
        "data": "synthetic (seeded counter-hash weights, N(0,1) activations/logits)",
        "config": {"workload": f"{wl}: E256 top-6 + shared, d_model 4096, d_ff {L.d_ff}"
                               + (" (TP8 shard of d_ff 2048)" if args.shard else "") + ", "
                               f"{T} token(s)/step, {sets} rotated layer sets"
                               + (", hot-16 +2.0 bias" if hot else "")
                               + (", router projection in the step (BF16 weights)"
                                  if args.router else ""),
                   "rows": T, "layer_sets": sets, "seed": seed},
        "step_hbm_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "eager_ms_per_step": round(eager_ms, 4),
        # per-step ms of each replayed rotation cycle: p10, median, p90
        "ms_per_step_p10_p50_p90": step_pct, "cycles": len(cycle_ms), "steps_per_cycle": cycle,
        "step_bytes": int(step_bytes),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if router is not None:
        line["router"] = router
    emit(line, args)


EAGER = False


class _EagerReplay:
    def __init__(self, fn):
        self.fn = fn

    def replay(self):
        self.fn()


def capture(torch, fn):
    """Capture fn's launches (on torch's current stream) into a HIP graph
    (with --eager: an object whose replay() simply runs fn again)."""
    if EAGER:
        fn()
        return _EagerReplay(fn)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def cpu_baseline(args, L, seed, T, m, synth, np, torch, dev, prefill):
    """The oracle, as it stands, on a bounded sample of the same workload: S
    fresh rows with the workload's distributions (about 10-15 s of CPU work
    on 16 threads), quantised, routed, grouped and run through the FFN."""
    import oracle

    S = args.cpu_sample or 256
    threads = min(16, len(os.sched_getaffinity(0)))
    x = synth.activations(seed, 1000 + T, S, L.d_model)
    lg = synth.router_logits(seed, 1000 + T, S, L.n_experts, hot_bias=2.0 if args.hot else 0.0)
    q, qs = oracle.quant_q8(x)
    ids, w = oracle.route(lg, L.top_k)
    need = set(int(e) for e in ids.reshape(-1)) | {L.n_experts}
    ex = {e: {k: v.cpu().numpy() for k, v in
              synth.expert_weights(seed, 0, e, L.d_model, L.d_ff, device=dev).items()}
          for e in sorted(need)}
    oracle.set_threads(threads)
    t0 = time.perf_counter()
    qo, qso = oracle.quant_q8(x)
    ido, wo = oracle.route(lg, L.top_k)
    oracle.group(ido, L.n_experts)
    oracle.ffn(ex, L.n_experts, L.top_k, True, qo, qso, ido, wo)
    dt = time.perf_counter() - t0
    # the same steps on one thread, over the first S1 rows of the sample
    S1 = min(S, 8)
    oracle.set_threads(1)
    t1 = time.perf_counter()
    qo, qso = oracle.quant_q8(x[:S1])
    ido, wo = oracle.route(lg[:S1], L.top_k)
    oracle.group(ido, L.n_experts)
    oracle.ffn(ex, L.n_experts, L.top_k, True, qo, qso, ido, wo)
    dt1 = time.perf_counter() - t1
    oracle.set_threads(threads)
    return {"value": round(S / dt, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{S} rows drawn like the workload's (layer set 0, {len(need)} experts): "
                      f"quant, route, group, FFN in fp64; {dt:.1f}s wall on {threads} threads",
            "value_1_thread": round(S1 / dt1, 4),
            "sample_1_thread": f"the first {S1} of those rows on 1 thread, {dt1:.1f}s wall"}


def bench_matvec(args, m, synth, np, torch, dev):
    c = synth.MATVEC
    N, D, K = c["n_out"], c["d_in"], (args.rows or 4)
    copies = args.sets or c["copies"]
    steps = args.steps or 2000
    warmup = args.warmup if args.warmup is not None else 100
    packs = []
    for i in range(copies):
        codes, scales = synth.matrix_weights(c["seed"], i, N, D, dev)
        packs.append(m.moe_pack_mxfp4(codes, scales, 0))
        del codes, scales
    x = torch.from_numpy(synth.activations(c["seed"], 0, K, D)).to(dev)
    q, qs = m.moe_quant_act_q8(x)
    y = torch.empty((K, N), device=dev)
    for i in range(max(warmup, copies)):
        m.moe_matvec_mxfp4(packs[i % copies], N, D, q, qs, y=y)
    torch.cuda.synchronize()
    reps, rem = divmod(steps, copies)
    g = capture(torch, lambda: [m.moe_matvec_mxfp4(packs[i], N, D, q, qs, y=y)
                                for i in range(copies)])
    g_rem = capture(torch, lambda: [m.moe_matvec_mxfp4(packs[i], N, D, q, qs, y=y)
                                    for i in range(rem)]) if rem else None
    g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        g.replay()
    if g_rem is not None:
        g_rem.replay()
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    nbytes = packs[0].numel() + K * (D + D // 8) + K * N * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = min(16, len(os.sched_getaffinity(0)))
        codes, scales = synth.matrix_weights(c["seed"], 0, N, D, dev)
        cn, sn = codes.cpu().numpy(), scales.cpu().numpy()
        xn = x.cpu().numpy()
        oracle.set_threads(threads)
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 5.0:
            qo, qso = oracle.quant_q8(xn)
            oracle.matvec(cn, sn, qo, qso)
            reps += 1
        dt = time.perf_counter() - t0
        cpu = {"value": round(reps * K / dt, 4), "unit": "rows/s", "cores": threads,
               "kind": "oracle", "sample": f"{reps} full matvecs of {K} rows, {dt:.1f}s wall"}
    line = {
        "metric": METRIC, "value": round(K / (us * 1e-6), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4(e2m1+e8m0) x int8 -> exact block dots, f32 accumulate",
        "data": "synthetic", "config": {"workload": f"matvec {N}x{D}, {K} rows, {copies} copies",
                                        "rows": K},
        "roofline": dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4), traffic=traffic_for(("matvec", K)),
                         kernel="stream_kernel<matvec>", avg_us=round(us, 3)),
        "cpu_baseline": cpu,
    }
    emit(line, args)


def bench_copy(args, torch, dev):
    """Plain device copy of a known size (1 GiB read + 1 GiB written per launch),
    rotated over 4 source buffers so no launch reads what the MALL holds."""
    n = 1 << 30
    srcs = [torch.full((n // 4,), float(i), dtype=torch.float32, device=dev) for i in range(4)]
    dst = torch.empty(n // 4, dtype=torch.float32, device=dev)
    steps = args.steps or 40
    warmup = args.warmup if args.warmup is not None else 4
    for i in range(warmup):
        dst.copy_(srcs[i % 4])
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        dst.copy_(srcs[i % 4])
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    line = {
        "metric": "calibration: device copy", "value": round(2 * n / (us * 1e-6) / 1e9, 1),
        "unit": "GB/s (read + write)", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(us / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "copy 1 GiB -> 1 GiB, 4 rotated sources"},
        "bytes_read_per_launch": n, "bytes_written_per_launch": n,
    }
    emit(line, args)


def emit(line, args):
    s = json.dumps(line)
    print(s, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(s + "\n")


if __name__ == "__main__":
    main()
