#!/usr/bin/env python3
"""Benchmark of the routed-expert MXFP4 MoE FFN hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
resident in HBM: per-32 int8 activation quantisation, top-k routing + expert
grouping, gate/up projection + SwiGLU + requant, down projection, weighted
combine.  Layer weight sets are rotated per step so the MALL (256 MB) cannot
hold them.  Prints one JSON line.

With no --workload, the line's value is the 1-row decode step (the DS-V4
layer, 8 rotated layer sets) and its "configs" object times every other
configuration of the metric in the same run: decode at 2, 4, 8, 16 rows
(uniform and hot-16 routes), prefill at 512 and 4096 rows, and the MXFP4
matvec at K = 1..5 rows, each with its dominant kernel's roofline.

One workload alone (--workload), e.g. under a profiler:
  decode        1 token per step, 8 layer sets (27.5 GB)
  decode-batch  --rows 2/4/8/16 tokens per step (--hot: +2.0 logit bias on 16
                experts)
  prefill       --rows 512 or 4096 tokens per step, 2 layer sets
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
I8_MFMA_PEAK_TOPS = 5000.0
FP4_MFMA_PEAK_TFLOPS = 10100.0

# Issue ceiling of the prefill GEMMs.  Per 32x32 output tile and 32-element
# block a SIMD issues one scaled 32x32x64 instruction (E2M1 weights x E3M2
# digit planes; 32.5 cycles measured) and sixteen wave64 fp32 FMAs (the
# activation scale; about 2.3 cycles each with two waves per SIMD, measured;
# no packed fp32), which do not overlap the matrix core when two waves share
# a SIMD: 70.8 cycles measured for the pattern in isolation.  At the 2.4 GHz
# peak clock on 1024 SIMDs:
GEMM_UNIT_CYCLES = 70.8
GEMM_CLOCK_GHZ = 2.4
GEMM_SIMDS = 1024

# HBM bytes per launch of each workload's dominant kernel, from rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) on the native counters driver
# replaying this benchmark's own inputs, scaled by the plain-copy calibration:
# read = 2 x FETCH_SIZE, written = WRITE_SIZE.  Counted offline (the source is
# named in the line); valid only for the kernel sources they were taken with
# (hash below, over the device code in csrc/): after any change to it the
# benchmark reports traffic as null.
TRAFFIC_DOC = "profiles/hbm_traffic_counters.md (moe_counters under rocprofv3 --pmc, offline)"
TRAFFIC_SRC = "5fb566e52a374d56"
TRAFFIC = {  # (workload, rows[, variant]): (read bytes, written bytes)
    ("decode", 1): (2 * 36676.4 * 1024, 48.6 * 1024),
    ("decode-batch", 16): (2 * 349812.3 * 1024, 675.5 * 1024),
    ("decode-batch", 16, "hot"): (2 * 171103.4 * 1024, 672.7 * 1024),
    ("prefill", 4096): (2 * 1277591.8 * 1024, 93724.5 * 1024),
    ("prefill", 512): (2 * 1167079.6 * 1024, 12216.2 * 1024),
    ("matvec", 5): (2 * 15414.7 * 1024, 280.0 * 1024),
}


def kernel_sources_hash():
    """Hash of the device code (csrc/*.hip and *.h; host-only .cpp excluded),
    with // comments and blank lines left out, so that only a change to the
    code itself marks the counted traffic stale."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mxfp4_routed_expert_e2m1_amd",
                     "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if not f.endswith((".hip", ".h")):
            continue
        h.update(f.encode())
        with open(os.path.join(d, f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def traffic_for(key):
    """Counted HBM bytes per launch for this workload and where they come
    from, or (None, reason): not counted, or the kernels changed since."""
    if key not in TRAFFIC:
        return None, "not counted for this workload"
    if kernel_sources_hash() != TRAFFIC_SRC:
        return None, f"stale: counted on kernel sources {TRAFFIC_SRC}, now {kernel_sources_hash()}"
    r, w = TRAFFIC[key]
    return int(r + w), TRAFFIC_DOC


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None,
                    choices=["decode", "decode-batch", "prefill", "matvec", "copy"],
                    help="time this workload alone (default: the 1-row decode step as the "
                         "value plus every configuration of the metric)")
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
    env = Env(m, synth, np, torch, dev)

    wl = args.workload
    if wl == "matvec":
        return emit(bench_matvec(env, args, args.rows or 4, args.steps, args.warmup,
                                 not args.no_cpu_baseline), args)
    if wl == "copy":
        return bench_copy(args, torch, dev)
    if wl is not None:
        T = args.rows or {"decode": 1, "decode-batch": 16, "prefill": 4096}[wl]
        r = run_ffn(env, args, wl, T, args.hot, args.steps, args.warmup)
        if r is None:   # --dump-inputs
            return
        cpu = None
        if not args.no_cpu_baseline:
            cpu = cpu_baseline(env, args, r["L"], r["seed"], T, wl == "prefill")
        return emit(line_of(r, args, cpu), args)

    # the whole metric: the 1-row step is the value, every other configuration
    # goes into "configs" (a few seconds each, layer sets packed once per seed)
    t_all = time.perf_counter()
    head = run_ffn(env, args, "decode", 1, False, args.steps, args.warmup)
    configs = {"decode_t1": summary(head)}
    plan = ([("decode-batch", t, False) for t in (2, 4, 8, 16)]
            + [("decode-batch", t, True) for t in (2, 4, 8, 16)]
            + [("prefill", 512, False), ("prefill", 4096, False)])
    for wl2, T, hot in plan:
        r = run_ffn(env, args, wl2, T, hot, None, None)
        configs[f"{'prefill' if wl2 == 'prefill' else 'decode'}_t{T}{'_hot' if hot else ''}"] = \
            summary(r)
        print(f"[bench] {wl2} {T}{' hot' if hot else ''}: {r['ms_step']:.4f} ms/step, "
              f"{r['roof']['kernel']} {r['roof']['avg_us']} us", file=sys.stderr, flush=True)
    env.drop_layers()
    for K in (1, 2, 3, 4, 5):
        mv = bench_matvec(env, args, K, None, None, False)
        configs[f"matvec_k{K}"] = {"rows": K, "ms_per_step": mv["ms_per_step"],
                                   "rows_per_s": mv["value"], "roofline": mv["roofline"]}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(env, args, head["L"], head["seed"], 1, False)
    line = line_of(head, args, cpu)
    line["configs"] = configs
    line["bench_wall_s"] = round(time.perf_counter() - t_all, 1)
    emit(line, args)


class Env:
    """Torch, the binding and the packed layer sets of the last seed used."""

    def __init__(self, m, synth, np, torch, dev):
        self.m, self.synth, self.np, self.torch, self.dev = m, synth, np, torch, dev
        self.key, self.layers = None, None

    def layer_sets(self, L, seed, sets):
        key = (L, seed, sets)
        if self.key != key:
            self.drop_layers()
            t0 = time.time()
            out = []
            for s in range(sets):
                fn = lambda e, s=s: self.synth.expert_weights(seed, s, e, L.d_model, L.d_ff,
                                                              device=self.dev)
                out.append(self.m.pack_layer(L.d_model, L.d_ff, L.n_experts, L.top_k, fn, True,
                                             self.dev))
            self.torch.cuda.synchronize()
            print(f"[bench] packed {sets} layer sets (seed {seed}) in {time.time() - t0:.1f}s",
                  file=sys.stderr, flush=True)
            self.key, self.layers = key, out
        return self.layers

    def drop_layers(self):
        self.key, self.layers = None, None
        self.torch.cuda.empty_cache()


def expert_bytes(L):
    """Algorithmic bytes of one expert: E2M1 codes (half a byte) + one E8M0
    byte per 32 weights, gate/up (2F x D) and down (D x F)."""
    gu = 2 * L.d_ff * L.d_model // 2 + 2 * L.d_ff * L.d_model // 32
    dn = L.d_model * L.d_ff // 2 + L.d_model * L.d_ff // 32
    return gu, dn


def run_ffn(env, args, wl, T, hot, steps, warmup):
    """Time `steps` whole steps of one FFN workload (graph replays over the
    rotated layer sets and inputs), then its dominant kernel alone."""
    m, synth, np, torch, dev = env.m, env.synth, env.np, env.torch, env.dev
    stream = torch.cuda.current_stream()
    L = synth.DSV4_LAYER
    if args.shard == "tp8":
        L = synth.Layer(n_experts=L.n_experts, top_k=L.top_k, d_model=L.d_model,
                        d_ff=L.d_ff // 8, has_shared=L.has_shared)
    if wl == "decode":
        seed, sets = synth.DECODE["seed"], 8
    elif wl == "decode-batch":
        seed, sets = synth.DECODE_BATCH["seed"], 8
    else:
        seed, sets = synth.PREFILL["seed"], 2
    sets = args.sets or sets
    prefill = wl == "prefill"
    steps = steps or (200 if prefill else 1000)
    warmup = warmup if warmup is not None else (20 if prefill else 50)
    n_inputs = 4 if prefill else 16
    hot_bias = 2.0 if hot else 0.0

    layers = env.layer_sets(L, seed, sets)
    base_layers = layers
    wrs = []
    if args.router:
        wrs = [torch.from_numpy(synth.router_weights(seed, s, L.n_experts, L.d_model)
                                .view(np.int16)).to(dev) for s in range(sets)]
        layers = [lay.variant(router=wr) for lay, wr in zip(base_layers, wrs)]

    xs = [torch.from_numpy(synth.activations(seed, i, T, L.d_model)).to(dev)
          for i in range(n_inputs)]
    lgs = [torch.from_numpy(synth.router_logits(seed, i, T, L.n_experts, hot_bias=hot_bias))
           .to(dev) for i in range(n_inputs)]
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

    def step(i):
        lg = lgs[i % n_inputs]
        if prefill:
            m.moe_quant_act_q8(xs[i % n_inputs], q=q, scales=qs)
            if args.router:
                lg = m.moe_router_logits(xs[i % n_inputs], wrs[i % sets], logits=lg_out)
            m.moe_route_group(lg, L.top_k, out=route_out)
            ids, w, counts, offsets, srt = route_out
            m.moe_ffn_prefill(layers[i % sets], q, qs, ids, w, offsets, srt, y=y, ws=ws)
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
        return None
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
    # percentiles of the per-cycle step time, only with enough cycles to mean one
    step_pct = ([round(float(v), 5) for v in np.percentile(cycle_ms, [10, 50, 90])]
                if len(cycle_ms) >= 3 else None)
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / steps
    tok_s = T * steps / (ms_total / 1e3)

    gu_bytes, dn_bytes = expert_bytes(L)
    A = T * L.top_k + T
    mean_touched = float(np.mean(touched))
    # the step's algorithmic bytes: the touched experts' weights, x and the
    # logits in, y out (int8 codes and hidden codes stay in the workspace)
    step_bytes = (mean_touched * (gu_bytes + dn_bytes) + T * L.d_model * 4
                  + T * L.n_experts * 4 + T * L.d_model * 4)
    if args.router:
        step_bytes += L.n_experts * L.d_model * 2

    # dominant kernel, alone over the rotated sets in a graph: the gate/up
    # projection (decode) or the gate/up GEMM without the digit-plane prep
    # (prefill: MOE_STAGE_REUSE_ACTS; the timed step ran the prep just before)
    ids, w, counts, offsets, srt = route_out   # routes of input `last`
    n_k = sets * max(1, 64 // sets)
    fused1 = not prefill and T == 1   # one row: quantiser + router + gate/up, one kernel
    if fused1:
        kcall = lambda i: m.moe_ffn_decode_step(
            base_layers[i % sets], xs[last % n_inputs], lgs[last % n_inputs], q=q, scales=qs,
            route_out=route_out, y=y, ws=ws, stage_mask=m.MOE_STAGE_GATE_UP)
    else:
        mask = m.MOE_STAGE_GATE_UP | (m.MOE_STAGE_REUSE_ACTS if prefill else 0)
        kcall = lambda i: m.moe_ffn_stages(base_layers[i % sets], int(prefill), mask,
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
    counts_np = counts.cpu().numpy()
    tkey = ((wl, T) + (("hot",) if hot else ())
            if not args.shard and (not args.router or (T == 1 and not hot)) else None)
    traffic, traffic_src = traffic_for(tkey)
    # algorithmic bytes of the gate/up launch: the touched experts' gate/up
    # weights, each token's int8 codes and scales once (T (D + D/8)), one
    # byte per hidden code and its fp32 scale out (A (F + F/8))
    k_bytes = last_touched * gu_bytes + T * (L.d_model + L.d_model // 8) + A * (L.d_ff + L.d_ff // 8)
    if prefill:
        k_flops = 2.0 * A * (2 * L.d_ff) * L.d_model
        achieved = k_flops / (k_us * 1e-6) / 1e12
        hbm_gbs = k_bytes / (k_us * 1e-6) / 1e9
        # what this implementation's layout moves by design: the tokens'
        # digit planes (1.5 bytes per code) gathered per assignment, hidden
        # codes written as digit planes too
        impl_bytes = (last_touched * gu_bytes + A * (L.d_model * 3 // 2 + L.d_model // 8)
                      + A * (L.d_ff * 3 // 2 + L.d_ff // 8))
        # issue ceiling: 32 x 32 output tiles x 32-element blocks, with each
        # expert's rows padded to whole 32-row tiles as the GEMM runs them
        rows32 = int(sum((int(c) + 31) // 32 * 32 for c in counts_np)) + (T + 31) // 32 * 32
        units = rows32 / 32 * (2 * L.d_ff / 32) * (L.d_model / 32)
        ceil_us = units * GEMM_UNIT_CYCLES / GEMM_SIMDS / (GEMM_CLOCK_GHZ * 1e3)
        # the method's contraction is int8 activations x FP4 weights: priced
        # against the dense int8 matrix-core peak (bf16 and FP4 fractions
        # beside it).  The bound is whichever lower bound on the kernel's
        # time is larger: its issue ceiling, or its algorithmic bytes at the
        # HBM peak.
        ridge = I8_MFMA_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        intensity = k_flops / k_bytes
        hbm_floor_us = k_bytes / (HBM_PEAK_GBS * 1e9) * 1e6
        issue_bound = ceil_us >= hbm_floor_us
        roof = dict(kernel="gemm_kernel<gate/up>", avg_us=round(k_us, 3),
                    bound="mfma" if issue_bound else "hbm",
                    achieved=round(achieved, 2) if issue_bound else round(hbm_gbs, 1),
                    peak=I8_MFMA_PEAK_TOPS if issue_bound else HBM_PEAK_GBS,
                    unit="TFLOP/s" if issue_bound else "GB/s",
                    frac=round(achieved / I8_MFMA_PEAK_TOPS if issue_bound
                               else hbm_gbs / HBM_PEAK_GBS, 4),
                    hbm_floor_us=round(hbm_floor_us, 1),
                    tflops=round(achieved, 2),
                    bf16_peak_frac=round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                    i8_peak_frac=round(achieved / I8_MFMA_PEAK_TOPS, 4),
                    fp4_peak_frac=round(achieved / FP4_MFMA_PEAK_TFLOPS, 4),
                    issue_ceiling_us=round(ceil_us, 1),
                    issue_ceiling_frac=round(ceil_us / k_us, 4),
                    hbm_gbs=round(hbm_gbs, 1), hbm_frac=round(hbm_gbs / HBM_PEAK_GBS, 4),
                    bytes_per_launch=int(k_bytes), impl_bytes_per_launch=int(impl_bytes),
                    flop_per_byte=round(intensity, 1), ridge_flop_per_byte=round(ridge, 1),
                    traffic=traffic, traffic_src=traffic_src, experts_touched=last_touched)
    else:
        kname = "stream_kernel<gate/up>"
        if fused1:   # the fp32 row and its logits in, its codes and routes out
            k_bytes += T * (L.d_model * 4 + L.n_experts * 4)
            kname = "stream_step1_kernel<quantise + route + gate/up>"
        # the layout's hidden codes are bf16 values (2 bytes per code)
        impl_bytes = k_bytes + A * L.d_ff
        achieved = k_bytes / (k_us * 1e-6) / 1e9
        roof = dict(kernel=kname, avg_us=round(k_us, 3), bound="hbm", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                    bytes_per_launch=int(k_bytes), impl_bytes_per_launch=int(impl_bytes),
                    traffic=traffic, traffic_src=traffic_src, experts_touched=last_touched)

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
    del g_step, g_rem, g_k
    return dict(wl=wl, T=T, hot=hot, L=L, seed=seed, sets=sets, steps=steps, warmup=warmup,
                ms_step=ms_step, tok_s=tok_s, step_pct=step_pct, cycles=len(cycle_ms),
                cycle=cycle, step_bytes=step_bytes, eager_ms=eager_ms, roof=roof, router=router,
                mean_touched=mean_touched)


def summary(r):
    """One configuration's entry in the line's "configs" object."""
    out = {"rows": r["T"], "ms_per_step": round(r["ms_step"], 5),
           "tokens_per_s": round(r["tok_s"], 1),
           "step_hbm_gbs": round(r["step_bytes"] / (r["ms_step"] * 1e-3) / 1e9, 1),
           "experts_touched_mean": round(r["mean_touched"], 2),
           "roofline": r["roof"]}
    if r["step_pct"] is not None:
        out["ms_per_step_p10_p50_p90"] = r["step_pct"]
        out["cycles"] = r["cycles"]
    return out


def line_of(r, args, cpu):
    L, T, wl = r["L"], r["T"], r["wl"]
    line = {
        "metric": METRIC, "value": round(r["tok_s"], 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": r["steps"], "warmup": r["warmup"], "ms_per_step": round(r["ms_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4(e2m1+e8m0) x int8 -> exact block dots, f32 accumulate",
        "data": "synthetic (seeded counter-hash weights, N(0,1) activations/logits)",
        "config": {"workload": f"{wl}: E256 top-6 + shared, d_model 4096, d_ff {L.d_ff}"
                               + (" (TP8 shard of d_ff 2048)" if args.shard else "") + ", "
                               f"{T} token(s)/step, {r['sets']} rotated layer sets"
                               + (", hot-16 +2.0 bias" if r["hot"] else "")
                               + (", router projection in the step (BF16 weights)"
                                  if args.router else ""),
                   "rows": T, "layer_sets": r["sets"], "seed": r["seed"]},
        "step_hbm_gbs": round(r["step_bytes"] / (r["ms_step"] * 1e-3) / 1e9, 1),
        "eager_ms_per_step": round(r["eager_ms"], 4),
        "cycles": r["cycles"], "steps_per_cycle": r["cycle"],
        "step_bytes": int(r["step_bytes"]),
        "roofline": r["roof"],
        "cpu_baseline": cpu,
    }
    if r["step_pct"] is not None:   # per-step ms of the replayed cycles: p10, median, p90
        line["ms_per_step_p10_p50_p90"] = r["step_pct"]
    if r["router"] is not None:
        line["router"] = r["router"]
    return line


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


def host_info():
    """What the CPU figures ran on: logical CPUs (all, and this process's
    affinity), the CPU model, OMP_NUM_THREADS, and the threads the oracle
    uses: every CPU of the affinity mask, capped by OMP_NUM_THREADS when that
    is set (the host's share for one GPU)."""
    aff = len(os.sched_getaffinity(0))
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = aff
    if omp and omp.isdigit() and int(omp) > 0:
        threads = min(aff, int(omp))
    return {"nproc": os.cpu_count(), "affinity_cpus": aff, "cpu_model": model,
            "OMP_NUM_THREADS": omp}, threads


def cpu_baseline(env, args, L, seed, T, prefill):
    """The oracle, as it stands, on a bounded sample of the same workload: S
    fresh rows with the workload's distributions (about 10-20 s of CPU work),
    quantised, routed, grouped and run through the FFN, on the host's threads;
    then the same steps on one thread over the first rows of the sample."""
    import oracle

    synth, torch, dev = env.synth, env.torch, env.dev
    info, threads = host_info()
    S = args.cpu_sample or 256
    x = synth.activations(seed, 1000 + T, S, L.d_model)
    lg = synth.router_logits(seed, 1000 + T, S, L.n_experts, hot_bias=2.0 if args.hot else 0.0)
    q, qs = oracle.quant_q8(x)
    ids, w = oracle.route(lg, L.top_k)
    need = set(int(e) for e in ids.reshape(-1)) | {L.n_experts}
    ex = {e: {k: v.cpu().numpy() for k, v in
              synth.expert_weights(seed, 0, e, L.d_model, L.d_ff, device=dev).items()}
          for e in sorted(need)}

    def run(rows, nthreads):
        oracle.set_threads(nthreads)
        t0 = time.perf_counter()
        qo, qso = oracle.quant_q8(x[:rows])
        ido, wo = oracle.route(lg[:rows], L.top_k)
        oracle.group(ido, L.n_experts)
        oracle.ffn(ex, L.n_experts, L.top_k, True, qo, qso, ido, wo)
        return time.perf_counter() - t0

    dt = run(S, threads)
    S1 = min(S, 16)
    dt1 = run(S1, 1)
    oracle.set_threads(threads)
    return {"value": round(S / dt, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{S} rows drawn like the workload's (layer set 0, {len(need)} experts): "
                      f"quant, route, group, FFN in fp64; {dt:.1f}s wall on {threads} threads",
            "value_1_thread": round(S1 / dt1, 4),
            "sample_1_thread": f"the first {S1} of those rows on 1 thread, {dt1:.1f}s wall",
            **info}


def bench_matvec(env, args, K, steps, warmup, with_cpu):
    m, synth, torch, dev = env.m, env.synth, env.torch, env.dev
    c = synth.MATVEC
    N, D = c["n_out"], c["d_in"]
    copies = args.sets or c["copies"]
    steps = steps or 2000
    warmup = warmup if warmup is not None else 100
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
    # algorithmic bytes: the packed matrix (codes + E8M0), K int8 rows and
    # their scales in, K fp32 rows out
    nbytes = packs[0].numel() + K * (D + D // 8) + K * N * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    traffic, traffic_src = traffic_for(("matvec", K))
    cpu = None
    if with_cpu:
        import oracle
        info, threads = host_info()
        codes, scales = synth.matrix_weights(c["seed"], 0, N, D, dev)
        cn, sn = codes.cpu().numpy(), scales.cpu().numpy()
        xn = x.cpu().numpy()
        oracle.set_threads(threads)
        n_rep, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 5.0:
            qo, qso = oracle.quant_q8(xn)
            oracle.matvec(cn, sn, qo, qso)
            n_rep += 1
        dt = time.perf_counter() - t0
        cpu = {"value": round(n_rep * K / dt, 4), "unit": "rows/s", "cores": threads,
               "kind": "oracle", "sample": f"{n_rep} full matvecs of {K} rows, {dt:.1f}s wall",
               **info}
    del g, g_rem, packs
    torch.cuda.empty_cache()
    return {
        "metric": METRIC, "value": round(K / (us * 1e-6), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4(e2m1+e8m0) x int8 -> exact block dots, f32 accumulate",
        "data": "synthetic", "config": {"workload": f"matvec {N}x{D}, {K} rows, {copies} copies",
                                        "rows": K},
        "roofline": dict(kernel="stream_kernel<matvec>", avg_us=round(us, 3), bound="hbm",
                         achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4), bytes_per_launch=int(nbytes),
                         traffic=traffic, traffic_src=traffic_src),
        "cpu_baseline": cpu,
    }


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
