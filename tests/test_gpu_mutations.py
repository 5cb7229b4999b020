"""Seeded mutation sweep of the routed-expert layer ([gfx90a] §8.2 checks its
down consumer over mutated inputs, routes, weights and scales).

Each seed draws a handful of mutations of the layer's inputs -- activation
magnitudes, zero and one-element blocks, values sitting exactly on a
quantiser rounding tie, outliers, router logits with exact ties, saturated or
hot logits, sentinel routes -- and of its weights and scales -- runs of the
extreme E2M1 codes (+-6, -0, 0), constant code bytes, E8M0 exponents spread
over [-30, +6] per block, per row or in a fixed pattern -- and checks the GPU
layer stage by stage against the fp64 oracle (activation codes, routes and
grouping bit for bit, hidden codes with the rounding-boundary allowance, y
within the tolerance).  The DeepSeek-V4 16-row decode is also compared bit for
bit with the oracle's exact-rows mode.

Two sweeps of 100 seeds: the tiny layer (8 experts, top-2, d_model 256, d_ff
512, 4 rows; decode, step and prefill entries in turn) and a 16-row decode of
the DeepSeek-V4 layer (256 experts, top-6 + shared, d_model 4096, d_ff 2048),
whose mutated experts are packed into a resident layer and restored after
each case."""
import numpy as np
import pytest
import torch

import oracle
import synth
from ffn_case import run_case

pytestmark = pytest.mark.gpu

m = pytest.importorskip("mxfp4_routed_expert_e2m1_amd")
DEV = "cuda"
N_SEEDS = 100


# ------------------------------------------------------------- mutations
def _tie_block(rng):
    # one element at 127 c and the others at (k + 1/2) c, c a power of two:
    # d = 127 c / 127 = c exactly and every other x / d is an exact tie
    c = np.float32(2.0 ** rng.integers(-6, 7))
    k = rng.integers(-127, 127, 32).astype(np.float32) + np.float32(0.5)
    b = k * c
    b[rng.integers(32)] = np.float32(127.0) * c * rng.choice([-1, 1])
    return b.astype(np.float32)


def mutate_x(rng, x):
    """Activation mutations; returns the names applied."""
    T, D = x.shape
    nb = D // 32
    done = []
    for kind in rng.choice(["scale", "zero", "single", "tie", "outlier", "const"],
                           size=rng.integers(1, 4), replace=False):
        if kind == "scale":
            x *= (10.0 ** rng.uniform(-3, 3, (T, 1))).astype(np.float32)
        elif kind == "zero":
            for _ in range(rng.integers(1, 3 * T + 1)):
                t, b = rng.integers(T), rng.integers(nb)
                x[t, 32 * b:32 * b + 32] = 0
            if rng.random() < 0.5:
                x[rng.integers(T)] = 0
        elif kind == "single":
            for _ in range(rng.integers(1, 3 * T + 1)):
                t, b = rng.integers(T), rng.integers(nb)
                v = x[t, 32 * b + rng.integers(32)]
                x[t, 32 * b:32 * b + 32] = 0
                x[t, 32 * b + rng.integers(32)] = v if v != 0 else 1.0
        elif kind == "tie":
            for _ in range(rng.integers(1, 4 * T + 1)):
                t, b = rng.integers(T), rng.integers(nb)
                x[t, 32 * b:32 * b + 32] = _tie_block(rng)
        elif kind == "outlier":
            n = rng.integers(1, 4 * T + 1)
            x[rng.integers(T, size=n), rng.integers(D, size=n)] *= np.float32(1e3)
        elif kind == "const":
            t, b = rng.integers(T), rng.integers(nb)
            x[t, 32 * b:32 * b + 32] = np.float32(rng.normal())
        done.append(f"x:{kind}")
    return done


def mutate_logits(rng, lg, top_k):
    """Router mutations; returns (names, ids_override or None)."""
    T, E = lg.shape
    done, ids_override = [], None
    kinds = list(rng.choice(["ties", "hot", "saturate", "flat", "sentinel"],
                            size=rng.integers(1, 3), replace=False))
    kinds.sort(key=lambda k: k == "sentinel")  # routes are taken after the logits change
    for kind in kinds:
        if kind == "ties":
            lg[:] = np.round(lg * 2.0) / 2.0  # a coarse grid: many exact ties
        elif kind == "hot":
            hot = rng.choice(E, size=min(E, 4), replace=False)
            lg[:, hot] += np.float32(rng.uniform(1, 4))
        elif kind == "saturate":
            rows = rng.random(T) < 0.5
            lg[rows] *= np.float32(rng.uniform(15, 40))
        elif kind == "flat":
            lg[rng.integers(T)] = np.float32(rng.normal())  # every expert tied
        elif kind == "sentinel":
            ids, _ = oracle.route(lg, top_k)
            ids = ids.copy()
            ids[rng.random(ids.shape) < 0.3] = -1
            ids[rng.integers(T)] = -1  # a token owned by no local expert
            ids_override = ids
        done.append(f"routes:{kind}")
    return done, ids_override


def mutate_expert(rng, w):
    """Weight and scale mutations of one expert's canonical weights (numpy,
    modified in place); returns the names applied."""
    done = []
    mats = [("gate_up_codes", "gate_up_scales"), ("down_codes", "down_scales")]
    for kind in rng.choice(["extreme", "const", "wide", "rowconst", "pattern"],
                           size=rng.integers(1, 3), replace=False):
        cn, sn = mats[rng.integers(2)]
        c, s = w[cn], w[sn]
        n, half = c.shape
        if kind == "extreme":
            rows = rng.choice(n, size=rng.integers(1, 33), replace=False)
            c[rows] = rng.choice(np.array([0x77, 0xFF, 0x88, 0x00, 0x7F, 0xF7], np.uint8),
                                 size=(len(rows), 1))
        elif kind == "const":
            r0 = rng.integers(n)
            c[r0:r0 + 16, :] = np.uint8(rng.integers(256))
        elif kind == "wide":
            s[:] = (127 + rng.integers(-30, 7, s.shape)).astype(np.uint8)
        elif kind == "rowconst":
            s[:] = (127 + rng.integers(-20, 5, (n, 1))).astype(np.uint8)
        elif kind == "pattern":
            s[:] = (120 + (np.arange(s.shape[1]) % 9)).astype(np.uint8)[None, :]
        done.append(f"{cn.split('_c')[0]}:{kind}")
    return done


def _to_dev(w):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for k, v in w.items()}


# ------------------------------------------------------------ tiny layer
TINY = synth.TINY["layer"]
_TINY_W = {}


def tiny_weights():
    if not _TINY_W:
        for e in range(TINY.n_experts):
            _TINY_W[e] = {k: v.cpu().numpy() for k, v in synth.expert_weights(
                synth.TINY["seed"], 0, e, TINY.d_model, TINY.d_ff, device=DEV).items()}
    return _TINY_W


@pytest.mark.parametrize("seed", range(N_SEEDS))
def test_mutation_tiny_layer(seed):
    rng = np.random.default_rng(10_000 + seed)
    base = tiny_weights()
    ex = {e: {k: v.copy() for k, v in base[e].items()} for e in base}
    names = []
    for e in rng.choice(TINY.n_experts, size=rng.integers(1, 4), replace=False):
        names += [f"e{e}:{n}" for n in mutate_expert(rng, ex[int(e)])]
    T = synth.TINY["rows"]
    x = synth.activations(synth.TINY["seed"], 100 + seed, T, TINY.d_model)
    lg = synth.router_logits(synth.TINY["seed"], 100 + seed, T, TINY.n_experts)
    names += mutate_x(rng, x)
    rn, ids_override = mutate_logits(rng, lg, TINY.top_k)
    names += rn
    entry = ["moe_ffn_decode", "step", "moe_ffn_prefill"][seed % 3]
    if entry == "step" and ids_override is not None:
        entry = "moe_ffn_decode"
    dev_w = {e: _to_dev(w) for e, w in ex.items()}
    layer = m.pack_layer(TINY.d_model, TINY.d_ff, TINY.n_experts, TINY.top_k,
                         lambda e: dev_w[e], has_shared=False, device=DEV)
    print(f"seed {seed} [{entry}]: {' '.join(names)}", flush=True)
    r = run_case(TINY, synth.TINY["seed"], x, lg, entry=entry, ids_override=ids_override,
                 layer=layer, experts=lambda e: ex[e])
    print(f"  worst err/tol {r['worst']:.3f}, flips {r['flips']}")


# ------------------------------------------- DeepSeek-V4 16-row decode
DSV4 = synth.DSV4_LAYER
_DS = {}


def ds_state():
    """The resident DS-V4 layer of the decode-batch seed and the canonical
    weights of all its experts on the host (generated once)."""
    if not _DS:
        seed = synth.DECODE_BATCH["seed"]
        fn = lambda e: synth.expert_weights(seed, 0, e, DSV4.d_model, DSV4.d_ff, device=DEV)
        _DS["layer"] = m.pack_layer(DSV4.d_model, DSV4.d_ff, DSV4.n_experts, DSV4.top_k, fn,
                                    has_shared=True, device=DEV)
        _DS["host"] = {e: {k: v.cpu().numpy() for k, v in fn(e).items()}
                       for e in range(DSV4.n_experts + 1)}
    return _DS


def _pack_expert(layer, e, w):
    gu, dn, sgu, sdn = layer.tensors[:4]
    d = _to_dev(w)
    m.moe_pack_mxfp4(d["gate_up_codes"], d["gate_up_scales"], 1,
                     out=gu[e] if e < DSV4.n_experts else sgu)
    m.moe_pack_mxfp4(d["down_codes"], d["down_scales"], 0,
                     out=dn[e] if e < DSV4.n_experts else sdn)


@pytest.mark.parametrize("seed", range(N_SEEDS))
def test_mutation_dsv4_decode_16_rows(seed):
    st = ds_state()
    layer, host = st["layer"], st["host"]
    rng = np.random.default_rng(20_000 + seed)
    T, bseed = 16, synth.DECODE_BATCH["seed"]
    x = synth.activations(bseed, 5000 + seed, T, DSV4.d_model)
    lg = synth.router_logits(bseed, 5000 + seed, T, DSV4.n_experts)
    names = mutate_x(rng, x)
    rn, ids_override = mutate_logits(rng, lg, DSV4.top_k)
    names += rn
    # mutate 1-3 of the experts this step touches (and sometimes the shared one)
    ids_now, _ = oracle.route(lg, DSV4.top_k)
    touched = np.unique(ids_now[ids_now >= 0])
    pick = [int(e) for e in rng.choice(touched, size=min(len(touched), rng.integers(1, 4)),
                                       replace=False)]
    if rng.random() < 0.3:
        pick.append(DSV4.n_experts)
    mutated = {}
    for e in pick:
        w = {k: v.copy() for k, v in host[e].items()}
        names += [f"e{e}:{n}" for n in mutate_expert(rng, w)]
        mutated[e] = w
    entry = "step" if (seed % 2 and ids_override is None) else "moe_ffn_decode"
    print(f"seed {seed} [{entry}]: {' '.join(names)}", flush=True)
    try:
        for e, w in mutated.items():
            _pack_expert(layer, e, w)
        experts = lambda e: mutated.get(e, host[e])
        r = run_case(DSV4, bseed, x, lg, entry=entry, ids_override=ids_override, layer=layer,
                     experts=experts)
        # exact rows: the same routes and weights through the oracle's named
        # fp32 order give the GPU's bits
        with oracle.exact_rows():
            w_used = r["w"]
            if ids_override is None:
                _, w_used = oracle.route(lg, DSV4.top_k)
                np.testing.assert_array_equal(w_used, r["w"])
            y_x = oracle.ffn(r["ex"], DSV4.n_experts, DSV4.top_k, True, r["q_o"], r["qs_o"],
                             r["ids"], w_used)
        np.testing.assert_array_equal(r["y"].cpu().numpy(), y_x)
        print(f"  worst err/tol {r['worst']:.3f}, flips {r['flips']}, exact rows: bitwise")
    finally:
        for e in mutated:
            _pack_expert(layer, e, host[e])
