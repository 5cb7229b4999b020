"""Pins for the oracle's BF16-intermediate mode (CPU only).

The mode rounds each SwiGLU output to the nearest BF16 value (ties to even)
before its group-32 requantisation, the reading of the gfx90a report's §8.2
down chain, which reads an already-rounded BF16 intermediate.  The rounding is
pinned against torch's CPU float32 -> bfloat16 cast, which is written
independently of the oracle, and against hand-worked values of the format.
"""
import numpy as np
import pytest
import torch

import bruteforce
import oracle
import synth


def _torch_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _same_bits(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    nan = np.isnan(a) & np.isnan(b)
    return np.all(nan | (a.view(np.uint32) == b.view(np.uint32)))


def test_round_bf16_worked_values():
    # BF16 keeps 8 significant bits: the spacing at 1 is 2^-7.
    f = float.fromhex
    cases = [
        (1.0, 1.0),
        (f("0x1.01p+0"), 1.0),                       # 1 + 2^-8: tie, to the even 1
        (f("0x1.03p+0"), f("0x1.04p+0")),            # 1 + 3*2^-8: tie, to even 1 + 2^-6
        (f("0x1.0101p+0"), f("0x1.02p+0")),          # just above the tie: up
        (f("0x1.00fep+0"), 1.0),                     # just below the tie: down
        (-f("0x1.03p+0"), -f("0x1.04p+0")),          # sign symmetric
        (f("0x1.ffp+0"), 2.0),                       # tie at the top of a binade, carry
        (f("0x1.fep+127"), f("0x1.fep+127")),        # largest finite BF16
        (f("0x1.ffp+127"), float("inf")),            # its tie with 2^128: overflow
        (f("0x1p-126"), f("0x1p-126")),              # smallest normal
        (f("0x1p-133"), f("0x1p-133")),              # smallest BF16 subnormal
        (f("0x1p-134"), 0.0),                        # half of it: tie, to even 0
        (f("0x1.8p-133"), f("0x1p-132")),            # 1.5 steps: tie, to even 2
        (0.0, 0.0),
        (float("inf"), float("inf")),
        (-float("inf"), -float("inf")),
    ]
    x = np.array([c[0] for c in cases], np.float32)
    want = np.array([c[1] for c in cases], np.float32)
    got = oracle.round_bf16(x)
    for xi, g, w in zip(x, got, want):
        assert g == w, (float(xi).hex(), float(g).hex(), float(w).hex())
    assert np.signbit(oracle.round_bf16(np.array([-0.0], np.float32))[0])
    assert np.isnan(oracle.round_bf16(np.array([np.nan], np.float32))[0])


def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(5)
    # every class of fp32 bit pattern: random bits, exact ties (low half
    # 0x8000) with even and odd kept bits, its neighbours, subnormals, the
    # overflow edge
    bits = rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32)
    hi = rng.integers(0, 1 << 16, 20000, dtype=np.uint64).astype(np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001, hi | 0xFFFF, hi])
    sub = rng.integers(0, 1 << 23, 20000, dtype=np.uint64).astype(np.uint32)
    edge = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7FFFFF, 0x7F800000,
                     0xFF7F8000, 0x00008000, 0x00018000, 0x80008000], np.uint32)
    x = np.concatenate([bits, ties, sub, sub | 0x80000000, edge]).view(np.float32)
    assert _same_bits(oracle.round_bf16(x), _torch_bf16(x))


def test_round_bf16_idempotent_and_monotone():
    rng = np.random.default_rng(6)
    x = np.sort(rng.standard_normal(50000).astype(np.float32) * 1e3)
    r = oracle.round_bf16(x)
    assert _same_bits(oracle.round_bf16(r), r)
    assert np.all(np.diff(r.astype(np.float64)) >= 0)
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    # nearest: no BF16 value lies closer than the chosen one
    up = (r.view(np.uint32) + np.uint32(0x10000)).view(np.float32)
    dn = (r.view(np.uint32) - np.uint32(0x10000)).view(np.float32)
    e = np.abs(x.astype(np.float64) - r)
    assert np.all(e <= np.abs(x.astype(np.float64) - up))
    assert np.all(e <= np.abs(x.astype(np.float64) - dn))


def _layer_inputs(seed, E=6, k=2, D=128, F=96, T=3, shared=True):
    rng = np.random.default_rng(seed)
    experts = {}
    for e in range(E + int(shared)):
        experts[e] = dict(
            gate_up_codes=rng.integers(0, 256, (2 * F, D // 2), dtype=np.uint8),
            gate_up_scales=(127 + rng.integers(-8, 1, (2 * F, D // 32))).astype(np.uint8),
            down_codes=rng.integers(0, 256, (D, F // 2), dtype=np.uint8),
            down_scales=(127 + rng.integers(-8, 1, (D, F // 32))).astype(np.uint8))
    x = rng.standard_normal((T, D)).astype(np.float32)
    q, qs = oracle.quant_q8(x)
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    return experts, q, qs, ids, w


@pytest.mark.parametrize("shared", [False, True])
def test_ffn_bf16_mode_vs_bruteforce(shared):
    E, k = 6, 2
    experts, q, qs, ids, w = _layer_inputs(31, E, k, shared=shared)
    with oracle.bf16_intermediate():
        y, mid = oracle.ffn(experts, E, k, shared, q, qs, ids, w, want_intermediates=True)
    ref = bruteforce.ffn(experts, E, k, shared, q, qs, ids, w, bf16_mid=True)
    tol = 2 * np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) + 1e-40
    assert np.all(np.abs(y - ref) <= tol)
    # the requantised intermediate comes from BF16 values
    assert np.all((mid["h"].view(np.uint32) & 0xFFFF) == 0)
    hq2, hs2 = bruteforce.quant(mid["h"])
    np.testing.assert_array_equal(mid["hq"], hq2)
    np.testing.assert_array_equal(mid["hs"], hs2)
    # and the mode is no no-op on this layer
    y0 = oracle.ffn(experts, E, k, shared, q, qs, ids, w)
    assert np.any(y0 != y)


@pytest.mark.parametrize("exact", [False, True])
def test_bf16_mode_rounds_the_default_intermediate(exact):
    # same projections and SwiGLU; the mode only inserts the rounding, in
    # either arithmetic mode, and is restored on exit
    cfg = synth.TINY
    L = cfg["layer"]
    experts = {e: {kk: v.numpy() for kk, v in synth.expert_weights(
        cfg["seed"], 0, e, L.d_model, L.d_ff).items()} for e in range(L.n_experts)}
    x = synth.activations(cfg["seed"], 0, cfg["rows"], L.d_model)
    lg = synth.router_logits(cfg["seed"], 0, cfg["rows"], L.n_experts)
    old = oracle.set_exact_rows(exact)
    try:
        q, qs = oracle.quant_q8(x)
        ids, w = oracle.route(lg, L.top_k)
        _, mid0 = oracle.ffn(experts, L.n_experts, L.top_k, False, q, qs, ids, w,
                             want_intermediates=True)
        with oracle.bf16_intermediate():
            _, mid1 = oracle.ffn(experts, L.n_experts, L.top_k, False, q, qs, ids, w,
                                 want_intermediates=True)
        assert not oracle.set_bf16_intermediate(False)
    finally:
        oracle.set_exact_rows(old)
    assert _same_bits(mid1["h"], _torch_bf16(mid0["h"]))
    hq2, hs2 = bruteforce.quant(mid1["h"])
    np.testing.assert_array_equal(mid1["hq"], hq2)
    np.testing.assert_array_equal(mid1["hs"], hs2)
