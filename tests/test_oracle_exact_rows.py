"""Pins for the oracle's exact-rows mode (CPU only): fp32 arithmetic in one
named order ([strix] "The exact-rows contract"), pinned against exact rational
arithmetic, IEEE single-precision emulation in numpy, the fp64 reference mode
and the mathematical exp -- never against the mode itself."""
import math
from fractions import Fraction

import numpy as np
import pytest

import bruteforce
import oracle
import synth


def _f32(fr: Fraction) -> float:
    """The float32 nearest to an exact rational (ties to even; normal range)."""
    if fr == 0:
        return 0.0
    sign = -1.0 if fr < 0 else 1.0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    scaled = a / Fraction(2) ** (e - 23)          # in [2^23, 2^24)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return sign * m * 2.0 ** (e - 23)


def _fma(a, b, c) -> float:
    """IEEE fused multiply-add in float32, from its definition."""
    return _f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def test_exp_rows_within_one_ulp_of_exp():
    x = np.linspace(-87.0, 88.7, 400_001, dtype=np.float32)
    y = oracle.exp_rows(x).astype(np.float64)
    t = np.exp(x.astype(np.float64))
    ulp = np.spacing(t.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(y - t) / ulp) <= 1.0
    sp = oracle.exp_rows(np.array([0.0, -0.0, -200.0, 100.0, np.nan], np.float32))
    assert sp[0] == 1.0 and sp[1] == 1.0 and sp[2] == 0.0 and np.isinf(sp[3])
    assert np.isnan(sp[4])


def test_exp_rows_steps_by_definition():
    # the named sequence retyped from its definition with exact rational fmas
    log2e, hi, lo = (float.fromhex(h) for h in ('0x1.715476p+0', '0x1.62e4p-1',
                                               '0x1.7f7d1cp-20'))
    c = [np.float32(1.0 / math.factorial(n)) for n in range(8)]
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.uniform(-80, 80, 200), [0.5, -0.5, 1e-3, 20.0]]).astype(np.float32)
    got = oracle.exp_rows(xs)
    for x, g in zip(xs, got):
        k = np.rint(np.float32(x) * np.float32(log2e))
        r = _fma(-k, hi, x)
        r = _fma(-k, lo, r)
        p = float(c[7])
        for n in range(6, -1, -1):
            p = _fma(p, r, c[n])
        assert np.float32(math.ldexp(p, int(k))) == g, x


def _weights(rng, n_out, d_in):
    codes = rng.integers(0, 256, (n_out, d_in // 2), dtype=np.uint8)
    scales = (127 + rng.integers(-8, 1, (n_out, d_in // 32))).astype(np.uint8)
    return codes, scales


def test_exact_matvec_matches_rational_run_order():
    # runs of 16 blocks, block terms folded with fmaf from zero, runs added in
    # order -- emulated with exact rationals rounded per operation
    rng = np.random.default_rng(4)
    n_out, d_in, rows = 3, 1024 + 512, 2       # three runs, the last one full
    codes, scales = _weights(rng, n_out, d_in)
    x = rng.standard_normal((rows, d_in)).astype(np.float32)
    q, qs = oracle.quant_q8(x)
    with oracle.exact_rows():
        y = oracle.matvec(codes, scales, q, qs)
    x2 = bruteforce.e2m1_table()        # twice the E2M1 value of each code
    for t in range(rows):
        for n in range(n_out):
            total = 0.0
            for b0 in range(0, d_in // 32, 16):
                run = 0.0
                for b in range(b0, b0 + 16):
                    nib = codes[n, b * 16:(b + 1) * 16]
                    w = [int(x2[c]) for byte in nib for c in (byte & 15, byte >> 4)]
                    dot = sum(wi * int(qi) for wi, qi in zip(w, q[t, b * 32:(b + 1) * 32]))
                    term = Fraction(dot) * Fraction(2) ** (int(scales[n, b]) - 128)
                    assert _f32(term) == float(term)        # exact in fp32
                    run = _fma(float(term), qs[t, b], run)
                total = _f32(Fraction(total) + Fraction(run))
            assert np.float32(total) == y[t, n], (t, n)


def test_exact_matvec_close_to_fp64_reference():
    rng = np.random.default_rng(5)
    codes, scales = _weights(rng, 64, 2048)
    q, qs = oracle.quant_q8(rng.standard_normal((4, 2048)).astype(np.float32))
    ref = oracle.matvec(codes, scales, q, qs)
    with oracle.exact_rows():
        y = oracle.matvec(codes, scales, q, qs)
    assert np.max(np.abs(y - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_exact_swiglu_and_route_weights_by_fp32_emulation():
    rng = np.random.default_rng(6)
    g = (rng.standard_normal(4096) * 4).astype(np.float32)
    u = rng.standard_normal(4096).astype(np.float32)
    with oracle.exact_rows():
        h = oracle.swiglu(g, u)
    den = np.float32(1.0) + oracle.exp_rows(-g)
    np.testing.assert_array_equal(h, (g / den) * u)           # numpy float32 = IEEE single
    h64 = oracle.swiglu(g, u)                                   # fp64 reference mode
    assert np.max(np.abs(h - h64) / (np.abs(h64) + 1e-30)) < 4e-7
    logits = synth.router_logits(7, 0, 6, 256)
    ids0, w0 = oracle.route(logits, 6)
    with oracle.exact_rows():
        ids, w = oracle.route(logits, 6)
    np.testing.assert_array_equal(ids, ids0)
    np.testing.assert_allclose(w, w0, rtol=2e-6)
    for t in range(6):
        sig = np.float32(1.0) / (np.float32(1.0) + oracle.exp_rows(-logits[t, ids[t]]))
        s = np.float32(0.0)
        for v in sig:
            s = np.float32(s + v)
        np.testing.assert_array_equal(w[t], sig / s)
        assert abs(float(np.sum(w[t], dtype=np.float64)) - 1.0) < 1e-6


def test_exact_combine_by_rational_fma():
    rng = np.random.default_rng(8)
    T, k, D = 3, 4, 16
    ids = rng.integers(0, 8, (T, k)).astype(np.int32)
    ids[1, 2] = -1                                             # a sentinel slot
    w = rng.random((T, k)).astype(np.float32)
    Y = rng.standard_normal((T * (k + 1), D)).astype(np.float32)
    with oracle.exact_rows():
        y = oracle.combine(ids, w, Y, True)
    for t in range(T):
        for n in range(D):
            v = 0.0
            for i in range(k):
                if ids[t, i] >= 0:
                    v = _fma(w[t, i], Y[t * (k + 1) + i, n], v)
            v = float(np.float32(v) + Y[t * (k + 1) + k, n])
            assert np.float32(v) == y[t, n]


def test_exact_layer_close_to_fp64_reference():
    # the whole tiny layer in both modes: intermediates agree to fp32
    # rounding and y to the parity tolerance
    c = synth.TINY
    L = c["layer"]
    x = synth.activations(c["seed"], 0, c["rows"], L.d_model)
    lg = synth.router_logits(c["seed"], 0, c["rows"], L.n_experts)
    ex = {e: {k: v.numpy() for k, v in synth.expert_weights(c["seed"], 0, e, L.d_model,
                                                            L.d_ff).items()}
          for e in range(L.n_experts)}
    q, qs = oracle.quant_q8(x)
    ids, w = oracle.route(lg, L.top_k)
    y0, m0 = oracle.ffn(ex, L.n_experts, L.top_k, L.has_shared, q, qs, ids, w,
                        want_intermediates=True)
    with oracle.exact_rows():
        ids1, w1 = oracle.route(lg, L.top_k)
        y1, m1 = oracle.ffn(ex, L.n_experts, L.top_k, L.has_shared, q, qs, ids1, w1,
                            want_intermediates=True)
    np.testing.assert_array_equal(ids1, ids)
    assert np.max(np.abs(m1["h"] - m0["h"])) <= 1e-5 * np.max(np.abs(m0["h"]))
    row_max = np.max(np.abs(y0), axis=1, keepdims=True)
    assert np.all(np.abs(y1 - y0) <= 1e-3 * row_max + 1e-6)
