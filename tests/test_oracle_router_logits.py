"""Pins for the oracle's router projection (CPU only): BF16 hidden state times
BF16 router weights into fp32 logits ([gfx90a] Fig. 1 "Router Top-6", Table 4's
BF16 router GEMM).  The BF16 cast of x is torch's own, the sums are numpy's
fp64 matmul and, for the exact-rows order, exact rationals rounded to fp32 at
every step -- nothing here re-calls the oracle's own routine."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from test_oracle_exact_rows import _f32, _fma


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _wval(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _inputs(seed, rows, E, D):
    x = synth.normal(seed, 1, (rows, D))
    wr = synth.router_weights(seed, 0, E, D)
    return x, wr


@pytest.mark.parametrize("D", [32, 544, 4096])
def test_default_mode_is_fp64_sum_rounded_once(D):
    x, wr = _inputs(11, 5, 24, D)
    got = oracle.router_logits(x, wr)
    want = (_bf16(x).astype(np.float64) @ _wval(wr).astype(np.float64).T).astype(np.float32)
    ulp = np.spacing(np.abs(want)).astype(np.float64)
    assert np.all(np.abs(got.astype(np.float64) - want) <= ulp)
    assert np.mean(got == want) > 0.99


def _named_order(xb, w):
    """The exact-rows order retyped from its definition with exact rationals."""
    D = xb.size
    p = []
    for l in range(64):
        acc = 0.0
        for j in range((D + 511) // 512):
            for i in range(8):
                k = 512 * j + 8 * l + i
                if k < D:
                    acc = _fma(xb[k], w[k], acc)
        p.append(acc)
    m = 32
    while m >= 1:
        p = [_f32(Fraction(p[l]) + Fraction(p[l ^ m])) for l in range(64)]
        m //= 2
    return p[0]


@pytest.mark.parametrize("D", [64, 544, 1056])
def test_exact_mode_named_order(D):
    x, wr = _inputs(12, 2, 3, D)
    with oracle.exact_rows():
        got = oracle.router_logits(x, wr)
    xb, wv = _bf16(x), _wval(wr)
    for t in range(2):
        for e in range(3):
            assert got[t, e] == np.float32(_named_order(xb[t], wv[e])), (t, e)


def test_exact_mode_close_to_fp64():
    x, wr = _inputs(13, 4, 64, 4096)
    with oracle.exact_rows():
        ex = oracle.router_logits(x, wr).astype(np.float64)
    want = _bf16(x).astype(np.float64) @ _wval(wr).astype(np.float64).T
    mag = np.abs(_bf16(x)).astype(np.float64) @ np.abs(_wval(wr)).astype(np.float64).T
    assert np.all(np.abs(ex - want) <= mag * 2.0 ** -18)
    assert np.any(ex != oracle.router_logits(x, wr))    # a different order indeed


@pytest.mark.parametrize("exact", [False, True])
def test_closed_forms(exact):
    D, E = 512, 4
    wr = synth.router_weights(14, 0, E, D)
    wv = _wval(wr)
    old = oracle.set_exact_rows(exact)
    try:
        # one-hot hidden state: the logit is that weight times the value, exactly
        x = np.zeros((3, D), np.float32)
        x[0, 7], x[1, 300], x[2, 511] = 1.0, -3.0, 0.5
        lg = oracle.router_logits(x, wr)
        np.testing.assert_array_equal(lg[0], wv[:, 7])
        np.testing.assert_array_equal(lg[1], -3.0 * wv[:, 300])
        np.testing.assert_array_equal(lg[2], 0.5 * wv[:, 511])
        # the hidden state is rounded to BF16 first: 1 + 2^-9 acts as 1, and
        # 1 + 3 * 2^-8 as 1 + 2^-6
        x2 = np.zeros((2, D), np.float32)
        x2[0, 7] = 1.0 + 2.0 ** -9
        x2[1, 7] = 1.0 + 3 * 2.0 ** -8
        lg2 = oracle.router_logits(x2, wr)
        np.testing.assert_array_equal(lg2[0], wv[:, 7])
        np.testing.assert_array_equal(lg2[1], np.float32(1.0 + 2.0 ** -6) * wv[:, 7])
        # zero rows give zero logits; rows are independent
        z = oracle.router_logits(np.zeros((1, D), np.float32), wr)
        assert np.all(z == 0)
        xr = synth.normal(15, 2, (4, D))
        full = oracle.router_logits(xr, wr)
        np.testing.assert_array_equal(oracle.router_logits(xr[2:3], wr), full[2:3])
    finally:
        oracle.set_exact_rows(old)


def test_router_weights_generator_spread():
    wr = synth.router_weights(2, 0, 256, 4096)
    assert wr.dtype == np.uint16 and wr.shape == (256, 4096)
    v = _wval(wr)
    assert abs(float(v.std()) * 64 - 1) < 0.01
    x = synth.activations(2, 0, 8, 4096)
    lg = oracle.router_logits(x, wr)
    assert 0.8 < float(lg.std()) < 1.2
