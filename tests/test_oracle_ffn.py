"""Pins for the oracle's projections, SwiGLU, combine and whole layer (CPU only)."""
import math

import numpy as np
import pytest

import bruteforce
import oracle
import synth


def _rand_weights(rng, n_out, d_in, exp_lo=-8, exp_hi=0):
    codes = rng.integers(0, 256, (n_out, d_in // 2), dtype=np.uint8)
    scales = (127 + rng.integers(exp_lo, exp_hi + 1, (n_out, d_in // 32))).astype(np.uint8)
    return codes, scales


def _ulp_close(a, b, ulps=1):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    tol = ulps * np.spacing(np.abs(b).astype(np.float32)).astype(np.float64) + 1e-40
    return np.all(np.abs(a - b) <= tol)


def test_matvec_vs_dequantised_fp64():
    rng = np.random.default_rng(0)
    codes, scales = _rand_weights(rng, 48, 256, -20, 20)  # non-constant scales
    x = rng.standard_normal((5, 256)).astype(np.float32)
    q, qs = oracle.quant_q8(x)
    y = oracle.matvec(codes, scales, q, qs)
    ref = bruteforce.matvec(codes, scales, q, qs)
    assert y.dtype == np.float32 and y.shape == (5, 48)
    assert _ulp_close(y, ref, 1)


def test_matvec_integer_exact_fixture():
    # d = 1 in every block (integer x with a +-127 in each block) and u = 127:
    # y = sum(value * q) exactly, a multiple of 0.5 well inside fp32's range
    rng = np.random.default_rng(1)
    codes, _ = _rand_weights(rng, 32, 512)
    scales = np.full((32, 16), 127, np.uint8)
    x = rng.integers(-127, 128, (3, 512)).astype(np.float32)
    x[:, ::32] = 127
    q, qs = oracle.quant_q8(x)
    assert np.all(qs == 1.0) and np.array_equal(q.astype(np.float32), x)
    tab = bruteforce.e2m1_table()
    nib = np.empty((32, 512), np.int64)
    nib[:, 0::2], nib[:, 1::2] = codes & 0xF, codes >> 4
    want2 = q.astype(np.int64) @ tab[nib].T  # 2*y, exact integers
    y = oracle.matvec(codes, scales, q, qs)
    np.testing.assert_array_equal(y.astype(np.float64) * 2, want2.astype(np.float64))


def test_matvec_scale_fingerprint():
    # non-constant per-row, per-block scales: rows differ only in their scale
    # pattern, so a transposed or shifted scale index changes the result
    codes = np.full((16, 64), 0x22, np.uint8)          # every weight 1.0
    scales = (120 + (np.arange(16)[:, None] + 3 * np.arange(4)[None, :]) % 9).astype(np.uint8)
    x = np.ones((1, 128), np.float32) * 127
    q, qs = oracle.quant_q8(x)
    y = oracle.matvec(codes, scales, q, qs)[0]
    want = [sum(32 * 127 * 2.0 ** (int(u) - 127) for u in scales[n]) for n in range(16)]
    np.testing.assert_array_equal(y, np.float32(want))


def test_swiglu_closed_forms():
    g = np.float32([0.0, 1.0, -1.0, 40.0, -800.0, 2.0])
    u = np.float32([3.0, 2.0, 2.0, 0.5, 1.0, -1.0])
    h = oracle.swiglu(g, u)
    assert h[0] == 0.0
    assert h[1] == np.float32(2 * 0.7310585786300049)
    assert h[2] == np.float32(2 * -0.2689414213699951)
    assert h[3] == np.float32(20.0)
    assert h[4] == 0.0 and math.copysign(1.0, h[4]) == -1.0  # silu(-800) -> -0
    assert h[5] == np.float32(-2.0 / (1 + math.exp(-2.0)))


def _layer_inputs(rng, E, k, D, F, T, shared):
    experts = {}
    for e in range(E + (1 if shared else 0)):
        gc, gs = _rand_weights(rng, 2 * F, D)
        dc, ds = _rand_weights(rng, D, F)
        experts[e] = dict(gate_up_codes=gc, gate_up_scales=gs, down_codes=dc, down_scales=ds)
    x = rng.standard_normal((T, D)).astype(np.float32)
    q, qs = oracle.quant_q8(x)
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    return experts, q, qs, ids, w


@pytest.mark.parametrize("shared", [False, True])
def test_ffn_vs_bruteforce(shared):
    rng = np.random.default_rng(21)
    E, k, D, F, T = 6, 2, 128, 96, 3
    experts, q, qs, ids, w = _layer_inputs(rng, E, k, D, F, T, shared)
    y, mid = oracle.ffn(experts, E, k, shared, q, qs, ids, w, want_intermediates=True)
    ref = bruteforce.ffn(experts, E, k, shared, q, qs, ids, w)
    assert _ulp_close(y, ref, 2)
    # intermediate codes agree with a numpy requant of the oracle's own h
    hq2, hs2 = bruteforce.quant(mid["h"])
    np.testing.assert_array_equal(mid["hq"], hq2)
    np.testing.assert_array_equal(mid["hs"], hs2)


def test_ffn_tiny_workload_vs_bruteforce():
    cfg = synth.TINY
    L = cfg["layer"]
    experts = {e: {k: v.numpy() for k, v in synth.expert_weights(cfg["seed"], 0, e, L.d_model,
                                                                 L.d_ff).items()}
               for e in range(L.n_experts)}
    x = synth.activations(cfg["seed"], 0, cfg["rows"], L.d_model)
    q, qs = oracle.quant_q8(x)
    ids, w = oracle.route(synth.router_logits(cfg["seed"], 0, cfg["rows"], L.n_experts), L.top_k)
    y = oracle.ffn(experts, L.n_experts, L.top_k, False, q, qs, ids, w)
    ref = bruteforce.ffn(experts, L.n_experts, L.top_k, False, q, qs, ids, w)
    assert _ulp_close(y, ref, 2)
    assert np.all(np.isfinite(y)) and np.abs(y).max() > 0


def test_ffn_identical_experts_equal_one_expert():
    # all experts share one weight set; weights sum to 1, so y == that expert's output
    rng = np.random.default_rng(8)
    E, k, D, F, T = 8, 3, 64, 64, 4
    one = dict(zip(("gate_up_codes", "gate_up_scales"), _rand_weights(rng, 2 * F, D)))
    one.update(zip(("down_codes", "down_scales"), _rand_weights(rng, D, F)))
    experts = {e: one for e in range(E)}
    x = rng.standard_normal((T, D)).astype(np.float32)
    q, qs = oracle.quant_q8(x)
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    y, mid = oracle.ffn(experts, E, k, False, q, qs, ids, w, want_intermediates=True)
    Y0 = mid["Y"].reshape(T, k + 1, D)[:, 0, :]
    assert _ulp_close(y, Y0, 2)


def test_ffn_top1_and_sentinels():
    rng = np.random.default_rng(12)
    E, D, F, T = 5, 64, 32, 3
    experts, q, qs, ids, w = _layer_inputs(rng, E, 1, D, F, T, True)
    # k = 1, no shared: y is exactly the routed expert's output (weight 1.0)
    y, mid = oracle.ffn(experts, E, 1, False, q, qs, ids, w, want_intermediates=True)
    assert np.all(w == 1.0)
    np.testing.assert_array_equal(y, mid["Y"].reshape(T, 2, D)[:, 0, :])
    # every route a sentinel: only the shared expert contributes
    neg = np.full_like(ids, -1)
    y2, mid2 = oracle.ffn(experts, E, 1, True, q, qs, neg, w, want_intermediates=True)
    np.testing.assert_array_equal(y2, mid2["Y"].reshape(T, 2, D)[:, 1, :])


def test_ffn_from_given_hidden_codes():
    # restarting the down projection from the oracle's own h codes reproduces y
    rng = np.random.default_rng(13)
    E, k, D, F, T = 4, 2, 64, 64, 2
    experts, q, qs, ids, w = _layer_inputs(rng, E, k, D, F, T, True)
    y, mid = oracle.ffn(experts, E, k, True, q, qs, ids, w, want_intermediates=True)
    y2 = oracle.ffn(experts, E, k, True, q, qs, ids, w, hq_in=mid["hq"], hs_in=mid["hs"])
    np.testing.assert_array_equal(y, y2)


def test_threads_do_not_change_results():
    rng = np.random.default_rng(14)
    E, k, D, F, T = 6, 2, 64, 64, 5
    experts, q, qs, ids, w = _layer_inputs(rng, E, k, D, F, T, True)
    oracle.set_threads(1)
    y1 = oracle.ffn(experts, E, k, True, q, qs, ids, w)
    oracle.set_threads(4)
    y4 = oracle.ffn(experts, E, k, True, q, qs, ids, w)
    oracle.set_threads(1)
    np.testing.assert_array_equal(y1, y4)
