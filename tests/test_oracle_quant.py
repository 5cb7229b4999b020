"""Pins for the oracle's per-32-block int8 quantiser (CPU only)."""
import numpy as np
import pytest

import oracle
from bruteforce import quant as np_quant
from conftest import golden_lines


def _parse(line):
    name, d, x, q = [p.strip() for p in line.split("|")]
    return (name, np.float32(d), np.array([float(v) for v in x.split()], np.float32),
            np.array([int(v) for v in q.split()], np.int8))


def test_worked_blocks():
    lines = golden_lines("quant_worked.txt")
    assert len(lines) == 4
    for line in lines:
        name, d, x, want = _parse(line)
        q, s = oracle.quant_q8(x[None, :])
        assert s[0, 0] == d, name
        np.testing.assert_array_equal(q[0], want, err_msg=name)


def test_invariants_random():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((37, 256)) * rng.uniform(1e-3, 50, (37, 1))).astype(np.float32)
    q, s = oracle.quant_q8(x)
    xb = x.reshape(37, 8, 32)
    qb = q.reshape(37, 8, 32).astype(np.int32)
    assert np.all(np.abs(qb) <= 127)
    # the absmax element of every block maps to +-127
    idx = np.argmax(np.abs(xb), axis=2)
    top = np.take_along_axis(qb, idx[:, :, None], 2)[:, :, 0]
    assert np.all(np.abs(top) == 127)
    # reconstruction error at most half a step (plus the rounding of x/d)
    err = np.abs(xb.astype(np.float64) - qb * s[:, :, None].astype(np.float64))
    assert np.all(err <= s[:, :, None] * 0.5 * (1 + 2.0 ** -20))
    # odd symmetry
    qn, sn = oracle.quant_q8(-x)
    np.testing.assert_array_equal(qn, -q)
    np.testing.assert_array_equal(sn, s)


def test_single_nonzero_and_zero_blocks():
    x = np.zeros((2, 64), np.float32)
    x[0, 5] = np.float32(3.3)
    x[1, 40] = np.float32(-1e-30)
    q, s = oracle.quant_q8(x)
    assert q[0, 5] == 127 and np.count_nonzero(q[0]) == 1
    assert s[0, 1] == 0 and np.all(q[0, 32:] == 0)
    assert q[1, 40] == -127 and s[1, 0] == 0


def test_matches_numpy_quantiser():
    # an independent numpy float32 implementation of the same reading
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    q, s = oracle.quant_q8(x)
    q2, s2 = np_quant(x)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s, s2)
