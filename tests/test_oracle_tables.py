"""Pins for the oracle's decode tables and block dot (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from conftest import golden_lines


def test_e2m1_matches_printed_set():
    # gfx90a report, section 6.1: nibble -> {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12}
    mags = [int(x) for x in golden_lines("e2m1_x2_values.txt")]
    got = [oracle.e2m1_x2(c) for c in range(16)]
    assert sorted(set(got)) == sorted(set(mags) | {-m for m in mags})
    # codes 0..7 take the listed magnitudes in the listed order; bit 3 is the sign
    assert got[:8] == mags
    assert got[8:] == [-m for m in mags]
    assert oracle.e2m1(1) == 0.5 and oracle.e2m1(7) == 6.0 and oracle.e2m1(13) == -3.0


def test_e2m1_negative_zero_is_zero():
    assert oracle.e2m1_x2(8) == 0
    assert oracle.e2m1(8) == 0.0


def test_e8m0_closed_form():
    for line in golden_lines("e8m0_values.txt"):
        u, v = line.split()
        want = 2.0 ** int(v[2:]) if v.startswith("2^") else float(v)
        assert oracle.e8m0(int(u)) == want
    assert math.isnan(oracle.e8m0(255))


def _parse_dot_line(line):
    name, cod, q, want = [p.strip() for p in line.split("|")]
    codes = np.array([int(b, 16) for b in cod.split()], np.uint8)
    qv = np.array([int(v) for v in q.split()], np.int8)
    return name, codes, qv, int(want)


def test_block_dot_worked_examples():
    lines = golden_lines("block_dot_worked.txt")
    assert len(lines) == 6
    for line in lines:
        name, codes, qv, want = _parse_dot_line(line)
        assert codes.size == 16 and qv.size == 32, name
        assert oracle.block_dot(codes, qv) == want, name


def test_block_dot_bruteforce_int64():
    # against an int64 brute force built on the printed table
    from bruteforce import e2m1_table
    tab = e2m1_table()
    rng = np.random.default_rng(7)
    for _ in range(200):
        codes = rng.integers(0, 256, 16, dtype=np.uint8)
        q = rng.integers(-127, 128, 32, dtype=np.int8)
        nib = np.empty(32, np.int64)
        nib[0::2], nib[1::2] = codes & 0xF, codes >> 4
        assert oracle.block_dot(codes, q) == int(np.dot(tab[nib], q.astype(np.int64)))


def test_block_dots_layout():
    # dots[t][n][b] indexes (activation row, weight row, block)
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, (5, 64), dtype=np.uint8)  # 5 rows, d_in 128
    q = rng.integers(-127, 128, (3, 128), dtype=np.int8)
    dots = oracle.block_dots(codes, q)
    assert dots.shape == (3, 5, 4)
    for t in range(3):
        for n in range(5):
            for b in range(4):
                assert dots[t, n, b] == oracle.block_dot(codes[n, b * 16:(b + 1) * 16],
                                                         q[t, b * 32:(b + 1) * 32])
