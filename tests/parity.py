"""Parity helpers: GPU results against the oracle.

Tolerance for fp32 outputs (per row t): |gpu - oracle| <= 1e-3 * max|oracle[t]| + 1e-6.

The one place where floating point decides an integer inside the layer is the
group-32 requant of the SwiGLU output.  Both sides take that decision in fp32,
but from fp32 projections accumulated in different orders (GPU: fp32 sums per
block in K order; oracle: fp64 sum rounded once), so a code whose oracle value
h/d sits within FLIP_EPS of a rounding boundary may legitimately land on the
neighbouring integer.  `check_hidden` accepts exactly those, and
`flip_bound` widens the row tolerance of y by the largest change such a flip
can cause, computed from the oracle's own quantities (its w, its d_h and the
dequantised down-projection column) -- never from GPU values.
"""
import os

import numpy as np

import oracle

TOL_REL, TOL_ABS = 1e-3, 1e-6
# |GPU h/d - oracle h/d| in code units: the fp32 projections differ by a few
# ulp (<= ~1e-6 relative), |h/d| <= 127 -> <= ~1.3e-4; 1e-3 leaves margin.
FLIP_EPS = 1e-3

_E2M1 = None


def host_threads():
    """Oracle threads for the parity tests: the host cores this process may
    use, at most 16 (a GPU machine's share).  The oracle splits work over rows and
    assignments only, so its results do not depend on the count."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def use_host_threads():
    oracle.set_threads(host_threads())


def e2m1_values():
    global _E2M1
    if _E2M1 is None:
        _E2M1 = np.array([oracle.e2m1(c) for c in range(16)], np.float64)
    return _E2M1


def row_tol(y_o):
    return TOL_REL * np.abs(y_o).max(axis=1) + TOL_ABS


def assert_rows_close(y_gpu, y_o, extra=None, what="y"):
    y_gpu = np.asarray(y_gpu, np.float64)
    y_o = np.asarray(y_o, np.float64)
    assert y_gpu.shape == y_o.shape, (y_gpu.shape, y_o.shape)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite GPU output"
    tol = row_tol(y_o)
    if extra is not None:
        tol = tol + extra
    err = np.abs(y_gpu - y_o).max(axis=1)
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, (f"{what}: {bad.size} rows out of tolerance, first row {bad[0]}: "
                           f"err {err[bad[0]]:.3e} tol {tol[bad[0]]:.3e}")
    return float((err / tol).max())


def boundary_mask(h, hs):
    """Codes whose oracle value h/d lies within FLIP_EPS of a .5 rounding boundary."""
    h = np.asarray(h, np.float32)
    d = np.repeat(np.asarray(hs, np.float32), 32, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(d > 0, h.astype(np.float64) / d.astype(np.float64), 0.0)
    frac = np.abs(r - np.floor(r) - 0.5)
    return (frac < FLIP_EPS) & (d > 0)


def hidden_error_bound(gu_codes, gu_scales, q_row, qs_row):
    """Bound on |h_gpu - h_oracle| for every feature of one (token, expert).

    The GPU forms each gate and up value as an fp32 sum of nb = d_model/32
    block terms t_b = dot_b * 2^(u_b - 128) * d_b (each exact, folded in with
    one rounding) plus a few run additions, so its error is at most
    (nb + 8) * 2^-24 * sum_b |t_b|; the oracle's value is the exact sum
    rounded once.  Through SwiGLU, h = silu(g) * u moves by at most
    |silu'(g)| |u| dg + (|silu(g)| + |silu'(g)| dg) du, plus the rounding of
    the SwiGLU arithmetic itself (the exp within 1 ulp, a division and a
    product: 8 ulp of |h| covers them).  Well-conditioned sums keep this far
    below FLIP_EPS; block scales spread over many binades make sum_b |t_b|
    much larger than |g| and the bound grows with it.  sum_b |t_b| comes from
    the oracle's exact integer block dots, g and u from its matvec."""
    gu_codes = np.asarray(gu_codes, np.uint8)
    F = gu_codes.shape[0] // 2
    q_row = np.asarray(q_row, np.int8)[None, :]
    qs_row = np.asarray(qs_row, np.float32)[None, :]
    gu = oracle.matvec(gu_codes, gu_scales, q_row, qs_row)[0].astype(np.float64)
    dots = oracle.block_dots(gu_codes, q_row)[0].astype(np.float64)     # [2F][nb], dot x 2
    sc = np.exp2(np.asarray(gu_scales, np.float64) - 128.0) * qs_row.astype(np.float64)
    a = (np.abs(dots) * sc).sum(axis=1)
    gamma = (dots.shape[1] + 8) * 2.0 ** -24
    g, u = gu[:F], gu[F:]
    dg, du = gamma * a[:F], gamma * a[F:]
    with np.errstate(over="ignore", invalid="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = np.abs(sig * (1.0 + g * (1.0 - sig)))
    return (dsilu * np.abs(u) * dg + (np.abs(silu) + dsilu * dg) * du
            + 8 * 2.0 ** -24 * np.abs(silu * u) + 1e-37)


def check_hidden(hq_gpu, hs_gpu, hq_o, hs_o, h_o, dh_fn=None):
    """GPU requant codes/scales vs the oracle's.  Returns per-element weights:
    how many code units each GPU code sits from the oracle's (0 where equal).

    First the plain bar: group scales within 1e-5 relative, and a code off by
    one only where the oracle's h/d lies within FLIP_EPS of a .5 boundary.
    Rows that miss it are checked again against the bound of their arithmetic
    (dh_fn(i) -> hidden_error_bound of row i): a group scale may then differ
    by max(dh)/127 over its group (the amax moves by at most the largest
    element error) plus 2 ulp, and a code may move by up to floor(e) + 1 where
    the oracle's h/d lies within e + FLIP_EPS of a boundary, e being the
    bound of |h_gpu/d_gpu - h_o/d_o| in code units."""
    hq_gpu = np.asarray(hq_gpu, np.int32)
    hq_o = np.asarray(hq_o, np.int32)
    hs_gpu = np.asarray(hs_gpu, np.float32)
    hs_o = np.asarray(hs_o, np.float32)
    diff = hq_gpu - hq_o
    flips = diff != 0
    near = boundary_mask(h_o, hs_o) if flips.any() else np.zeros(diff.shape, bool)
    s_bad = np.abs(hs_gpu.astype(np.float64) - hs_o) > 1e-5 * np.abs(hs_o.astype(np.float64))
    c_bad = flips & (~near | (np.abs(diff) > 1))
    bad_rows = np.nonzero(s_bad.any(axis=1) | c_bad.any(axis=1))[0]
    assert dh_fn is not None or bad_rows.size == 0, (
        f"hidden codes/scales of {bad_rows.size} rows outside the plain bar "
        f"(scales {int(s_bad.sum())}, codes {int(c_bad.sum())}) and no error bound given")
    F = hq_o.shape[1]
    for r in bad_rows:
        dh = np.asarray(dh_fn(r), np.float64)
        d_o = np.repeat(hs_o[r].astype(np.float64), 32)
        d_g = np.repeat(hs_gpu[r].astype(np.float64), 32)
        s_tol = (dh.reshape(F // 32, 32).max(axis=1) / 127.0
                 + 2 * np.spacing(hs_o[r]).astype(np.float64))
        ds = np.abs(hs_gpu[r].astype(np.float64) - hs_o[r])
        assert np.all(ds <= np.maximum(s_tol, 1e-5 * np.abs(hs_o[r]))), (
            f"hidden scale of row {r} beyond its error bound: {ds.max():.3e} "
            f"> {s_tol[np.argmax(ds - s_tol)]:.3e}")
        with np.errstate(divide="ignore", invalid="ignore"):
            x_o = np.where(d_o > 0, np.asarray(h_o[r], np.float64) / d_o, 0.0)
            e = np.where(d_o > 0, dh / d_o + np.abs(x_o) * np.abs(d_g - d_o) / d_o, 0.0)
        dist = np.abs(x_o - np.floor(x_o) - 0.5)
        f = np.nonzero(diff[r])[0]
        ok = (dist[f] <= e[f] + FLIP_EPS) & (np.abs(diff[r, f]) <= np.floor(e[f]) + 1)
        assert np.all(ok), (f"hidden code of row {r} beyond its error bound: feature "
                            f"{f[~ok][0]}, diff {diff[r, f[~ok][0]]}, e {e[f[~ok][0]]:.3e}")
    return np.abs(diff).astype(np.float64)


def bf16_tie_mask(h_pre, hs):
    """Elements whose oracle value before the BF16 rounding lies within
    FLIP_EPS * d of a BF16 rounding midpoint (either neighbour): there the GPU,
    from projections a few ulp away, may round to the other BF16 value."""
    h = np.ascontiguousarray(h_pre, np.float32)
    mag = h.view(np.uint32) & np.uint32(0x7FFFFFFF)
    base = mag & np.uint32(0xFFFF0000)
    up = (base | np.uint32(0x8000)).view(np.float32).astype(np.float64)
    dn = np.where(base > 0, base - np.uint32(0x8000), np.uint32(0)).astype(np.uint32)
    dn = dn.view(np.float32).astype(np.float64)
    a = np.abs(h.astype(np.float64))
    d = np.repeat(np.asarray(hs, np.float64), 32, axis=1)
    eps = FLIP_EPS * d
    return (np.abs(a - up) <= eps) | ((base > 0) & (np.abs(a - dn) <= eps))


def check_hidden_bf16(hq_gpu, hs_gpu, hq_o, hs_o, h_o, h_pre):
    """check_hidden for the BF16-intermediate mode.  A code may also move where
    the oracle's pre-rounding value sits at a BF16 midpoint (one BF16 step is at
    most 2^-7 |h| <= d, so at most 2 code units), and a group scale may move only
    when its largest element sits there; such a group's codes may then all move
    by up to 2.  Returns per-element flip weights in units of d * |W_down|."""
    hq_gpu = np.asarray(hq_gpu, np.int32)
    hq_o = np.asarray(hq_o, np.int32)
    hs_gpu = np.asarray(hs_gpu, np.float64)
    hs_o64 = np.asarray(hs_o, np.float64)
    tie = bf16_tie_mask(h_pre, hs_o)
    n, F = hq_o.shape
    G = F // 32
    a = np.abs(np.asarray(h_o, np.float64)).reshape(n, G, 32)
    top = a >= a.max(axis=2, keepdims=True) * (1 - 2.0 ** -6)
    tie_top = (tie.reshape(n, G, 32) & top).any(axis=2)
    same = np.isclose(hs_gpu, hs_o64, rtol=1e-5, atol=0)
    moved = ~same
    assert np.all(tie_top[moved]), "hidden scale moved without a BF16 midpoint at its max"
    assert np.all(np.abs(hs_gpu[moved] / hs_o64[moved] - 1) <= 2.0 ** -6), "hidden scale"
    diff = hq_gpu - hq_o
    weights = np.zeros((n, F), np.float64)
    g_moved = np.repeat(moved, 32, axis=1)
    weights[g_moved] = 3.0
    flips = (diff != 0) & ~g_moved
    if flips.any():
        near = boundary_mask(h_o, hs_o) | tie
        assert np.all(np.abs(diff[flips]) <= 2), "hidden code off by more than 2"
        assert np.all(near[flips]), "hidden code flipped away from a rounding boundary"
        weights[flips] = np.abs(diff[flips])
    assert np.all(np.abs(diff[g_moved]) <= 2), "hidden code off by more than 2"
    return weights


def flip_bound(flips, slot_weight, hs_o, down_col_absmax):
    """Per-token widening of the y tolerance for legitimate requant flips.

    flips:          bool [rows*(k+1)][F] (oracle row order)
    slot_weight:    f32  [rows*(k+1)] oracle combine weight of each hidden row
    hs_o:           f32  [rows*(k+1)][F/32] oracle hidden scales
    down_col_absmax: callable(row) -> f64 [F], max_n |W_down[n][f]| of that row's expert
    A numeric `flips` weights each element (code units it may have moved by).
    """
    n_rows, F = flips.shape
    out = np.zeros(n_rows, np.float64)
    for r in np.nonzero(flips.any(axis=1))[0]:
        f = np.nonzero(flips[r])[0]
        m = np.asarray(flips[r, f], np.float64)
        out[r] = np.sum(abs(float(slot_weight[r])) * hs_o[r, f // 32].astype(np.float64) *
                        down_col_absmax(r)[f] * m) * (1 + 1e-6)
    return out


def down_col_absmax(down_codes, down_scales):
    """max over output rows n of |dequantised W_down[n][f]|, for every f."""
    codes = np.asarray(down_codes, np.uint8)
    n, half = codes.shape
    nib = np.empty((n, half * 2), np.uint8)
    nib[:, 0::2], nib[:, 1::2] = codes & 0xF, codes >> 4
    vals = np.abs(e2m1_values()[nib])
    sc = np.power(2.0, np.asarray(down_scales, np.float64) - 127.0)
    return (vals * np.repeat(sc, 32, axis=1)).max(axis=0)


def covering_rows(ids, n_experts, top_k, rows, tile, base, seed):
    """A seeded sample of prefill rows for the parity check that still touches
    every part of the grouped GEMM: `base` random rows and the last row, plus
    rows so that every routed expert's last sorted assignment (the last row of
    its ragged last tile) is in, every row offset (sorted position - expert
    offset) mod `tile` of a routed tile occurs, and every token offset mod
    `tile` of the shared expert's tiles occurs.  ids: the oracle's routes
    (negative = not owned), grouped here by the oracle."""
    counts, offsets, srt = oracle.group(ids, n_experts)
    rng = np.random.default_rng(seed)
    pick = {rows - 1}
    pick.update(int(t) for t in rng.choice(rows, min(base, rows), replace=False))
    n_valid = int(offsets[-1])
    expert_of = np.repeat(np.arange(n_experts), counts)
    r_off = (np.arange(n_valid) - offsets[expert_of]) % tile
    tok = srt[:n_valid] // top_k
    for e in range(n_experts):
        if counts[e]:
            pick.add(int(tok[offsets[e + 1] - 1]))
    have = set(int(v) for v in r_off[np.isin(tok, sorted(pick))])
    for v in np.unique(r_off):
        if int(v) not in have:
            t = int(tok[rng.choice(np.nonzero(r_off == v)[0])])
            pick.add(t)
            have.update(int(x) for x in r_off[tok == t])
    shared = set(t % tile for t in pick)
    for v in range(min(tile, rows)):
        if v not in shared:
            pick.add(int(rng.choice(np.arange(v, rows, tile))))
    return np.array(sorted(pick))


def e3m2_value(code):
    """Value of a 6-bit E3M2 code (sign bit 5, exponent bits 4-2 with bias 3,
    mantissa bits 1-0; exponent 0 is subnormal), per the OCP microscaling
    format's FP6 E3M2 element."""
    code = np.asarray(code, np.int64)
    e, m = (code >> 2) & 7, code & 3
    mag = np.where(e == 0, m / 4.0 * 2.0 ** -2, (1 + m / 4.0) * 2.0 ** (e.astype(np.float64) - 3))
    return np.where(code & 32, -mag, mag)


def codes_from_digit_planes(raw, d_ff):
    """Hidden codes stored as E3M2 digit planes (the prefill GEMM's workspace
    format): per row, d_ff/32 blocks of 48 bytes in the first 1.5 d_ff bytes
    -- plane 0 bytes 0-15, plane 1 bytes 0-15, plane 0 bytes 16-23, plane 1
    bytes 16-23 -- plane s a 192-bit little-endian word holding digit s of the
    block's element e in bits 6e..6e+5; code = d0 + 16 d1.  raw: uint8
    [rows][>= 1.5 d_ff].  A digit that is not an integer in [-8, 8], or a
    low digit outside [-8, 7], is an error."""
    raw = np.asarray(raw, np.uint8)
    nb = d_ff // 32
    blk = raw[:, :nb * 48].reshape(raw.shape[0], nb, 48)
    planes = [np.concatenate([blk[:, :, 0:16], blk[:, :, 32:40]], axis=2),
              np.concatenate([blk[:, :, 16:32], blk[:, :, 40:48]], axis=2)]
    digits = []
    for pl in planes:
        bits = np.unpackbits(pl, axis=2, bitorder="little")  # [rows][nb][192]
        six = bits.reshape(raw.shape[0], nb, 32, 6)
        code = (six * (1 << np.arange(6))).sum(axis=3)
        v = e3m2_value(code)
        assert np.all((v == np.round(v)) & (np.abs(v) <= 8)), \
            "hidden digit plane holds a code that is not an integer digit in [-8, 8]"
        digits.append(v.astype(np.int32))
    assert np.all(digits[0] <= 7), "low hidden digit outside [-8, 7]"
    return (digits[0] + 16 * digits[1]).reshape(raw.shape[0], d_ff)
