"""Brute-force, dequantise-then-fp64 evaluation used to pin the oracle.

Written independently of oracle/: the E2M1 values come from the table typed in
tests/golden/e2m1_x2_values.txt (the list printed in the gfx90a report,
section 6.1), every weight is dequantised to float64 and the projections are
plain float64 matrix products.  Only for tiny shapes.
"""
import math

import numpy as np

from conftest import golden_lines


def e2m1_table():
    """code -> 2*value, codes 0..7 take the listed magnitudes in order, 8..15 negate."""
    mags = [int(x) for x in golden_lines("e2m1_x2_values.txt")]
    assert len(mags) == 8
    return np.array(mags + [-m for m in mags], dtype=np.int64)


def dequant_weights(codes, scales):
    """float64 [n_out][d_in] from canonical codes/scales."""
    codes = np.asarray(codes, np.uint8)
    scales = np.asarray(scales, np.uint8)
    n_out, half = codes.shape
    nib = np.empty((n_out, half * 2), np.int64)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    vals = e2m1_table()[nib].astype(np.float64) / 2.0
    blk_scale = np.power(2.0, scales.astype(np.float64) - 127.0)
    return vals * np.repeat(blk_scale, 32, axis=1)


def dequant_act(q, qs):
    q = np.asarray(q, np.int8).astype(np.float64)
    return q * np.repeat(np.asarray(qs, np.float32).astype(np.float64), 32, axis=1)


def matvec(codes, scales, q, qs):
    """float64 [rows][n_out]"""
    return dequant_act(q, qs) @ dequant_weights(codes, scales).T


def quant(x):
    """numpy float32 per-32 quantiser: d = amax/127, q = rint(x/d) (half even)."""
    x = np.asarray(x, np.float32)
    rows, cols = x.shape
    xb = x.reshape(rows, cols // 32, 32)
    amax = np.max(np.abs(xb), axis=2)
    d = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(d == 0, np.float32(1), d).astype(np.float32)
    qf = np.rint((xb / safe[:, :, None]).astype(np.float32))
    qf = np.clip(qf, -127, 127)
    qf[d == 0] = 0
    return qf.astype(np.int8).reshape(rows, cols), d


def route(logits, k):
    """full sort with key (-logit, index); sigmoid weights renormalised (fp64)."""
    lg = np.asarray(logits, np.float32)
    ids = np.zeros((lg.shape[0], k), np.int32)
    w = np.zeros((lg.shape[0], k), np.float64)
    for r in range(lg.shape[0]):
        order = sorted(range(lg.shape[1]), key=lambda e: (-float(lg[r, e]), e))[:k]
        ids[r] = order
        s = [1.0 / (1.0 + math.exp(-float(lg[r, e]))) for e in order]
        w[r] = [v / sum(s) for v in s]
    return ids, w


def group(ids, n_experts):
    flat = np.asarray(ids).reshape(-1)
    valid = [a for a in range(flat.size) if flat[a] >= 0]
    order = sorted(valid, key=lambda a: (int(flat[a]), a))
    counts = np.bincount(flat[flat >= 0], minlength=n_experts).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    srt = np.full(flat.size, -1, np.int32)
    srt[: len(order)] = order
    return counts, offsets, srt


def silu(z):
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def bf16(x):
    """Round fp32 values to BF16 (to nearest, ties to even) with torch's CPU cast."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def ffn(experts, n_experts, top_k, has_shared, q, qs, ids, w, bf16_mid=False):
    """float64 end-to-end: dequantised projections, fp64 SwiGLU rounded to fp32
    (then to BF16 with bf16_mid), numpy requant, dequantised down, fp64 combine."""
    rows = q.shape[0]
    d_model = experts[next(iter(experts))]["down_codes"].shape[0]
    y = np.zeros((rows, d_model), np.float64)
    for t in range(rows):
        slots = [(ids[t, i], float(w[t, i])) for i in range(top_k) if ids[t, i] >= 0]
        if has_shared:
            slots.append((n_experts, 1.0))
        for e, wt in slots:
            ex = experts[e]
            gu = matvec(ex["gate_up_codes"], ex["gate_up_scales"], q[t:t + 1], qs[t:t + 1])[0]
            f = gu.size // 2
            h = (silu(np.float32(gu[:f]).astype(np.float64)) *
                 np.float32(gu[f:]).astype(np.float64)).astype(np.float32)
            if bf16_mid:
                h = bf16(h)
            hq, hs = quant(h[None, :])
            Y = matvec(ex["down_codes"], ex["down_scales"], hq, hs)[0]
            y[t] += wt * np.float32(Y).astype(np.float64)
    return y
