"""TEST INFRASTRUCTURE ONLY: ctypes wrapper over the plain-C CPU oracle.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares nothing with the HIP library.  All arrays are numpy.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
BUILD_CMD = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
             "-fPIC", "-shared", _SRC, "-o", LIB_PATH, "-lm"]

_lib = None


def build() -> None:
    subprocess.run(BUILD_CMD, check=True)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = C.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


P = C.c_void_p
I = C.c_int
I64 = C.c_int64


def _declare(L):
    L.oracle_set_threads.argtypes = [I]
    L.oracle_get_threads.restype = I
    L.oracle_set_exact_rows.argtypes = [I]
    L.oracle_set_exact_rows.restype = I
    L.oracle_set_bf16_intermediate.argtypes = [I]
    L.oracle_set_bf16_intermediate.restype = I
    L.oracle_round_bf16.argtypes = [P, I, P]
    L.oracle_round_bf16.restype = None
    L.oracle_exp_rows.argtypes = [P, I, P]
    L.oracle_exp_rows.restype = None
    L.oracle_e2m1_x2.argtypes = [I]
    L.oracle_e2m1_x2.restype = I
    L.oracle_e2m1.argtypes = [I]
    L.oracle_e2m1.restype = C.c_double
    L.oracle_e8m0.argtypes = [I]
    L.oracle_e8m0.restype = C.c_double
    L.oracle_block_dot.argtypes = [P, P]
    L.oracle_block_dot.restype = C.c_int32
    L.oracle_quant_q8.argtypes = [P, I64, I, I, P, I64, P, I64]
    L.oracle_route.argtypes = [P, I64, I, I, I, P, P]
    L.oracle_group.argtypes = [P, I, I, P, P, P]
    L.oracle_router_logits.argtypes = [P, I64, I, I, P, I64, I, P, I64]
    L.oracle_router_logits.restype = I
    L.oracle_matvec.argtypes = [P, I64, P, I64, I, I, P, I64, P, I64, I, P, I64]
    L.oracle_block_dots.argtypes = [P, I64, I, I, P, I64, I, P]
    L.oracle_swiglu.argtypes = [P, P, I, P]
    L.oracle_swiglu.restype = None
    L.oracle_expert_hidden.argtypes = [P, P, I, I, P, I64, P, I64, I, P, I64]
    L.oracle_combine.argtypes = [I, I, I, I, P, P, P, P, I64]
    L.oracle_ffn.argtypes = [I, I, I, I, I, P, P, P, P, P, I64, P, I64, I, P, P, P, P,
                             P, I64, P, P, P, P]
    for f in ("oracle_quant_q8", "oracle_route", "oracle_group", "oracle_matvec",
              "oracle_block_dots", "oracle_expert_hidden", "oracle_combine", "oracle_ffn"):
        getattr(L, f).restype = I


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def get_threads() -> int:
    return lib().oracle_get_threads()


def set_exact_rows(on: bool) -> bool:
    """Exact-rows mode (fp32 in one named order, see moe_oracle.h) on or off;
    returns the previous setting."""
    return bool(lib().oracle_set_exact_rows(int(bool(on))))


class exact_rows:
    """with oracle.exact_rows(): ... runs its body in exact-rows mode."""

    def __enter__(self):
        self.old = set_exact_rows(True)

    def __exit__(self, *exc):
        set_exact_rows(self.old)


def set_bf16_intermediate(on: bool) -> bool:
    """BF16-intermediate mode (SwiGLU output rounded to BF16 before its
    requantisation) on or off; returns the previous setting."""
    return bool(lib().oracle_set_bf16_intermediate(int(bool(on))))


class bf16_intermediate:
    """with oracle.bf16_intermediate(): ... runs its body in that mode."""

    def __enter__(self):
        self.old = set_bf16_intermediate(True)

    def __exit__(self, *exc):
        set_bf16_intermediate(self.old)


def round_bf16(x):
    """The oracle's BF16 rounding (to nearest, ties to even), as fp32."""
    x = _c(x, np.float32)
    y = np.empty_like(x)
    lib().oracle_round_bf16(_p(x), x.size, _p(y))
    return y


def exp_rows(x):
    """The oracle's named fp32 exp, elementwise."""
    x = _c(x, np.float32)
    y = np.empty_like(x)
    lib().oracle_exp_rows(_p(x), x.size, _p(y))
    return y


def e2m1_x2(code: int) -> int:
    return lib().oracle_e2m1_x2(int(code))


def e2m1(code: int) -> float:
    return lib().oracle_e2m1(int(code))


def e8m0(u: int) -> float:
    return lib().oracle_e8m0(int(u))


def block_dot(codes16, q32) -> int:
    c = _c(codes16, np.uint8)
    q = _c(q32, np.int8)
    assert c.size == 16 and q.size == 32
    return lib().oracle_block_dot(_p(c), _p(q))


def quant_q8(x):
    x = _c(x, np.float32)
    rows, cols = x.shape
    q = np.zeros((rows, cols), np.int8)
    s = np.zeros((rows, cols // 32), np.float32)
    _check(lib().oracle_quant_q8(_p(x), cols, rows, cols, _p(q), cols, _p(s), cols // 32),
           "quant_q8")
    return q, s


def route(logits, top_k: int):
    lg = _c(logits, np.float32)
    rows, E = lg.shape
    ids = np.zeros((rows, top_k), np.int32)
    w = np.zeros((rows, top_k), np.float32)
    _check(lib().oracle_route(_p(lg), E, rows, E, top_k, _p(ids), _p(w)), "route")
    return ids, w


def router_logits(x, wr_bits):
    """logits [rows][E] from x fp32 [rows][D] and BF16 router weights given as
    their uint16 bit patterns [E][D]."""
    x = _c(x, np.float32)
    wr = _c(wr_bits, np.uint16)
    rows, D = x.shape
    E = wr.shape[0]
    assert wr.shape[1] == D
    lg = np.zeros((rows, E), np.float32)
    _check(lib().oracle_router_logits(_p(x), D, rows, D, _p(wr), D, E, _p(lg), E),
           "router_logits")
    return lg


def group(ids, n_experts: int):
    ids = _c(ids, np.int32).reshape(-1)
    A = ids.size
    counts = np.zeros(n_experts, np.int32)
    offsets = np.zeros(n_experts + 1, np.int32)
    srt = np.zeros(A, np.int32)
    _check(lib().oracle_group(_p(ids), A, n_experts, _p(counts), _p(offsets), _p(srt)),
           "group")
    return counts, offsets, srt


def matvec(codes, scales, q, qs):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    q = _c(q, np.int8)
    qs = _c(qs, np.float32)
    n_out, half = codes.shape
    d_in = half * 2
    rows = q.shape[0]
    y = np.zeros((rows, n_out), np.float32)
    _check(lib().oracle_matvec(_p(codes), half, _p(scales), scales.shape[1], n_out, d_in,
                               _p(q), q.shape[1], _p(qs), qs.shape[1], rows, _p(y), n_out),
           "matvec")
    return y


def block_dots(codes, q):
    codes = _c(codes, np.uint8)
    q = _c(q, np.int8)
    n_out, half = codes.shape
    d_in = half * 2
    rows = q.shape[0]
    dots = np.zeros((rows, n_out, d_in // 32), np.int32)
    _check(lib().oracle_block_dots(_p(codes), half, n_out, d_in, _p(q), q.shape[1], rows,
                                   _p(dots)), "block_dots")
    return dots


def swiglu(g, u):
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    h = np.zeros_like(g)
    lib().oracle_swiglu(_p(g), _p(u), g.size, _p(h))
    return h


def expert_hidden(gu_codes, gu_scales, q, qs):
    gu_codes = _c(gu_codes, np.uint8)
    gu_scales = _c(gu_scales, np.uint8)
    q = _c(q, np.int8)
    qs = _c(qs, np.float32)
    two_f, half = gu_codes.shape
    d_model, d_ff = half * 2, two_f // 2
    rows = q.shape[0]
    h = np.zeros((rows, d_ff), np.float32)
    _check(lib().oracle_expert_hidden(_p(gu_codes), _p(gu_scales), d_model, d_ff, _p(q),
                                      q.shape[1], _p(qs), qs.shape[1], rows, _p(h), d_ff),
           "expert_hidden")
    return h


def combine(ids, w, Y, has_shared: bool):
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    Y = _c(Y, np.float32)
    rows, top_k = ids.shape
    d_model = Y.shape[-1]
    y = np.zeros((rows, d_model), np.float32)
    _check(lib().oracle_combine(rows, top_k, int(has_shared), d_model, _p(ids), _p(w), _p(Y),
                                _p(y), d_model), "combine")
    return y


def ffn(experts: dict, n_experts: int, top_k: int, has_shared: bool, q, qs, ids, w,
        hq_in=None, hs_in=None, want_intermediates=False):
    """experts: {e: dict(gate_up_codes, gate_up_scales, down_codes, down_scales)} as
    numpy arrays; key n_experts is the shared expert.  Experts no route touches may be
    absent.  Returns y, or (y, dict(h, hq, hs, Y)) with want_intermediates."""
    q = _c(q, np.int8)
    qs = _c(qs, np.float32)
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    rows = q.shape[0]
    any_e = next(iter(experts.values()))
    d_ff = any_e["down_codes"].shape[1] * 2
    d_model = any_e["down_codes"].shape[0]
    n_tab = n_experts + 1
    keep = []

    def table(name, dtype):
        arr = (C.c_void_p * n_tab)()
        for e in range(n_tab):
            if e in experts:
                a = _c(experts[e][name], dtype)
                keep.append(a)
                arr[e] = a.ctypes.data
            else:
                arr[e] = None
        return arr

    gu_c, gu_s = table("gate_up_codes", np.uint8), table("gate_up_scales", np.uint8)
    dn_c, dn_s = table("down_codes", np.uint8), table("down_scales", np.uint8)
    slots = top_k + 1
    y = np.zeros((rows, d_model), np.float32)
    h = np.zeros((rows * slots, d_ff), np.float32) if want_intermediates else None
    hq = np.zeros((rows * slots, d_ff), np.int8) if want_intermediates else None
    hs = np.zeros((rows * slots, d_ff // 32), np.float32) if want_intermediates else None
    Y = np.zeros((rows * slots, d_model), np.float32) if want_intermediates else None
    if hq_in is not None:
        hq_in = _c(hq_in, np.int8)
        hs_in = _c(hs_in, np.float32)
    _check(lib().oracle_ffn(d_model, d_ff, n_experts, top_k, int(has_shared),
                            C.cast(gu_c, P), C.cast(gu_s, P), C.cast(dn_c, P), C.cast(dn_s, P),
                            _p(q), q.shape[1], _p(qs), qs.shape[1], rows, _p(ids), _p(w),
                            _p(hq_in), _p(hs_in), _p(y), d_model, _p(h), _p(hq), _p(hs),
                            _p(Y)), "ffn")
    if want_intermediates:
        return y, dict(h=h, hq=hq, hs=hs, Y=Y)
    return y
