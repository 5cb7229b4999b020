"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments before touching the GPU (CPU only: every call here fails validation,
so nothing is enqueued and no device is needed)."""
import ctypes as C
import os
import re

import pytest

from conftest import ROOT

import mxfp4_routed_expert_e2m1_amd as m

HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")

OK, INVALID, SHAPE, STRIDE, WORKSPACE, ALIGN = 0, -1, -2, -3, -4, -5
A = C.c_void_p(0x100000)        # 1 MiB-aligned fake device address, never dereferenced
MIS = C.c_void_p(0x100002)      # misaligned


def declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+[\s\*]+(moe_\w+)\s*\(", txt, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared()
    assert len(names) >= 12
    L = m.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(m.EXPORTS) == names


def test_status_strings():
    assert m.moe_status_string(0) == "ok"
    assert "workspace" in m.moe_status_string(WORKSPACE)
    assert m.moe_status_string(12345) == "unknown status"


def test_packed_bytes_and_workspace_queries():
    assert m.moe_packed_bytes(16, 128) == 1024 + 256
    # 14336 x 4096: exactly the canonical byte count (codes + one byte per 32)
    assert m.moe_packed_bytes(14336, 4096) == 14336 * 2048 + 14336 * 128
    assert m.moe_packed_bytes(15, 128) == 0 and m.moe_packed_bytes(16, 96) == 0
    lay = m.moe_layer_t(4096, 2048, 256, 6, 1, 0x100000, 8912896, 0x200000, 4456448, 0x300000,
                        0x400000)
    L = m.lib()
    # 7 hidden rows: 2-byte codes, f32 scales, f32 partials; 1 token row of
    # activation digit planes (48 bytes per 32 codes); each region 256-byte
    # aligned
    assert L.moe_ffn_workspace_bytes(C.byref(lay), 1) == (7 * 2048 * 2 + 7 * 64 * 4
                                                          + 7 * 4096 * 4 + 1 * 128 * 48)
    a, b, c = C.c_size_t(), C.c_size_t(), C.c_size_t()
    assert L.moe_ffn_workspace_layout(C.byref(lay), 1, C.byref(a), C.byref(b), C.byref(c)) == 0
    assert (a.value, b.value, c.value) == (0, 28672, 28672 + 1792)


def test_pack_validation():
    L = m.lib()
    f = L.moe_pack_mxfp4
    assert f(None, 64, A, 4, 16, 128, 0, A, 1 << 20, None) == INVALID
    assert f(A, 64, A, 4, 15, 128, 0, A, 1 << 20, None) == SHAPE
    assert f(A, 64, A, 4, 16, 96, 0, A, 1 << 20, None) == SHAPE
    assert f(A, 64, A, 4, 16, 128, 2, A, 1 << 20, None) == INVALID
    assert f(A, 64, A, 4, 16, 128, 1, A, 1 << 20, None) == SHAPE   # 16 rows: no gate/up pair
    assert f(A, 32, A, 4, 16, 128, 0, A, 1 << 20, None) == STRIDE
    assert f(A, 64, A, 3, 16, 128, 0, A, 1 << 20, None) == STRIDE
    assert f(MIS, 64, A, 4, 16, 128, 0, A, 1 << 20, None) == ALIGN
    assert f(A, 66, A, 4, 16, 128, 0, A, 1 << 20, None) == ALIGN
    assert f(A, 64, A, 4, 16, 128, 0, MIS, 1 << 20, None) == ALIGN
    assert f(A, 64, A, 4, 16, 128, 0, A, 1279, None) == WORKSPACE


def test_quant_validation():
    f = m.lib().moe_quant_act_q8
    assert f(A, 64, 0, 64, A, 64, A, 2, None) == OK          # rows == 0: no-op
    assert f(A, 64, -1, 64, A, 64, A, 2, None) == INVALID
    assert f(A, 64, 2, 48, A, 64, A, 2, None) == SHAPE
    assert f(None, 64, 2, 64, A, 64, A, 2, None) == INVALID
    assert f(A, 32, 2, 64, A, 64, A, 2, None) == STRIDE
    assert f(A, 64, 2, 64, A, 64, A, 1, None) == STRIDE
    assert f(MIS, 64, 2, 64, A, 64, A, 2, None) == ALIGN
    assert f(A, 66, 2, 64, A, 64, A, 2, None) == ALIGN
    assert f(A, 64, 2, 64, A, 68, A, 2, None) == ALIGN


def test_route_validation():
    f = m.lib().moe_route_group
    args = lambda rows, E, k, ld=256, counts=A: (A, ld, rows, E, k, A, A, counts, A, A, None)
    assert f(*args(4, 256, 0)) == SHAPE
    assert f(*args(4, 256, 17)) == SHAPE
    assert f(*args(4, 8, 9)) == SHAPE
    assert f(*args(4, 513, 6, 513)) == SHAPE
    assert f(*args(4, 256, 6, 255)) == STRIDE
    assert f(*args(4, 256, 6, counts=None)) == INVALID
    assert f(*args(-1, 256, 6)) == INVALID
    assert f(*args(1 << 22, 256, 6)) == SHAPE


def test_router_validation():
    f = m.lib().moe_router_logits
    args = lambda rows=4, D=4096, ldx=4096, w=A, ldw=4096, E=256, ldl=256, x=A, lg=A: (
        x, ldx, rows, D, w, ldw, E, lg, ldl, None)
    assert f(*args(rows=-1)) == INVALID
    assert f(*args(rows=0, x=None, w=None, lg=None)) == OK   # nothing to do
    assert f(*args(rows=0, ldl=255)) == STRIDE
    assert f(*args(x=None)) == INVALID
    assert f(*args(w=None)) == INVALID
    assert f(*args(lg=None)) == INVALID
    assert f(*args(D=4016, ldx=4016, ldw=4016)) == SHAPE     # d_model % 32
    assert f(*args(D=8224, ldx=8224, ldw=8224)) == SHAPE     # d_model > 8192
    assert f(*args(E=0)) == SHAPE
    assert f(*args(E=4097, ldl=4097)) == SHAPE
    assert f(*args(ldx=4092)) == STRIDE
    assert f(*args(ldw=4064)) == STRIDE
    assert f(*args(ldl=255)) == STRIDE
    assert f(*args(x=MIS)) == ALIGN
    assert f(*args(ldx=4098)) == ALIGN
    assert f(*args(w=C.c_void_p(0x100008))) == ALIGN
    assert f(*args(ldw=4100)) == ALIGN
    assert f(*args(lg=MIS)) == ALIGN


def test_decode_prep_validation():
    f = m.lib().moe_decode_prep

    def args(rows=4, cols=64, ldx=64, ldq=64, lds=2, x=A, E=256, k=6, ldl=256, counts=A):
        return (x, ldx, cols, A, ldq, A, lds, A, ldl, rows, E, k, A, A, counts, A, A, None)
    assert f(*args(rows=0)) == SHAPE                  # decode rows only: 1..16
    assert f(*args(rows=17)) == SHAPE
    assert f(*args(cols=48, ldx=64)) == SHAPE           # quantiser checks
    assert f(*args(x=None)) == INVALID
    assert f(*args(ldx=32)) == STRIDE
    assert f(*args(lds=1)) == STRIDE
    assert f(*args(x=MIS)) == ALIGN
    assert f(*args(ldq=68)) == ALIGN
    assert f(*args(k=0)) == SHAPE                       # router checks
    assert f(*args(E=8, k=9)) == SHAPE
    assert f(*args(ldl=255)) == STRIDE
    assert f(*args(counts=None)) == INVALID


def test_decode_step_validation():
    f = m.lib().moe_ffn_decode_step
    lay = _layer()

    def args(rows=1, x=A, ldx=4096, ldl=256, ldq=4096, ldqs=128, counts=A, y=A, ldy=4096,
             ws=A, wsb=1 << 30):
        return (C.byref(lay), x, ldx, A, ldl, rows, A, ldq, A, ldqs, A, A, counts, A, A, y, ldy,
                ws, wsb, None)
    assert f(*args(rows=0)) == SHAPE
    assert f(*args(rows=17)) == SHAPE
    assert f(*args(x=None)) == INVALID                  # quantiser checks
    assert f(*args(ldx=4000)) == STRIDE
    assert f(*args(x=MIS)) == ALIGN
    assert f(*args(ldl=255)) == STRIDE                  # router checks
    assert f(*args(counts=None)) == INVALID
    assert f(*args(ldqs=130)) == ALIGN                  # FFN checks
    assert f(*args(y=None)) == INVALID
    assert f(*args(ldy=4095)) == STRIDE
    assert f(*args(ws=None)) == INVALID
    assert f(*args(ws=MIS)) == ALIGN
    assert f(*args(wsb=1000)) == WORKSPACE
    assert f(C.byref(_layer(top_k=0)), *args()[1:]) == SHAPE
    # router weights in the layer: checked with the layer, then against x/logits
    assert f(C.byref(_layer(router=0x5000000, router_ld=4092)), *args()[1:]) == STRIDE
    assert f(C.byref(_layer(router=0x5000008, router_ld=4096)), *args()[1:]) == ALIGN
    assert f(C.byref(_layer(router=0x5000000, router_ld=4100)), *args()[1:]) == ALIGN
    lr = _layer(router=0x5000000, router_ld=4096)
    assert f(C.byref(lr), *args(ldx=4098)[1:]) == ALIGN       # the router's 16-byte rows of x


def test_decode_step_noalloc_validation():
    # the step's own checks, then the scratch limit (8 MiB), before the device
    f = m.lib().moe_ffn_decode_step_noalloc
    lay = _layer()

    def args(rows=1, x=A, ldx=4096, ldl=256, counts=A, y=A, ldy=4096):
        return (C.byref(lay), x, ldx, A, ldl, rows, A, 4096, A, 128, A, A, counts, A, A, y, ldy,
                None)
    assert f(*args(rows=0)) == SHAPE
    assert f(*args(rows=17)) == SHAPE
    assert f(*args(x=None)) == INVALID
    assert f(*args(ldx=4000)) == STRIDE
    assert f(*args(ldl=255)) == STRIDE
    assert f(*args(counts=None)) == INVALID
    assert f(*args(y=None)) == INVALID
    assert f(*args(ldy=4095)) == STRIDE
    assert f(C.byref(_layer(top_k=0)), *args()[1:]) == SHAPE
    # d_model 8192, d_ff 4096, top-16 + shared at 16 rows: 272 hidden rows,
    # more workspace than the scratch array holds
    gu = (m.moe_packed_bytes(8192, 8192) + 255) // 256 * 256
    dn = (m.moe_packed_bytes(8192, 4096) + 255) // 256 * 256
    big = _layer(d_model=8192, d_ff=4096, n_experts=32, top_k=16, gate_up_stride=gu,
                 down_stride=dn)
    assert m.lib().moe_ffn_workspace_bytes(C.byref(big), 16) > 8 << 20
    assert f(C.byref(big), A, 8192, A, 32, 16, A, 8192, A, 256, A, A, A, A, A, A, 8192,
             None) == WORKSPACE


def _layer(**kw):
    d = dict(d_model=4096, d_ff=2048, n_experts=256, top_k=6, has_shared=1,
             gate_up=0x1000000, gate_up_stride=8912896, down=0x2000000, down_stride=4456448,
             shared_gate_up=0x3000000, shared_down=0x4000000, flags=0, router=0,
             router_ld=0)
    d.update(kw)
    return m.moe_layer_t(*[d[k] for k, _ in m.moe_layer_t._fields_])


def _ffn(fn, lay, rows=1, q=A, ldq=4096, qs=A, ldqs=128, y=A, ldy=4096, ws=A, wsb=1 << 30):
    return fn(C.byref(lay) if lay is not None else None, q, ldq, qs, ldqs, rows, A, A, A, A,
              y, ldy, ws, wsb, None)


@pytest.mark.parametrize("name", ["moe_ffn_decode", "moe_ffn_prefill"])
def test_ffn_validation(name):
    f = getattr(m.lib(), name)
    assert _ffn(f, None) == INVALID
    assert _ffn(f, _layer(d_model=4000)) == SHAPE
    assert _ffn(f, _layer(d_ff=2000)) == SHAPE
    assert _ffn(f, _layer(top_k=0)) == SHAPE
    assert _ffn(f, _layer(top_k=17, n_experts=256)) == SHAPE
    assert _ffn(f, _layer(n_experts=600)) == SHAPE
    assert _ffn(f, _layer(has_shared=2)) == INVALID
    assert _ffn(f, _layer(shared_down=0)) == INVALID
    assert _ffn(f, _layer(flags=2)) == INVALID           # unknown layer flag bits
    assert _ffn(f, _layer(flags=-1)) == INVALID
    assert _ffn(f, _layer(gate_up_stride=8912896 - 256)) == STRIDE
    assert _ffn(f, _layer(down_stride=4456448 + 16)) == ALIGN
    assert _ffn(f, _layer(gate_up=0x1000010)) == ALIGN
    assert _ffn(f, _layer(), rows=0) == SHAPE
    assert _ffn(f, _layer(), q=None) == INVALID
    assert _ffn(f, _layer(), ldq=4000) == STRIDE
    assert _ffn(f, _layer(), ldy=4092) == STRIDE
    assert _ffn(f, _layer(), ldq=4100) == ALIGN
    assert _ffn(f, _layer(), qs=MIS) == ALIGN
    assert _ffn(f, _layer(), ws=MIS) == ALIGN
    assert _ffn(f, _layer(), wsb=1000) == WORKSPACE
    if name == "moe_ffn_decode":
        assert _ffn(f, _layer(), rows=17) == SHAPE


def test_matvec_and_debug_validation():
    L = m.lib()
    assert L.moe_matvec_mxfp4(A, 14336, 4096, A, 4096, A, 128, 0, A, 14336, None) == SHAPE
    assert L.moe_matvec_mxfp4(A, 14336, 4096, A, 4096, A, 128, 17, A, 14336, None) == SHAPE
    assert L.moe_matvec_mxfp4(A, 14330, 4096, A, 4096, A, 128, 1, A, 14336, None) == SHAPE
    assert L.moe_matvec_mxfp4(MIS, 14336, 4096, A, 4096, A, 128, 1, A, 14336, None) == ALIGN
    assert L.moe_matvec_mxfp4(A, 14336, 4096, A, 4096, A, 128, 1, A, 100, None) == STRIDE
    assert L.moe_debug_block_dots(None, 16, 128, A, 128, 1, A, None) == INVALID
    assert L.moe_debug_block_dots(A, 16, 128, A, 100, 1, A, None) == STRIDE
