"""MI355X (gfx950) routed-expert MXFP4 MoE FFN.

Thin ctypes binding over libmoe_mxfp4.so (include/moe_mxfp4.h).  Every
function has the name of the C entry point it calls and only marshals
arguments: torch tensors supply device pointers and strides, the current
torch stream is passed through, and a non-zero status raises MoeError.  All
computation happens in the HIP kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mxfp4.so")

MOE_MAX_TOP_K = 16
MOE_MAX_DECODE_ROWS = 16

EXPORTS = [
    "moe_packed_bytes", "moe_pack_mxfp4", "moe_unpack_mxfp4", "moe_quant_act_q8",
    "moe_route_group", "moe_router_logits", "moe_decode_prep", "moe_ffn_workspace_bytes", "moe_ffn_workspace_layout",
    "moe_ffn_decode", "moe_ffn_decode_step", "moe_ffn_decode_step_stages",
    "moe_ffn_decode_step_noalloc", "moe_ffn_prefill",
    "moe_ffn_stages",
    "moe_matvec_mxfp4",
    "moe_debug_block_dots", "moe_status_string",
]

MOE_STAGE_GATE_UP, MOE_STAGE_DOWN, MOE_STAGE_ALL, MOE_STAGE_REUSE_ACTS = 1, 2, 3, 4


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status} ({_status(status)})")
        self.status = status


class moe_layer_t(C.Structure):
    _fields_ = [("d_model", C.c_int), ("d_ff", C.c_int), ("n_experts", C.c_int),
                ("top_k", C.c_int), ("has_shared", C.c_int),
                ("gate_up", C.c_void_p), ("gate_up_stride", C.c_int64),
                ("down", C.c_void_p), ("down_stride", C.c_int64),
                ("shared_gate_up", C.c_void_p), ("shared_down", C.c_void_p),
                ("flags", C.c_int), ("router", C.c_void_p), ("router_ld", C.c_int64)]

MOE_LAYER_BF16_INTERMEDIATE = 1


_lib = None
P, I, I64, SZ = C.c_void_p, C.c_int, C.c_int64, C.c_size_t


def lib():
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950)")
        L = C.CDLL(LIB_PATH)
        L.moe_packed_bytes.argtypes = [I, I]
        L.moe_packed_bytes.restype = SZ
        L.moe_pack_mxfp4.argtypes = [P, I64, P, I64, I, I, I, P, SZ, P]
        L.moe_unpack_mxfp4.argtypes = [P, I, I, I, P, I64, P, I64, P]
        L.moe_quant_act_q8.argtypes = [P, I64, I, I, P, I64, P, I64, P]
        L.moe_route_group.argtypes = [P, I64, I, I, I, P, P, P, P, P, P]
        L.moe_router_logits.argtypes = [P, I64, I, I, P, I64, I, P, I64, P]
        L.moe_decode_prep.argtypes = [P, I64, I, P, I64, P, I64, P, I64, I, I, I, P, P, P, P, P,
                                      P]
        L.moe_ffn_workspace_bytes.argtypes = [C.POINTER(moe_layer_t), I]
        L.moe_ffn_workspace_bytes.restype = SZ
        L.moe_ffn_workspace_layout.argtypes = [C.POINTER(moe_layer_t), I,
                                               C.POINTER(SZ), C.POINTER(SZ), C.POINTER(SZ)]
        ffn_args = [C.POINTER(moe_layer_t), P, I64, P, I64, I, P, P, P, P, P, I64, P, SZ, P]
        L.moe_ffn_decode.argtypes = ffn_args
        L.moe_ffn_prefill.argtypes = ffn_args
        L.moe_ffn_stages.argtypes = [C.POINTER(moe_layer_t), I, I] + ffn_args[1:]
        step_args = [C.POINTER(moe_layer_t), P, I64, P, I64, I, P, I64, P, I64, P, P, P, P, P, P,
                     I64, P, SZ, P]
        L.moe_ffn_decode_step.argtypes = step_args
        L.moe_ffn_decode_step_stages.argtypes = [step_args[0], I] + step_args[1:]
        L.moe_ffn_decode_step_noalloc.argtypes = step_args[:17] + [P]
        L.moe_matvec_mxfp4.argtypes = [P, I, I, P, I64, P, I64, I, P, I64, P]
        L.moe_debug_block_dots.argtypes = [P, I, I, P, I64, I, P, P]
        L.moe_status_string.argtypes = [I]
        L.moe_status_string.restype = C.c_char_p
        for f in EXPORTS:
            if f not in ("moe_packed_bytes", "moe_ffn_workspace_bytes", "moe_status_string"):
                getattr(L, f).restype = I
        _lib = L
    return _lib


def _status(s):
    return lib().moe_status_string(int(s)).decode()


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _ld(t):
    assert t.dim() == 2 and t.stride(1) == 1, "rows must be contiguous (stride(1) == 1)"
    return t.stride(0)


def _call(fn, *args):
    rc = getattr(lib(), fn)(*args)
    if rc != 0:
        raise MoeError(fn, rc)


# ------------------------------------------------------------------- packing
def moe_packed_bytes(n_out: int, d_in: int) -> int:
    return int(lib().moe_packed_bytes(n_out, d_in))


def moe_pack_mxfp4(codes, scales, gate_up_interleave=0, out=None, stream=None):
    """codes uint8 [n_out][d_in/2], scales uint8 [n_out][d_in/32] on the GPU (row-strided
    views of wider buffers are fine).  Returns the packed blob (or fills `out`)."""
    n_out, d_in = codes.shape[0], codes.shape[1] * 2
    assert scales.shape == (n_out, d_in // 32), "scales must be [n_out][d_in/32] (views allowed)"
    nbytes = moe_packed_bytes(n_out, d_in)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    _call("moe_pack_mxfp4", _ptr(codes), _ld(codes), _ptr(scales), _ld(scales), n_out, d_in,
          int(gate_up_interleave), _ptr(out), out.numel(), _stream(stream))
    return out


def moe_unpack_mxfp4(packed, n_out, d_in, gate_up_interleave=0, codes=None, scales=None,
                     stream=None):
    dev = packed.device
    if codes is None:
        codes = torch.zeros((n_out, d_in // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.zeros((n_out, d_in // 32), dtype=torch.uint8, device=dev)
    _call("moe_unpack_mxfp4", _ptr(packed), n_out, d_in, int(gate_up_interleave), _ptr(codes),
          _ld(codes), _ptr(scales), _ld(scales), _stream(stream))
    return codes, scales


# ---------------------------------------------------------------- activations
def moe_quant_act_q8(x, cols=None, q=None, scales=None, stream=None):
    rows = x.shape[0]
    cols = x.shape[1] if cols is None else cols
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // 32), dtype=torch.float32, device=x.device)
    _call("moe_quant_act_q8", _ptr(x), _ld(x), rows, cols, _ptr(q), _ld(q), _ptr(scales),
          _ld(scales), _stream(stream))
    return q, scales


def moe_route_group(logits, top_k, n_experts=None, out=None, stream=None):
    """Returns (ids, w, counts, offsets, sorted)."""
    rows = logits.shape[0]
    E = logits.shape[1] if n_experts is None else n_experts
    dev = logits.device
    if out is None:
        out = (torch.empty((rows, top_k), dtype=torch.int32, device=dev),
               torch.empty((rows, top_k), dtype=torch.float32, device=dev),
               torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(max(rows * top_k, 1), dtype=torch.int32, device=dev))
    ids, w, counts, offsets, srt = out
    _call("moe_route_group", _ptr(logits), _ld(logits), rows, E, top_k, _ptr(ids), _ptr(w),
          _ptr(counts), _ptr(offsets), _ptr(srt), _stream(stream))
    return out


def moe_router_logits(x, w_router, logits=None, stream=None):
    """logits [rows][E] (f32) of x [rows][D] (f32) under BF16 router weights
    w_router [E][D] (torch.bfloat16, or their uint16/int16 bits)."""
    rows, D = x.shape
    E = w_router.shape[0]
    if logits is None:
        logits = torch.empty((rows, E), dtype=torch.float32, device=x.device)
    _call("moe_router_logits", _ptr(x), _ld(x), rows, D, _ptr(w_router), _ld(w_router), E,
          _ptr(logits), _ld(logits), _stream(stream))
    return logits


def moe_decode_prep(x, logits, top_k, n_experts=None, q=None, scales=None, out=None,
                    stream=None):
    """moe_quant_act_q8(x) and moe_route_group(logits, top_k) in one launch
    (decode rows, 1..16).  Returns (q, scales, ids, w, counts, offsets, sorted)."""
    rows, cols = x.shape[0], x.shape[1]
    E = logits.shape[1] if n_experts is None else n_experts
    dev = x.device
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.int8, device=dev)
    if scales is None:
        scales = torch.empty((rows, cols // 32), dtype=torch.float32, device=dev)
    if out is None:
        out = (torch.empty((rows, top_k), dtype=torch.int32, device=dev),
               torch.empty((rows, top_k), dtype=torch.float32, device=dev),
               torch.empty(E, dtype=torch.int32, device=dev),
               torch.empty(E + 1, dtype=torch.int32, device=dev),
               torch.empty(max(rows * top_k, 1), dtype=torch.int32, device=dev))
    ids, w, counts, offsets, srt = out
    _call("moe_decode_prep", _ptr(x), _ld(x), cols, _ptr(q), _ld(q), _ptr(scales), _ld(scales),
          _ptr(logits), _ld(logits), rows, E, top_k, _ptr(ids), _ptr(w), _ptr(counts),
          _ptr(offsets), _ptr(srt), _stream(stream))
    return (q, scales) + tuple(out)


# --------------------------------------------------------------------- layer
class Layer:
    """Packed weights of one routed-expert layer plus its moe_layer_t.

    gate_up: uint8 [E][stride_gu] packed (gate_up_interleave=1), down: uint8
    [E][stride_dn]; shared_gate_up / shared_down: packed blobs or None."""

    def __init__(self, d_model, d_ff, n_experts, top_k, gate_up, down, shared_gate_up=None,
                 shared_down=None, router=None):
        self.tensors = (gate_up, down, shared_gate_up, shared_down, router)  # keep alive
        has_shared = shared_gate_up is not None
        self.c = moe_layer_t(d_model, d_ff, n_experts, top_k, int(has_shared),
                             gate_up.data_ptr(), gate_up.stride(0) if gate_up.dim() == 2 else 0,
                             down.data_ptr(), down.stride(0) if down.dim() == 2 else 0,
                             shared_gate_up.data_ptr() if has_shared else None,
                             shared_down.data_ptr() if has_shared else None, 0,
                             router.data_ptr() if router is not None else None,
                             _ld(router) if router is not None else 0)
        self.d_model, self.d_ff, self.n_experts, self.top_k = d_model, d_ff, n_experts, top_k
        self.has_shared = has_shared

    def variant(self, bf16_intermediate=False, router=None):
        """The same packed weights with other layer flags (moe_layer_t.flags)
        and, if given, BF16 router weights [E][D] (moe_layer_t.router)."""
        v = Layer.__new__(Layer)
        v.__dict__.update(self.__dict__)
        v.c = moe_layer_t.from_buffer_copy(self.c)
        v.c.flags = MOE_LAYER_BF16_INTERMEDIATE if bf16_intermediate else 0
        if router is not None:
            v.tensors = self.tensors[:4] + (router,)
            v.c.router, v.c.router_ld = router.data_ptr(), _ld(router)
        return v


def moe_ffn_workspace_bytes(layer: Layer, rows: int) -> int:
    return int(lib().moe_ffn_workspace_bytes(C.byref(layer.c), rows))


def moe_ffn_workspace_layout(layer: Layer, rows: int):
    a, b, c = SZ(), SZ(), SZ()
    _call("moe_ffn_workspace_layout", C.byref(layer.c), rows, C.byref(a), C.byref(b),
          C.byref(c))
    return a.value, b.value, c.value


def _ffn(fn, layer, q, qs, ids, w, offsets, srt, y, ws, stream):
    rows = q.shape[0]
    if y is None:
        y = torch.empty((rows, layer.d_model), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(moe_ffn_workspace_bytes(layer, rows), dtype=torch.uint8,
                         device=q.device)
    _call(fn, C.byref(layer.c), _ptr(q), _ld(q), _ptr(qs), _ld(qs), rows, _ptr(ids), _ptr(w),
          _ptr(offsets), _ptr(srt), _ptr(y), _ld(y), _ptr(ws), ws.numel(), _stream(stream))
    return y


def moe_ffn_decode(layer, q, qs, ids, w, offsets, srt, y=None, ws=None, stream=None):
    return _ffn("moe_ffn_decode", layer, q, qs, ids, w, offsets, srt, y, ws, stream)


def _step_outputs(layer, x, logits, q, scales, route_out, y):
    rows, D = x.shape[0], layer.d_model
    dev = x.device
    E, k = layer.c.n_experts, layer.c.top_k
    if logits is None:
        assert layer.c.router, "logits are needed when the layer has no router weights"
        logits = torch.empty((rows, E), dtype=torch.float32, device=dev)
    if q is None:
        q = torch.empty((rows, D), dtype=torch.int8, device=dev)
    if scales is None:
        scales = torch.empty((rows, D // 32), dtype=torch.float32, device=dev)
    if route_out is None:
        route_out = (torch.empty((rows, k), dtype=torch.int32, device=dev),
                     torch.empty((rows, k), dtype=torch.float32, device=dev),
                     torch.empty(E, dtype=torch.int32, device=dev),
                     torch.empty(E + 1, dtype=torch.int32, device=dev),
                     torch.empty(rows * k, dtype=torch.int32, device=dev))
    if y is None:
        y = torch.empty((rows, D), dtype=torch.float32, device=dev)
    return logits, q, scales, route_out, y


def moe_ffn_decode_step(layer, x, logits=None, q=None, scales=None, route_out=None, y=None,
                        ws=None, stream=None, stage_mask=None):
    """One decode step from the layer input: quantise x, route and group the
    logits, run the FFN.  Returns (q, scales, ids, w, counts, offsets, sorted, y),
    every output the separate calls would produce.  stage_mask selects stages
    (moe_ffn_decode_step_stages).  With router weights in the layer, logits is
    where the step writes the router's logits (allocated when None)."""
    rows = x.shape[0]
    logits, q, scales, route_out, y = _step_outputs(layer, x, logits, q, scales, route_out, y)
    if ws is None:
        ws = torch.empty(moe_ffn_workspace_bytes(layer, rows), dtype=torch.uint8,
                         device=x.device)
    ids, w, counts, offsets, srt = route_out
    fn, pre = (("moe_ffn_decode_step", ()) if stage_mask is None else
               ("moe_ffn_decode_step_stages", (int(stage_mask),)))
    _call(fn, C.byref(layer.c), *pre, _ptr(x), _ld(x), _ptr(logits), _ld(logits), rows,
          _ptr(q), _ld(q), _ptr(scales), _ld(scales), _ptr(ids), _ptr(w), _ptr(counts),
          _ptr(offsets), _ptr(srt), _ptr(y), _ld(y), _ptr(ws), ws.numel(), _stream(stream))
    return (q, scales) + tuple(route_out) + (y,)


def moe_ffn_decode_step_noalloc(layer, x, logits=None, q=None, scales=None, route_out=None,
                                y=None, stream=None):
    """moe_ffn_decode_step with the library's own per-GPU scratch as workspace
    (no workspace argument; the C call allocates nothing).  Outputs that are
    None are allocated here, by torch, before the call."""
    rows = x.shape[0]
    logits, q, scales, route_out, y = _step_outputs(layer, x, logits, q, scales, route_out, y)
    ids, w, counts, offsets, srt = route_out
    _call("moe_ffn_decode_step_noalloc", C.byref(layer.c), _ptr(x), _ld(x), _ptr(logits),
          _ld(logits), rows, _ptr(q), _ld(q), _ptr(scales), _ld(scales), _ptr(ids), _ptr(w),
          _ptr(counts), _ptr(offsets), _ptr(srt), _ptr(y), _ld(y), _stream(stream))
    return (q, scales) + tuple(route_out) + (y,)


def moe_ffn_prefill(layer, q, qs, ids, w, offsets, srt, y=None, ws=None, stream=None):
    return _ffn("moe_ffn_prefill", layer, q, qs, ids, w, offsets, srt, y, ws, stream)


def moe_ffn_stages(layer, prefill, stage_mask, q, qs, ids, w, offsets, srt, y, ws,
                   stream=None):
    rows = q.shape[0]
    _call("moe_ffn_stages", C.byref(layer.c), int(prefill), int(stage_mask), _ptr(q), _ld(q),
          _ptr(qs), _ld(qs), rows, _ptr(ids), _ptr(w), _ptr(offsets), _ptr(srt), _ptr(y), _ld(y),
          _ptr(ws), ws.numel(), _stream(stream))
    return y


def moe_matvec_mxfp4(w_packed, n_out, d_in, q, qs, y=None, stream=None):
    rows = q.shape[0]
    if y is None:
        y = torch.empty((rows, n_out), dtype=torch.float32, device=q.device)
    _call("moe_matvec_mxfp4", _ptr(w_packed), n_out, d_in, _ptr(q), _ld(q), _ptr(qs), _ld(qs),
          rows, _ptr(y), _ld(y), _stream(stream))
    return y


def moe_debug_block_dots(w_packed, n_out, d_in, q, stream=None):
    rows = q.shape[0]
    dots = torch.empty((rows, n_out, d_in // 32), dtype=torch.int32, device=q.device)
    _call("moe_debug_block_dots", _ptr(w_packed), n_out, d_in, _ptr(q), _ld(q), rows,
          _ptr(dots), _stream(stream))
    return dots


def moe_status_string(status: int) -> str:
    return _status(status)


# ------------------------------------------------------------------ helpers
def pack_layer(d_model, d_ff, n_experts, top_k, expert_fn, has_shared=True, device="cuda",
               stream=None) -> Layer:
    """Pack every expert of a layer into two contiguous buffers.

    expert_fn(e) returns the canonical weights of expert e as device tensors
    {gate_up_codes [2F][D/2], gate_up_scales [2F][D/32], down_codes [D][F/2],
    down_scales [D][F/32]}; e == n_experts is the shared expert."""
    gu_bytes = (moe_packed_bytes(2 * d_ff, d_model) + 255) // 256 * 256
    dn_bytes = (moe_packed_bytes(d_model, d_ff) + 255) // 256 * 256
    gate_up = torch.empty((n_experts, gu_bytes), dtype=torch.uint8, device=device)
    down = torch.empty((n_experts, dn_bytes), dtype=torch.uint8, device=device)
    sgu = torch.empty(gu_bytes, dtype=torch.uint8, device=device) if has_shared else None
    sdn = torch.empty(dn_bytes, dtype=torch.uint8, device=device) if has_shared else None
    for e in range(n_experts + (1 if has_shared else 0)):
        w = expert_fn(e)
        gu_dst = gate_up[e] if e < n_experts else sgu
        dn_dst = down[e] if e < n_experts else sdn
        moe_pack_mxfp4(w["gate_up_codes"], w["gate_up_scales"], 1, out=gu_dst, stream=stream)
        moe_pack_mxfp4(w["down_codes"], w["down_scales"], 0, out=dn_dst, stream=stream)
        del w
    return Layer(d_model, d_ff, n_experts, top_k, gate_up, down, sgu, sdn)
