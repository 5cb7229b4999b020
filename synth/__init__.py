"""Seeded synthetic workloads for the routed-expert MXFP4 MoE FFN.

This module holds random-number generation and workload shapes only: none of
the method's arithmetic (no decode, quantisation, routing or projection).  It
is the one piece shared by the oracle-side tests and the GPU-side callers.

* Weight codes and E8M0 exponents come from a counter-based 32-bit hash, so any
  slice (one expert of one layer set) can be regenerated on the CPU or on the
  GPU and gives identical bytes.  Codes are uniform over all 16 E2M1 patterns
  (so -0 occurs); exponents are uniform in [-8, 0], stored as 127 + e.
* Activations and router logits are N(0,1) from numpy's PCG64 on the host,
  drawn in fp64 and cast to fp32; BF16 router weights are such draws scaled
  by 1/sqrt(d_model) with their low 16 bits cut off.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

M32 = 0xFFFFFFFF

# matrix ids inside one expert
GATE_UP_CODES, GATE_UP_SCALES, DOWN_CODES, DOWN_SCALES = 0, 1, 2, 3


def _mix32_int(x: int) -> int:
    """lowbias32 integer finaliser (C. Wellons), on a Python int."""
    x &= M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & M32
    x ^= x >> 16
    return x


def _mix32(x: torch.Tensor) -> torch.Tensor:
    """Same finaliser on an int64 tensor holding values in [0, 2^32)."""
    x = x ^ (x >> 16)
    x = (x * 0x7FEB352D) & M32
    x = x ^ (x >> 15)
    x = (x * 0x846CA68B) & M32
    x = x ^ (x >> 16)
    return x


def stream_key(*parts: int) -> int:
    """Derive a 32-bit stream key from integers (seed, layer, expert, ...)."""
    k = 0x6A09E667
    for p in parts:
        k = _mix32_int(k ^ _mix32_int(int(p) + 0x9E3779B9))
    return k


def hash_words(key: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """Words start..start+n-1 of stream `key`, as int64 in [0, 2^32)."""
    i = torch.arange(start, start + n, dtype=torch.int64, device=device)
    return _mix32(_mix32(i ^ key) ^ 0x5BD1E995)


def _words_to_bytes(w: torch.Tensor) -> torch.Tensor:
    w = torch.where(w >= 2**31, w - 2**32, w).to(torch.int32)
    return w.view(torch.uint8)


def codes(key: int, n_rows: int, d_in: int, device="cpu") -> torch.Tensor:
    """uint8 [n_rows][d_in/2]: uniform E2M1 codes, element 2i in the low nibble."""
    assert d_in % 32 == 0
    nbytes = n_rows * d_in // 2
    return _words_to_bytes(hash_words(key, nbytes // 4, device)).reshape(n_rows, d_in // 2)


def scales(key: int, n_rows: int, d_in: int, device="cpu", exp_lo=-8, exp_hi=0) -> torch.Tensor:
    """uint8 [n_rows][d_in/32]: E8M0 bytes 127+e, e uniform in [exp_lo, exp_hi]."""
    assert d_in % 32 == 0
    n = n_rows * d_in // 32
    w = hash_words(key, n, device)
    u = 127 + exp_lo + torch.remainder(w, exp_hi - exp_lo + 1)
    return u.to(torch.uint8).reshape(n_rows, d_in // 32)


def expert_weights(seed: int, layer: int, expert: int, d_model: int, d_ff: int,
                   device="cpu") -> dict:
    """Canonical weights of one expert (gate rows first, then up rows)."""
    k = lambda m: stream_key(seed, layer, expert, m)
    return {
        "gate_up_codes": codes(k(GATE_UP_CODES), 2 * d_ff, d_model, device),
        "gate_up_scales": scales(k(GATE_UP_SCALES), 2 * d_ff, d_model, device),
        "down_codes": codes(k(DOWN_CODES), d_model, d_ff, device),
        "down_scales": scales(k(DOWN_SCALES), d_model, d_ff, device),
    }


def matrix_weights(seed: int, copy: int, n_out: int, d_in: int, device="cpu"):
    """Canonical codes/scales of one stand-alone matrix (matvec workload)."""
    return (codes(stream_key(seed, copy, 0xC0DE), n_out, d_in, device),
            scales(stream_key(seed, copy, 0x5CA1E), n_out, d_in, device))


def normal(seed: int, stream: int, shape) -> np.ndarray:
    """N(0,1) fp32 array (drawn in fp64 with PCG64, then cast)."""
    rng = np.random.Generator(np.random.PCG64([seed, stream]))
    return rng.standard_normal(shape, dtype=np.float64).astype(np.float32)


def hot_experts(seed: int, n_experts: int, n_hot: int) -> np.ndarray:
    """Experts that get a logit bias in the expert-sharing variant."""
    rng = np.random.Generator(np.random.PCG64([seed, 0xB1A5]))
    return np.sort(rng.choice(n_experts, size=n_hot, replace=False))


def router_logits(seed: int, step: int, rows: int, n_experts: int, hot_bias=0.0,
                  n_hot=16) -> np.ndarray:
    lg = normal(seed, 0x10000 + step, (rows, n_experts))
    if hot_bias:
        lg[:, hot_experts(seed, n_experts, n_hot)] += np.float32(hot_bias)
    return lg


def activations(seed: int, step: int, rows: int, d_model: int) -> np.ndarray:
    return normal(seed, 0x20000 + step, (rows, d_model))


def router_weights(seed: int, layer: int, n_experts: int, d_model: int) -> np.ndarray:
    """BF16 router weights as uint16 bit patterns [n_experts][d_model]:
    N(0, 1/d_model) drawn in fp64, cast to fp32 and cut to its top 16 bits, so
    that N(0,1) activations give logits of about unit spread."""
    v = normal(seed, 0x30000 + layer, (n_experts, d_model)) * np.float32(1.0 / np.sqrt(d_model))
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@dataclass(frozen=True)
class Layer:
    """Shape of one routed-expert layer."""
    n_experts: int
    top_k: int
    d_model: int
    d_ff: int
    has_shared: bool

    @property
    def expert_bytes(self) -> int:
        """Canonical bytes of one expert: codes (1/2 B per weight) + one
        exponent byte per 32 weights, for gate/up [2F][D] and down [D][F]."""
        n_gu = 2 * self.d_ff * self.d_model
        n_dn = self.d_model * self.d_ff
        return (n_gu + n_dn) // 2 + (n_gu + n_dn) // 32


# The workloads (shapes, seeds).  Names describe what they are.
TINY = dict(name="tiny-moe-e8-top2-d256-f512-t4", layer=Layer(8, 2, 256, 512, False),
            rows=4, seed=0)
MATVEC = dict(name="mxfp4-matvec-14336x4096", n_out=14336, d_in=4096,
              rows=(1, 2, 3, 4, 5), copies=16, seed=1)
DSV4_LAYER = Layer(256, 6, 4096, 2048, True)
DECODE = dict(name="decode-e256-top6+shared-d4096-f2048", layer=DSV4_LAYER, rows=1,
              sets=8, seed=2)
DECODE_BATCH = dict(name="decode-batch-e256-top6+shared-d4096-f2048", layer=DSV4_LAYER,
                    rows=(2, 4, 8, 16), sets=8, seed=3, hot_bias=2.0, n_hot=16)
PREFILL = dict(name="prefill-e256-top6+shared-d4096-f2048", layer=DSV4_LAYER,
               rows=(512, 4096), seed=4)
