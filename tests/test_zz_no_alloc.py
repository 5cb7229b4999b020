"""The allocation-free decode step (moe_ffn_decode_step_noalloc) against the
workspace decode step (moe_ffn_decode_step): the same kernels on the same
inputs, so every output must have the same bits.  Two or more calls in a row
share the library's scratch; later calls take fewer rows, so a later call
must not depend on what an earlier, larger one left there."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

m = pytest.importorskip("mxfp4_routed_expert_e2m1_amd")
DEV = "cuda"


def _layer(L, seed):
    fn = lambda e: synth.expert_weights(seed, 0, e, L.d_model, L.d_ff, device=DEV)
    return m.pack_layer(L.d_model, L.d_ff, L.n_experts, L.top_k, fn, has_shared=L.has_shared,
                        device=DEV)


def _outputs(rows, L, fill):
    # outputs pre-filled with garbage, so nothing passes by leaving them alone
    E, k, D = L.n_experts, L.top_k, L.d_model
    return dict(q=torch.full((rows, D), fill, dtype=torch.int8, device=DEV),
                scales=torch.full((rows, D // 32), float(fill), device=DEV),
                route_out=(torch.full((rows, k), fill, dtype=torch.int32, device=DEV),
                           torch.full((rows, k), float(fill), device=DEV),
                           torch.full((E,), fill, dtype=torch.int32, device=DEV),
                           torch.full((E + 1,), fill, dtype=torch.int32, device=DEV),
                           torch.full((rows * k,), fill, dtype=torch.int32, device=DEV)),
                y=torch.full((rows, D), float(fill), device=DEV))


@pytest.mark.parametrize("shape", ["dsv4", "tiny"])
def test_noalloc_step_equals_workspace_step(shape):
    if shape == "dsv4":
        L, seed, row_seq, hot = synth.DSV4_LAYER, synth.DECODE_BATCH["seed"], [16, 3, 1, 9], 2.0
    else:
        L, seed, row_seq, hot = synth.TINY["layer"], synth.TINY["seed"], [16, 4, 1], 0.0
    layer = _layer(L, seed)
    for j, rows in enumerate(row_seq):
        x = torch.from_numpy(synth.activations(seed, 4000 + j, rows, L.d_model)).to(DEV)
        lg = torch.from_numpy(synth.router_logits(seed, 4000 + j, rows, L.n_experts,
                                                  hot_bias=hot)).to(DEV)
        got = m.moe_ffn_decode_step_noalloc(layer, x, lg, **_outputs(rows, L, 5))
        want = m.moe_ffn_decode_step(layer, x, lg, **_outputs(rows, L, 9))
        torch.cuda.synchronize()
        names = ("q", "scales", "ids", "w", "counts", "offsets", "sorted", "y")
        for name, a, b in zip(names, got, want):
            assert torch.equal(a, b), f"call {j} ({rows} rows): {name} differs"
        assert torch.isfinite(got[-1]).all()
        print(f"{shape} call {j}: {rows} rows, max|y| {float(got[-1].abs().max()):.3e}")
