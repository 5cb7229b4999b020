"""GPU parity of the router projection (BF16 hidden state x BF16 router
weights -> fp32 logits) through the C ABI: bit for bit against the oracle's
exact-rows order at every tiling the kernel picks, and the decode step that
starts from the hidden state."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

m = pytest.importorskip("mxfp4_routed_expert_e2m1_amd")
DEV = "cuda"


def _wr_dev(wr):
    return torch.from_numpy(wr.view(np.int16)).to(DEV)


def _run(x, wr, pad_x=0, pad_l=0):
    T, D = x.shape
    E = wr.shape[0]
    xw = torch.zeros((T, D + pad_x), device=DEV)
    xw[:, :D] = torch.from_numpy(x).to(DEV)
    lw = torch.full((T, E + pad_l), 5.0, device=DEV)
    m.moe_router_logits(xw[:, :D], _wr_dev(wr), logits=lw[:, :E])
    torch.cuda.synchronize()
    if pad_l:
        assert torch.all(lw[:, E:] == 5.0)
    return lw[:, :E].cpu().numpy()


# (rows, d_model, n_experts): one row and the decode tilings, the many-row
# tile kernel (ragged last row tile, expert counts not a multiple of its 4 or
# 64), a d_model below one 512-wide piece (lanes past it idle), 8192 (16
# pieces, smaller row tiles), a ragged last piece (2080)
CASES = [(1, 4096, 256), (3, 4096, 256), (16, 4096, 256), (17, 4096, 256), (100, 1024, 64),
         (5, 384, 16), (2, 8192, 40), (9, 2080, 6), (64, 4096, 257), (20, 8192, 24),
         (33, 384, 70), (41, 2080, 5)]


@pytest.mark.parametrize("rows,D,E", CASES)
def test_router_bitwise_equals_exact_rows_oracle(rows, D, E):
    seed = 300 + rows
    x = synth.activations(seed, 0, rows, D)
    wr = synth.router_weights(seed, 0, E, D)
    got = _run(x, wr, pad_x=8, pad_l=3)
    with oracle.exact_rows():
        want = oracle.router_logits(x, wr)
    np.testing.assert_array_equal(got, want)
    # and within the fp64 mode's rounding of the same sum
    ref = oracle.router_logits(x, wr).astype(np.float64)
    mag = np.abs(x).astype(np.float64) @ np.abs((wr.astype(np.uint32) << 16).view(np.float32)).T
    assert np.all(np.abs(got - ref) <= mag * 2.0 ** -18)


def test_router_prefill_rows_sampled():
    # 4096 rows at the DS-V4 shape; rows are independent, so the oracle checks
    # a sample including the ragged tail
    rows, D, E = 4096, 4096, 256
    x = synth.activations(7, 4096, rows, D)
    wr = synth.router_weights(7, 0, E, D)
    got = _run(x, wr)
    sample = np.array([0, 1, 7, 8, 1000, 2047, 3333, 4088, 4095])
    with oracle.exact_rows():
        want = oracle.router_logits(x[sample], wr)
    np.testing.assert_array_equal(got[sample], want)


def test_router_zero_rows_and_special_values():
    D, E = 512, 8
    wr = synth.router_weights(8, 0, E, D)
    lg = torch.full((1, E), 3.0, device=DEV)
    # zero rows: nothing is read or written
    m.moe_router_logits(torch.zeros((0, D), device=DEV), _wr_dev(wr), logits=lg[:0])
    torch.cuda.synchronize()
    assert torch.all(lg == 3.0)
    # ties of the BF16 rounding of x, values that round up to a carry, tiny
    # and huge values
    f = float.fromhex
    x = np.zeros((2, D), np.float32)
    x[0, :6] = [1 + 2 ** -8, 1 + 3 * 2 ** -8, f("0x1.ffp+0"), f("0x1p-130"), -1e30, 7.0]
    x[1] = synth.normal(8, 1, D)
    got = _run(x, wr)
    with oracle.exact_rows():
        want = oracle.router_logits(x, wr)
    np.testing.assert_array_equal(got, want)


DSV4 = synth.DSV4_LAYER
_LAYER = {}


def _layer_with_router(seed):
    if seed not in _LAYER:
        _LAYER.clear()
        torch.cuda.empty_cache()
        L = DSV4
        fn = lambda e: synth.expert_weights(seed, 0, e, L.d_model, L.d_ff, device=DEV)
        base = m.pack_layer(L.d_model, L.d_ff, L.n_experts, L.top_k, fn, has_shared=True,
                            device=DEV)
        wr = synth.router_weights(seed, 0, L.n_experts, L.d_model)
        _LAYER[seed] = (base, base.variant(router=_wr_dev(wr)), wr)
        torch.cuda.synchronize()
    return _LAYER[seed]


@pytest.mark.parametrize("rows", [1, 3, 16])
def test_decode_step_from_hidden_bitwise(rows):
    # the step with router weights: logits, routes, codes and y all equal the
    # exact-rows oracle's from the same hidden state; and equal the step fed
    # those logits without a router
    seed = synth.DECODE_BATCH["seed"]
    base, lay, wr = _layer_with_router(seed)
    L = DSV4
    x = synth.activations(seed, 700 + rows, rows, L.d_model)
    xd = torch.from_numpy(x).to(DEV)
    lg = torch.full((rows, L.n_experts), 9.0, device=DEV)
    outs = m.moe_ffn_decode_step(lay, xd, logits=lg)
    outs = [o.clone() for o in outs]
    lg_gpu = lg.clone()
    outs2 = m.moe_ffn_decode_step(base, xd, lg_gpu)
    torch.cuda.synchronize()
    for a, b in zip(outs, outs2):
        assert torch.equal(a, b)
    with oracle.exact_rows():
        lg_o = oracle.router_logits(x, wr)
        q_o, qs_o = oracle.quant_q8(x)
        ids_o, w_o = oracle.route(lg_o, L.top_k)
        need = set(int(e) for e in ids_o.reshape(-1)) | {L.n_experts}
        ex = {e: {k: v.cpu().numpy() for k, v in synth.expert_weights(
            seed, 0, e, L.d_model, L.d_ff, device=DEV).items()} for e in sorted(need)}
        y_o = oracle.ffn(ex, L.n_experts, L.top_k, True, q_o, qs_o, ids_o, w_o)
    np.testing.assert_array_equal(lg.cpu().numpy(), lg_o)
    np.testing.assert_array_equal(outs[2].cpu().numpy(), ids_o)
    np.testing.assert_array_equal(outs[3].cpu().numpy(), w_o)
    np.testing.assert_array_equal(outs[-1].cpu().numpy(), y_o)


def test_decode_step_from_hidden_graph_replays():
    seed = synth.DECODE_BATCH["seed"]
    _, lay, _ = _layer_with_router(seed)
    L = DSV4
    xs = [torch.from_numpy(synth.activations(seed, 800 + i, 2, L.d_model)).to(DEV)
          for i in range(3)]
    x = xs[0].clone()
    lg = torch.empty((2, L.n_experts), device=DEV)
    ws = torch.empty(m.moe_ffn_workspace_bytes(lay, 2), dtype=torch.uint8, device=DEV)
    y = torch.empty((2, L.d_model), device=DEV)
    eager = []
    for xi in xs:
        eager.append(m.moe_ffn_decode_step(lay, xi, logits=lg, ws=ws)[-1].clone())
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        m.moe_ffn_decode_step(lay, x, logits=lg, y=y, ws=ws, stream=s)  # warm-up
        with torch.cuda.graph(g, stream=s):
            m.moe_ffn_decode_step(lay, x, logits=lg, y=y, ws=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(2):
        for i, xi in enumerate(xs):
            x.copy_(xi)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, eager[i]), (rep, i)
