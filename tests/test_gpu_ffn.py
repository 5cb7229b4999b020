"""GPU parity of the whole routed-expert layer (decode and prefill) through the
C ABI, stage by stage, against the oracle, at the workloads' real shapes."""
from contextlib import nullcontext

import numpy as np
import pytest
import torch

import oracle
import synth
from ffn_case import canonical_experts, layer_for, run_case
from parity import covering_rows, use_host_threads

pytestmark = pytest.mark.gpu

m = pytest.importorskip("mxfp4_routed_expert_e2m1_amd")
DEV = "cuda"
TINY = synth.TINY["layer"]
DSV4 = synth.DSV4_LAYER


def test_tiny_layer_all_rows():
    c = synth.TINY
    x = synth.activations(c["seed"], 0, c["rows"], TINY.d_model)
    lg = synth.router_logits(c["seed"], 0, c["rows"], TINY.n_experts)
    r = run_case(TINY, c["seed"], x, lg)
    assert r["flips"] == 0


def test_tiny_layer_prefill_entry_matches_decode():
    c = synth.TINY
    x = synth.activations(c["seed"], 1, 40, TINY.d_model)
    lg = synth.router_logits(c["seed"], 1, 40, TINY.n_experts)
    run_case(TINY, c["seed"], x, lg, entry="moe_ffn_prefill")


def test_decode_one_token():
    c = synth.DECODE
    x = synth.activations(c["seed"], 0, 1, DSV4.d_model)
    lg = synth.router_logits(c["seed"], 0, 1, DSV4.n_experts)
    run_case(DSV4, c["seed"], x, lg)


@pytest.mark.parametrize("rows", [2, 4, 8, 16])
@pytest.mark.parametrize("hot", [0.0, 2.0])
def test_decode_batch(rows, hot):
    c = synth.DECODE_BATCH
    x = synth.activations(c["seed"], rows, rows, DSV4.d_model)
    lg = synth.router_logits(c["seed"], rows, rows, DSV4.n_experts, hot_bias=hot)
    run_case(DSV4, c["seed"], x, lg)


def test_decode_deterministic_and_padded():
    c = synth.DECODE_BATCH
    x = synth.activations(c["seed"], 99, 5, DSV4.d_model)
    lg = synth.router_logits(c["seed"], 99, 5, DSV4.n_experts)
    r1 = run_case(DSV4, c["seed"], x, lg, pads=(64, 128, 36))
    r2 = run_case(DSV4, c["seed"], x, lg)
    assert torch.equal(r1["y"], r2["y"])


@pytest.mark.parametrize("T", [1, 3, 6, 12])
def test_decode_sentinel_routes(T):
    c = synth.DECODE_BATCH
    x = synth.activations(c["seed"], 7, T, DSV4.d_model)
    lg = synth.router_logits(c["seed"], 7, T, DSV4.n_experts)
    ids_o, _ = oracle.route(lg, DSV4.top_k)
    ids_s = ids_o.copy()
    ids_s[0, 1] = -1
    ids_s[min(3, T - 1), :] = -1   # a token owned by no local expert: shared expert only
    ids_s[T - 1, 5] = -1
    run_case(DSV4, c["seed"], x, lg, ids_override=ids_s)


def prefill_sample(L, lg, rows, ids=None, seed=0):
    """Rows a prefill parity test checks: every row of chunks up to 512 rows;
    above that a covering sample of at least 256 rows (every routed expert's
    ragged last tile, every row offset inside the 128-row tiles of routed and
    shared experts, the last row)."""
    if rows <= 512:
        return None
    if ids is None:
        ids, _ = oracle.route(lg, L.top_k)
    return covering_rows(ids, L.n_experts, L.top_k, rows, 128, 256, seed)


@pytest.mark.parametrize("rows", [512, 4096])
def test_prefill_rows(rows):
    # 512 rows (32-row tiles): every row; 4096 rows (128-row tiles): the
    # covering sample
    c = synth.PREFILL
    x = synth.activations(c["seed"], rows, rows, DSV4.d_model)
    lg = synth.router_logits(c["seed"], rows, rows, DSV4.n_experts)
    sample = prefill_sample(DSV4, lg, rows, seed=rows)
    r = run_case(DSV4, c["seed"], x, lg, sample=sample, entry="moe_ffn_prefill")
    n = rows if sample is None else len(sample)
    print(f"prefill {rows}: {n} rows checked, worst err/tol {r['worst']:.3f}, "
          f"flips {r['flips']}")


@pytest.mark.parametrize("T", [1, 4, 12])
def test_decode_graph_replays_match_eager(T):
    # quant + route/group + FFN captured in one HIP graph; every replay, with
    # other eager work and synchronisations in between, equals the eager result
    # (4 and 12 rows: three kernels; 1 row: the row-organised down kernel)
    c = synth.DECODE_BATCH
    layer = layer_for(DSV4, c["seed"])
    x = torch.from_numpy(synth.activations(c["seed"], 50, T, DSV4.d_model)).to(DEV)
    lg = torch.from_numpy(synth.router_logits(c["seed"], 50, T, DSV4.n_experts)).to(DEV)
    q = torch.empty((T, DSV4.d_model), dtype=torch.int8, device=DEV)
    qs = torch.empty((T, DSV4.d_model // 32), dtype=torch.float32, device=DEV)
    rt = (torch.empty((T, 6), dtype=torch.int32, device=DEV),
          torch.empty((T, 6), dtype=torch.float32, device=DEV),
          torch.empty(256, dtype=torch.int32, device=DEV),
          torch.empty(257, dtype=torch.int32, device=DEV),
          torch.empty(T * 6, dtype=torch.int32, device=DEV))
    y = torch.empty((T, DSV4.d_model), device=DEV)
    ws = torch.empty(m.moe_ffn_workspace_bytes(layer, T), dtype=torch.uint8, device=DEV)

    def step():
        m.moe_quant_act_q8(x, q=q, scales=qs)
        ids, w, counts, offsets, srt = m.moe_route_group(lg, 6, out=rt)
        m.moe_ffn_decode(layer, q, qs, ids, w, offsets, srt, y=y, ws=ws)

    step()
    torch.cuda.synchronize()
    y_eager = y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    x2 = torch.from_numpy(synth.activations(c["seed"], 51, T, DSV4.d_model)).to(DEV)
    for r in range(4):
        y.zero_()
        ws.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r}"
        # unrelated eager work between replays
        q2, qs2 = m.moe_quant_act_q8(x2)
        other = m.moe_ffn_decode(layer, q2, qs2, *m.moe_route_group(lg, 6)[:2],
                                 *m.moe_route_group(lg, 6)[3:])
        torch.cuda.synchronize()
        assert torch.isfinite(other).all()


# Layer shapes with other K splits than the DS-V4 layer (d_model x d_ff =
# 2048x2048, 2048x4096 without shared expert, 8192x2048, 1024x1024), through
# the decode entry and through two stage calls.
OTHER_SHAPES = [
    synth.Layer(n_experts=16, top_k=4, d_model=2048, d_ff=2048, has_shared=True),
    synth.Layer(n_experts=32, top_k=8, d_model=2048, d_ff=4096, has_shared=False),
    synth.Layer(n_experts=8, top_k=2, d_model=8192, d_ff=2048, has_shared=True),
    synth.Layer(n_experts=16, top_k=4, d_model=1024, d_ff=1024, has_shared=True),
]


@pytest.mark.parametrize("shape", range(len(OTHER_SHAPES)))
@pytest.mark.parametrize("rows", [8, 11, 16])
def test_decode_other_shapes(shape, rows):
    L = OTHER_SHAPES[shape]
    seed = 11 + shape
    x = synth.activations(seed, rows, rows, L.d_model)
    lg = synth.router_logits(seed, rows, rows, L.n_experts, hot_bias=1.0, n_hot=4)
    r1 = run_case(L, seed, x, lg)
    r2 = run_case(L, seed, x, lg, entry="stages")
    print(f"shape {shape} rows {rows}: worst {r1['worst']:.3f} / {r2['worst']:.3f}")


def test_decode_all_sentinels_gives_zero():
    # no shared expert and every slot a sentinel: nothing to do, y = 0
    L = OTHER_SHAPES[1]
    layer = layer_for(L, 12)
    T = 9
    q = torch.ones((T, L.d_model), dtype=torch.int8, device=DEV)
    qs = torch.ones((T, L.d_model // 32), dtype=torch.float32, device=DEV)
    ids = torch.full((T, L.top_k), -1, dtype=torch.int32, device=DEV)
    w = torch.zeros((T, L.top_k), dtype=torch.float32, device=DEV)
    offsets = torch.zeros(L.n_experts + 1, dtype=torch.int32, device=DEV)
    srt = torch.full((T * L.top_k,), -1, dtype=torch.int32, device=DEV)
    y = torch.full((T, L.d_model), 5.0, device=DEV)
    ws = torch.empty(m.moe_ffn_workspace_bytes(layer, T), dtype=torch.uint8, device=DEV)
    for T2 in (1, T):  # one row: the row-organised down kernel
        y = torch.full((T2, L.d_model), 5.0, device=DEV)
        m.moe_ffn_decode(layer, q[:T2], qs[:T2], ids[:T2], w[:T2], offsets, srt[: T2 * L.top_k],
                         y=y, ws=ws)
        torch.cuda.synchronize()
        assert torch.all(y == 0), T2


def test_decode_workspace_reuse_across_row_counts():
    # one workspace serves calls of different row counts in a row: every
    # result equals that of a fresh workspace, bit for bit
    c = synth.DECODE_BATCH
    layer = layer_for(DSV4, c["seed"])
    ws = torch.empty(m.moe_ffn_workspace_bytes(layer, 16), dtype=torch.uint8, device=DEV)
    for j, T in enumerate([16, 3, 9, 1, 16]):
        x = torch.from_numpy(synth.activations(c["seed"], 300 + j, T, DSV4.d_model)).to(DEV)
        lg = torch.from_numpy(synth.router_logits(c["seed"], 300 + j, T, DSV4.n_experts)).to(DEV)
        q, qs = m.moe_quant_act_q8(x)
        ids, w, counts, offsets, srt = m.moe_route_group(lg, DSV4.top_k)
        y1 = m.moe_ffn_decode(layer, q, qs, ids, w, offsets, srt, ws=ws)
        y2 = m.moe_ffn_decode(layer, q, qs, ids, w, offsets, srt)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), f"call {j} (rows {T})"


# Prefill shapes off the DS-V4 path: d_model 384 is not a multiple of 256, so
# moe_ffn_prefill walks the 16-column decode tiles instead of the grouped GEMM;
# 1 and 17 rows take the GEMM with nearly empty tiles.
ODD = synth.Layer(n_experts=16, top_k=4, d_model=384, d_ff=640, has_shared=True)


@pytest.mark.parametrize("rows", [1, 17, 100])
def test_prefill_tile_fallback_shape(rows):
    seed = 21
    x = synth.activations(seed, rows, rows, ODD.d_model)
    lg = synth.router_logits(seed, rows, rows, ODD.n_experts, hot_bias=1.0, n_hot=3)
    run_case(ODD, seed, x, lg, entry="moe_ffn_prefill")


# A layer whose every dimension takes the prefill grouped GEMM, with routes
# that give its 128-row tiles each count of 32-token tiles from 1 to 4 (the
# two token parts of a workgroup then hold 0, 1 or 2 of them), in both
# passes.
GEMM_MIX = synth.Layer(n_experts=16, top_k=2, d_model=256, d_ff=256, has_shared=True)


@pytest.mark.parametrize("rows", [200, 330])
def test_prefill_gemm_tile_mixes(rows):
    seed = 31
    L = GEMM_MIX
    lg = synth.router_logits(seed, rows, rows, L.n_experts, hot_bias=0.5, n_hot=4)
    ids_o, _ = oracle.route(lg, L.top_k)
    counts = np.bincount(ids_o[ids_o >= 0].ravel(), minlength=L.n_experts)
    assert rows * L.top_k > 16 * L.n_experts  # 128-row tiles
    n32 = {-(-min(c - s, 128) // 32) for c in list(counts) + [rows] for s in range(0, c, 128)}
    assert n32 == {1, 2, 3, 4}
    x = synth.activations(seed, rows, rows, L.d_model)
    run_case(L, seed, x, lg, entry="moe_ffn_prefill")
    # and every row bit for bit equal to the oracle's exact-rows mode
    layer = layer_for(L, seed)
    xt, lt = torch.from_numpy(x).to(DEV), torch.from_numpy(lg).to(DEV)
    q, qs = m.moe_quant_act_q8(xt)
    ids, w, _, offsets, srt = m.moe_route_group(lt, L.top_k)
    y = m.moe_ffn_prefill(layer, q, qs, ids, w, offsets, srt)
    with oracle.exact_rows():
        q_o, qs_o = oracle.quant_q8(x)
        ids_e, w_e = oracle.route(lg, L.top_k)
        ex = canonical_experts(L, seed, 0, range(L.n_experts + 1))
        y_o = oracle.ffn(ex, L.n_experts, L.top_k, L.has_shared, q_o, qs_o, ids_e, w_e)
    np.testing.assert_array_equal(y.cpu().numpy(), y_o)


@pytest.mark.parametrize("rows", [1, 17])
def test_prefill_gemm_small_rows(rows):
    c = synth.PREFILL
    x = synth.activations(c["seed"], 7000 + rows, rows, DSV4.d_model)
    lg = synth.router_logits(c["seed"], 7000 + rows, rows, DSV4.n_experts)
    run_case(DSV4, c["seed"], x, lg, entry="moe_ffn_prefill")


def test_prefill_sentinel_routes_sampled():
    # a prefill chunk whose routes are partly owned elsewhere (-1 sentinels):
    # whole tokens and single slots dropped, regrouped by the oracle
    c = synth.PREFILL
    T = 600
    x = synth.activations(c["seed"], 600, T, DSV4.d_model)
    lg = synth.router_logits(c["seed"], 600, T, DSV4.n_experts)
    ids_o, _ = oracle.route(lg, DSV4.top_k)
    ids_s = ids_o.copy()
    rng = np.random.default_rng(600)
    ids_s[rng.random(ids_s.shape) < 0.3] = -1
    ids_s[5, :] = -1
    sample = prefill_sample(DSV4, lg, T, ids=ids_s, seed=600)
    sample = np.union1d(sample, [5])   # the token with every route elsewhere
    run_case(DSV4, c["seed"], x, lg, sample=sample, entry="moe_ffn_prefill", ids_override=ids_s)


def test_prefill_stages_match_full_call():
    # gate/up and down as two moe_ffn_stages calls give the full call's y, bit for bit
    c = synth.PREFILL
    layer = layer_for(DSV4, c["seed"])
    T = 300
    x = torch.from_numpy(synth.activations(c["seed"], 300, T, DSV4.d_model)).to(DEV)
    lg = torch.from_numpy(synth.router_logits(c["seed"], 300, T, DSV4.n_experts)).to(DEV)
    q, qs = m.moe_quant_act_q8(x)
    ids, w, counts, offsets, srt = m.moe_route_group(lg, DSV4.top_k)
    y1 = m.moe_ffn_prefill(layer, q, qs, ids, w, offsets, srt)
    ws = torch.zeros(m.moe_ffn_workspace_bytes(layer, T), dtype=torch.uint8, device=DEV)
    y2 = torch.empty_like(y1)
    m.moe_ffn_stages(layer, 1, m.MOE_STAGE_GATE_UP, q, qs, ids, w, offsets, srt, y2, ws)
    m.moe_ffn_stages(layer, 1, m.MOE_STAGE_DOWN, q, qs, ids, w, offsets, srt, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("shape", range(len(OTHER_SHAPES)))
def test_decode_one_row_other_shapes(shape):
    # one row takes the row-organised down kernel: d_ff 1024..4096, with and
    # without a shared expert
    L = OTHER_SHAPES[shape]
    seed = 31 + shape
    x = synth.activations(seed, 1, 1, L.d_model)
    lg = synth.router_logits(seed, 1, 1, L.n_experts)
    run_case(L, seed, x, lg)


@pytest.mark.parametrize("step", [0, 1])
def test_decode_step_one_row(step):
    # the whole step from the layer input; one row: quantiser and router inside
    # the gate/up kernel (padded strides on the second case)
    c = synth.DECODE
    x = synth.activations(c["seed"], 500 + step, 1, DSV4.d_model)
    lg = synth.router_logits(c["seed"], 500 + step, 1, DSV4.n_experts)
    run_case(DSV4, c["seed"], x, lg, entry="step", pads=(16, 64, 32) if step else (0, 0, 0))


@pytest.mark.parametrize("shape", range(len(OTHER_SHAPES)))
@pytest.mark.parametrize("rows", [1, 3, 5])
def test_decode_step_other_shapes(shape, rows):
    # one row with d_model 2048 / 1024 takes the fused kernel (4 and 2 waves,
    # with and without a shared expert); 8192 and more rows the three calls
    L = OTHER_SHAPES[shape]
    seed = 51 + shape
    x = synth.activations(seed, rows, rows, L.d_model)
    lg = synth.router_logits(seed, rows, rows, L.n_experts)
    run_case(L, seed, x, lg, entry="step")


@pytest.mark.parametrize("rows,hot", [(2, 0.0), (3, 2.0), (4, 0.0), (4, 2.0)])
def test_decode_step_few_rows(rows, hot):
    # 2-4 rows through the step entry (the three calls; down and combine by
    # output rows); hot experts give tiles of several columns; padded strides
    # on the 4-row cases
    c = synth.DECODE_BATCH
    x = synth.activations(c["seed"], 800 + rows, rows, DSV4.d_model)
    lg = synth.router_logits(c["seed"], 800 + rows, rows, DSV4.n_experts, hot_bias=hot)
    run_case(DSV4, c["seed"], x, lg, entry="step", pads=(16, 64, 32) if rows == 4 else (0, 0, 0))


def test_decode_step_tiny_and_hot():
    x = synth.activations(43, 1, 4, TINY.d_model)
    run_case(TINY, 43, x[:1], synth.router_logits(43, 1, 1, TINY.n_experts), entry="step")
    run_case(TINY, 43, x, synth.router_logits(43, 2, 4, TINY.n_experts), entry="step")
    c = synth.DECODE_BATCH
    x = synth.activations(c["seed"], 600, 12, DSV4.d_model)
    lg = synth.router_logits(c["seed"], 600, 12, DSV4.n_experts, hot_bias=2.0)
    run_case(DSV4, c["seed"], x, lg, entry="step", sample=[0, 5, 11])


def test_decode_step_graph_replays_match_eager():
    c = synth.DECODE
    layer = layer_for(DSV4, c["seed"])
    xs = [torch.from_numpy(synth.activations(c["seed"], 700 + i, 1, DSV4.d_model)).to(DEV)
          for i in range(2)]
    lgs = [torch.from_numpy(synth.router_logits(c["seed"], 700 + i, 1, DSV4.n_experts)).to(DEV)
           for i in range(2)]
    ws = torch.empty(m.moe_ffn_workspace_bytes(layer, 1), dtype=torch.uint8, device=DEV)
    outs = m.moe_ffn_decode_step(layer, xs[0], lgs[0], ws=ws)
    eager = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        m.moe_ffn_decode_step(layer, xs[0], lgs[0], *outs[:2], route_out=outs[2:7], y=outs[7],
                              ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        m.moe_ffn_decode_step(layer, xs[0], lgs[0], *outs[:2], route_out=outs[2:7], y=outs[7],
                              ws=ws)
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), f"replay {r}"
        other = m.moe_ffn_decode_step(layer, xs[1], lgs[1])  # unrelated eager step
        torch.cuda.synchronize()
        assert torch.isfinite(other[-1]).all()


def test_decode_step_one_row_all_ones_nan_logits():
    """The one-row step from logits with only 3 real values (the rest the
    all-ones NaN, outside the contract): its ids, counts, offsets and sorted
    list are moe_route_group's -- 3 picks, then sentinels -- and it runs
    (only the picks' weights are NaN)."""
    c = synth.DECODE
    layer = layer_for(DSV4, c["seed"])
    rng = np.random.default_rng(23)
    bits = np.full((1, DSV4.n_experts), 0xFFFFFFFF, np.uint32)
    ex = rng.choice(DSV4.n_experts, 3, replace=False)
    bits[0, ex] = rng.standard_normal(3).astype(np.float32).view(np.uint32)
    lg = torch.from_numpy(bits.view(np.float32)).to(DEV)
    x = torch.from_numpy(synth.activations(c["seed"], 710, 1, DSV4.d_model)).to(DEV)
    outs = m.moe_ffn_decode_step(layer, x, lg)
    ids, w, counts, offsets, srt = m.moe_route_group(lg, DSV4.top_k)
    torch.cuda.synchronize()
    assert torch.equal(outs[2], ids) and torch.equal(outs[4], counts)
    assert torch.equal(outs[5], offsets) and torch.equal(outs[6], srt)
    got = ids.cpu().numpy()[0]
    assert sorted(got[:3].tolist()) == sorted(ex.tolist()) and np.all(got[3:] == -1)


# The one-row step's router selects the picks (the top_k-th key, bit by bit)
# from 64 experts per lane slot: full and part-filled slots, top_k 6..16.
ROUTER_TIES = [
    synth.Layer(n_experts=256, top_k=16, d_model=2048, d_ff=512, has_shared=True),
    synth.Layer(n_experts=256, top_k=8, d_model=1024, d_ff=512, has_shared=False),
    synth.Layer(n_experts=200, top_k=6, d_model=4096, d_ff=256, has_shared=True),
    synth.Layer(n_experts=512, top_k=9, d_model=4096, d_ff=256, has_shared=True),
]


@pytest.mark.parametrize("shape", range(len(ROUTER_TIES)))
def test_decode_step_one_row_tied_logits(shape):
    """Logits rounded to integers tie within and across lane slots, also at
    the cut: the picks among equal logits are the lowest experts, as the
    oracle's, in the oracle's order."""
    L = ROUTER_TIES[shape]
    seed = 71 + shape
    x = synth.activations(seed, 1, 1, L.d_model)
    lg = np.round(synth.router_logits(seed, 1, 1, L.n_experts)) + np.float32(0.0)  # (no -0)
    run_case(L, seed, x, lg.astype(np.float32), entry="step")


def test_decode_exact_rows_across_batch_sizes():
    # Exact rows ([strix] "The exact-rows contract"): a row's output does not
    # depend on the rows sharing its step.  The same rows decoded all 16
    # together (streaming down + combine), in groups of every width 1..16
    # (5-16 rows: streaming down + combine; 2-4: down + combine by rows; 1:
    # the one-row step kernel) and through the three calls give the same
    # bits.
    c = synth.DECODE_BATCH
    layer = layer_for(DSV4, c["seed"])
    x = torch.from_numpy(synth.activations(c["seed"], 900, 16, DSV4.d_model)).to(DEV)
    lg = torch.from_numpy(synth.router_logits(c["seed"], 900, 16, DSV4.n_experts,
                                              hot_bias=1.0)).to(DEV)
    y_all = m.moe_ffn_decode_step(layer, x, lg)[-1].clone()
    groups = [list(range(0, 8)), list(range(8, 13)), [13, 14, 15, 0], [1, 5, 9], [2, 3],
              [4], [11], [15]]
    # and every width 1..16: the rows w..w+n-1 (mod 16) for n rows, so every
    # row sits at several positions across the widths
    groups += [[(n + i) % 16 for i in range(n)] for n in range(1, 17)]
    for g in groups:
        idx = torch.tensor(g, device=DEV)
        y = m.moe_ffn_decode_step(layer, x[idx].contiguous(), lg[idx].contiguous())[-1]
        torch.cuda.synchronize()
        assert torch.equal(y, y_all[idx]), g
    # one row through the three separate calls
    q, qs = m.moe_quant_act_q8(x[7:8])
    ids, w, counts, offsets, srt = m.moe_route_group(lg[7:8].contiguous(), DSV4.top_k)
    y = m.moe_ffn_decode(layer, q, qs, ids, w, offsets, srt)
    torch.cuda.synchronize()
    assert torch.equal(y, y_all[7:8])


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("rows", [1, 3, 16])
def test_decode_bitwise_equals_exact_rows_oracle(rows, bf16):
    # Exact rows, second half: the oracle's exact-rows mode takes the same fp32
    # steps in the same named order (runs of 16 blocks, fmaf, exp_rows, slot
    # order), so every output of a decode step -- codes, scales, routes,
    # weights, hidden codes and scales, y -- must have the oracle's bits.
    # 1 row: the one-row step kernel; 3: down by rows; 16: streaming down.
    # bf16: the layer flag and the oracle mode that round the SwiGLU output to
    # BF16 before its requant.
    c = synth.DECODE_BATCH
    L = DSV4
    layer = layer_for(L, c["seed"])
    if bf16:
        layer = layer.variant(bf16_intermediate=True)
    x = synth.activations(c["seed"], 950 + rows, rows, L.d_model)
    lg = synth.router_logits(c["seed"], 950 + rows, rows, L.n_experts)
    ws = torch.full((m.moe_ffn_workspace_bytes(layer, rows),), 0x7F, dtype=torch.uint8,
                    device=DEV)
    q, qs, ids, w, counts, offsets, srt, y = m.moe_ffn_decode_step(
        layer, torch.from_numpy(x).to(DEV), torch.from_numpy(lg).to(DEV), ws=ws)
    torch.cuda.synchronize()
    with oracle.exact_rows(), (oracle.bf16_intermediate() if bf16 else nullcontext()):
        q_o, qs_o = oracle.quant_q8(x)
        ids_o, w_o = oracle.route(lg, L.top_k)
        need = set(int(e) for e in ids_o.reshape(-1)) | {L.n_experts}
        ex = canonical_experts(L, c["seed"], 0, need)
        y_o, mid = oracle.ffn(ex, L.n_experts, L.top_k, L.has_shared, q_o, qs_o, ids_o,
                              w_o, want_intermediates=True)
    np.testing.assert_array_equal(q.cpu().numpy(), q_o)
    np.testing.assert_array_equal(qs.cpu().numpy(), qs_o)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_o)
    np.testing.assert_array_equal(w.cpu().numpy(), w_o)
    # hidden codes and scales from the workspace: sorted position p for the
    # routed slots, rows*k + t for the shared expert
    off_h, off_hs, _ = m.moe_ffn_workspace_layout(layer, rows)
    k, slots, A = L.top_k, L.top_k + 1, rows * L.top_k
    hb = ws[off_h: off_h + (A + rows) * L.d_ff * 2].view(torch.bfloat16).view(A + rows, L.d_ff)
    hs = ws[off_hs: off_hs + (A + rows) * (L.d_ff // 32) * 4].view(torch.float32)
    hb = hb.float().cpu().numpy()
    hs = hs.view(A + rows, L.d_ff // 32).cpu().numpy()
    srt_n = srt.cpu().numpy()
    pos = np.empty(A, np.int64)
    pos[srt_n[:A]] = np.arange(A)
    for t in range(rows):
        for i in range(slots):
            g_row = pos[t * k + i] if i < k else A + t
            np.testing.assert_array_equal(hb[g_row], mid["hq"][t * slots + i].astype(np.float32))
            np.testing.assert_array_equal(hs[g_row], mid["hs"][t * slots + i])
    np.testing.assert_array_equal(y.cpu().numpy(), y_o)


def test_decode_one_row_tiny_and_odd():
    for L, seed in ((TINY, 41), (ODD, 42)):
        x = synth.activations(seed, 1, 1, L.d_model)
        lg = synth.router_logits(seed, 1, 1, L.n_experts)
        run_case(L, seed, x, lg)


@pytest.mark.parametrize("case", ["tiny-decode", "odd-decode", "odd-prefill-tiles",
                                  "dsv4-prefill-33", "dsv4-decode-12"])
def test_bf16_intermediate_other_paths(case):
    # the BF16-intermediate flag on every gate/up epilogue: the one-pass
    # projection kernel (shapes the streaming kernel does not take), the
    # streaming kernel with streaming down, and both prefill tile heights;
    # against the fp64 oracle in its BF16 mode
    L, rows, entry = {"tiny-decode": (TINY, synth.TINY["rows"], "moe_ffn_decode"),
                      "odd-decode": (ODD, 5, "moe_ffn_decode"),
                      "odd-prefill-tiles": (ODD, 100, "moe_ffn_prefill"),
                      "dsv4-prefill-33": (DSV4, 33, "moe_ffn_prefill"),
                      "dsv4-decode-12": (DSV4, 12, "moe_ffn_decode")}[case]
    seed = 77
    x = synth.activations(seed, rows, rows, L.d_model)
    lg = synth.router_logits(seed, rows, rows, L.n_experts)
    r = run_case(L, seed, x, lg, entry=entry, bf16_mid=True)
    print(f"{case}: worst err/tol {r['worst']:.3f}, moved codes {r['flips']}")


@pytest.mark.parametrize("rows", [512, 4096])
def test_prefill_bf16_intermediate_rows(rows):
    # 512 rows: 32-row tiles, every row; 4096 rows: 128-row tiles, the covering
    # sample
    c = synth.PREFILL
    x = synth.activations(c["seed"], rows, rows, DSV4.d_model)
    lg = synth.router_logits(c["seed"], rows, rows, DSV4.n_experts)
    sample = prefill_sample(DSV4, lg, rows, seed=rows + 1)
    r = run_case(DSV4, c["seed"], x, lg, sample=sample, entry="moe_ffn_prefill", bf16_mid=True)
    print(f"prefill {rows} bf16: worst err/tol {r['worst']:.3f}, moved codes {r['flips']}")


def test_bf16_flag_is_per_layer_struct():
    # one set of packed weights, flag off and on: the flag is read per call, a
    # flagged copy leaves the original untouched, and it changes the output
    c = synth.DECODE_BATCH
    layer = layer_for(DSV4, c["seed"])
    lay_b = layer.variant(bf16_intermediate=True)
    x = torch.from_numpy(synth.activations(c["seed"], 990, 4, DSV4.d_model)).to(DEV)
    lg = torch.from_numpy(synth.router_logits(c["seed"], 990, 4, DSV4.n_experts)).to(DEV)
    y0 = m.moe_ffn_decode_step(layer, x, lg)[-1].clone()
    y1 = m.moe_ffn_decode_step(lay_b, x, lg)[-1].clone()
    y2 = m.moe_ffn_decode_step(layer, x, lg)[-1].clone()
    torch.cuda.synchronize()
    assert torch.equal(y0, y2)
    assert not torch.equal(y0, y1)
    assert layer.c.flags == 0 and lay_b.c.flags == m.MOE_LAYER_BF16_INTERMEDIATE


# What one GPU of a sharded layer runs, at its real shape.  TP8: every expert
# with d_ff split 8 ways (2048 / 8 = 256 features per GPU).  EP8: 32 of the
# 256 experts live on this GPU (plus the shared expert); the global top-6
# routes to other GPUs' experts are -1 sentinels and the local ones are
# renumbered 0..31.
TP8 = synth.Layer(n_experts=256, top_k=6, d_model=4096, d_ff=256, has_shared=True)
EP8 = synth.Layer(n_experts=32, top_k=6, d_model=4096, d_ff=2048, has_shared=True)


def ep8_routes(seed, step, rows, share=3):
    """Global top-6 over 256 experts, kept only where this GPU's 32 own them."""
    lg = synth.router_logits(seed, step, rows, 256)
    ids, _ = oracle.route(lg, 6)
    lo = 32 * share
    local = np.where((ids >= lo) & (ids < lo + 32), ids - lo, -1).astype(np.int32)
    return lg[:, lo:lo + 32].copy(), local


@pytest.mark.parametrize("rows,entry", [(1, "moe_ffn_decode"), (16, "moe_ffn_decode"),
                                        (16, "step"), (512, "moe_ffn_prefill")])
def test_tp8_shard_shape(rows, entry):
    seed = 61
    x = synth.activations(seed, rows, rows, TP8.d_model)
    lg = synth.router_logits(seed, rows, rows, TP8.n_experts)
    r = run_case(TP8, seed, x, lg, entry=entry, sample=prefill_sample(TP8, lg, rows))
    print(f"TP8 {rows} {entry}: worst err/tol {r['worst']:.3f}, flips {r['flips']}")


@pytest.mark.parametrize("rows,entry", [(1, "moe_ffn_decode"), (16, "moe_ffn_decode"),
                                        (4096, "moe_ffn_prefill")])
def test_ep8_share_shape(rows, entry):
    seed = 62
    x = synth.activations(seed, rows, rows, EP8.d_model)
    lg_local, ids_local = ep8_routes(seed, rows, rows)
    sample = prefill_sample(EP8, lg_local, rows, ids=ids_local, seed=rows + 2)
    r = run_case(EP8, seed, x, lg_local, entry=entry, sample=sample, ids_override=ids_local)
    owned = int((ids_local >= 0).sum())
    print(f"EP8 {rows} {entry}: {owned} of {rows * 6} routes local, worst err/tol "
          f"{r['worst']:.3f}, flips {r['flips']}")


@pytest.mark.parametrize("rows", [16, 512, 4096])
def test_prefill_rows_bitwise_equal_decode_and_exact_rows(rows):
    # Exact rows in prefill ([strix] "The two gates": every kernel keeps each
    # row's reduction order identical to the one-token path): the grouped
    # GEMM sums in the decode kernels' runs of 16 blocks, so each prefill row
    # equals the same row decoded in a step of 16 rows, and the oracle's
    # exact-rows mode, bit for bit (16 and 512 rows: every row; 4096: the
    # covering sample).  The fp64 checks of the same path stay in
    # test_prefill_rows.
    use_host_threads()
    c = synth.PREFILL
    L = DSV4
    layer = layer_for(L, c["seed"])
    x = synth.activations(c["seed"], 8000 + rows, rows, L.d_model)
    lg = synth.router_logits(c["seed"], 8000 + rows, rows, L.n_experts)
    xt, lt = torch.from_numpy(x).to(DEV), torch.from_numpy(lg).to(DEV)
    q, qs = m.moe_quant_act_q8(xt)
    ids, w, counts, offsets, srt = m.moe_route_group(lt, L.top_k)
    y = m.moe_ffn_prefill(layer, q, qs, ids, w, offsets, srt)
    sample = prefill_sample(L, lg, rows, seed=rows + 3)
    sample = np.arange(rows) if sample is None else sample
    for i in range(0, len(sample), 16):
        idx = torch.from_numpy(sample[i:i + 16]).to(DEV)
        y_d = m.moe_ffn_decode_step(layer, xt[idx].contiguous(), lt[idx].contiguous())[-1]
        torch.cuda.synchronize()
        assert torch.equal(y_d, y[idx]), f"rows {sample[i:i + 16]}"
    with oracle.exact_rows():
        q_o, qs_o = oracle.quant_q8(x[sample])
        ids_o, w_o = oracle.route(lg[sample], L.top_k)
        need = set(int(e) for e in ids_o.reshape(-1)) | {L.n_experts}
        ex = canonical_experts(L, c["seed"], 0, need)
        y_o = oracle.ffn(ex, L.n_experts, L.top_k, L.has_shared, q_o, qs_o, ids_o, w_o)
    np.testing.assert_array_equal(y.cpu().numpy()[sample], y_o)
