"""The stage-wise parity harness of the routed-expert layer on the GPU: run
the layer through the C ABI, then check it against the oracle stage by stage
(activation codes, routes and grouping bit for bit; the requantised hidden
codes read back from the documented workspace, with the rounding-boundary
allowance; y within the tolerance, widened only by what legitimate hidden-code
flips can move).  Shared by the GPU test modules."""
import numpy as np
import torch

import oracle
import synth
from parity import (assert_rows_close, check_hidden, check_hidden_bf16,
                    codes_from_digit_planes, down_col_absmax, flip_bound, hidden_error_bound,
                    use_host_threads)

import mxfp4_routed_expert_e2m1_amd as m

DEV = "cuda"

_CACHE = {}


def layer_for(L: synth.Layer, seed: int, set_idx: int = 0):
    """Packed layer on the GPU (one cached at a time: a DS-V4 layer is 3.4 GB)."""
    key = (L, seed, set_idx)
    if key not in _CACHE:
        _CACHE.clear()
        torch.cuda.empty_cache()
        fn = lambda e: synth.expert_weights(seed, set_idx, e, L.d_model, L.d_ff, device=DEV)
        _CACHE[key] = m.pack_layer(L.d_model, L.d_ff, L.n_experts, L.top_k, fn,
                                   has_shared=L.has_shared, device=DEV)
        torch.cuda.synchronize()
    return _CACHE[key]


def canonical_experts(L, seed, set_idx, experts):
    return {e: {k: v.cpu().numpy() for k, v in
                synth.expert_weights(seed, set_idx, e, L.d_model, L.d_ff, device=DEV).items()}
            for e in sorted(experts)}


def prefill_gemm(L, entry):
    """Whether a call takes the prefill grouped GEMM, whose workspace holds the
    hidden codes as digit planes: moe_ffn_prefill with d_model and 2 d_ff
    multiples of 256 (other prefill shapes use the decode tiles)."""
    return entry == "moe_ffn_prefill" and L.d_model % 256 == 0 and (2 * L.d_ff) % 256 == 0


def run_case(L, seed, x, logits, sample=None, entry="moe_ffn_decode", set_idx=0,
             ids_override=None, pads=(0, 0, 0), bf16_mid=False, layer=None, experts=None):
    """Run the GPU layer and check it against the oracle on rows `sample`
    (bf16_mid: the layer flag and the oracle mode that round the SwiGLU output
    to BF16 before its requant).  layer / experts: a packed layer and a
    function e -> canonical numpy weights of expert e to use instead of the
    generated weights of (seed, set_idx)."""
    T = x.shape[0]
    use_host_threads()
    if layer is None:
        layer = layer_for(L, seed, set_idx)
    if bf16_mid:
        layer = layer.variant(bf16_intermediate=True)
    pad_x, pad_q, pad_y = pads
    xw = torch.zeros((T, L.d_model + pad_x), device=DEV)
    xw[:, : L.d_model] = torch.from_numpy(x).to(DEV)
    qw = torch.zeros((T, L.d_model + pad_q), dtype=torch.int8, device=DEV)
    sw = torch.zeros((T, L.d_model // 32 + pad_q // 8), dtype=torch.float32, device=DEV)
    q, qs = m.moe_quant_act_q8(xw[:, : L.d_model], q=qw[:, : L.d_model],
                               scales=sw[:, : L.d_model // 32])
    ids, w, counts, offsets, srt = m.moe_route_group(torch.from_numpy(logits).to(DEV), L.top_k)
    # oracle side: its own quantiser, router and grouping on the same inputs
    q_o, qs_o = oracle.quant_q8(x)
    ids_o, w_o = oracle.route(logits, L.top_k)
    c_o, off_o, srt_o = oracle.group(ids_o, L.n_experts)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), q_o)
    np.testing.assert_array_equal(qs.cpu().numpy(), qs_o)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_o)
    np.testing.assert_array_equal(offsets.cpu().numpy(), off_o)
    np.testing.assert_array_equal(srt.cpu().numpy()[: srt_o.size], srt_o)
    if ids_override is not None:  # sentinel-edited routes, regrouped by the oracle
        ids_o = ids_override
        c_o, off_o, srt_o = oracle.group(ids_o, L.n_experts)
        ids = torch.from_numpy(ids_o).to(DEV)
        w = torch.from_numpy(w_o).to(DEV)
        offsets = torch.from_numpy(off_o).to(DEV)
        srt = torch.from_numpy(srt_o).to(DEV)
    yw = torch.full((T, L.d_model + pad_y), 3.0, device=DEV)
    ws = torch.full((m.moe_ffn_workspace_bytes(layer, T),), 0x7F, dtype=torch.uint8, device=DEV)
    if entry == "stages":  # decode as two stage calls (gate/up, then down + combine)
        y = m.moe_ffn_stages(layer, 0, m.MOE_STAGE_ALL, q, qs, ids, w, offsets, srt,
                             yw[:, : L.d_model], ws)
    elif entry == "step":  # from the layer input; its own outputs must equal the calls'
        qw2 = torch.full((T, L.d_model + pad_q), 7, dtype=torch.int8, device=DEV)
        sw2 = torch.full((T, L.d_model // 32 + pad_q // 8), 7.0, device=DEV)
        outs = m.moe_ffn_decode_step(layer, xw[:, : L.d_model], torch.from_numpy(logits).to(DEV),
                                     q=qw2[:, : L.d_model], scales=sw2[:, : L.d_model // 32],
                                     y=yw[:, : L.d_model], ws=ws)
        y = outs[-1]
        torch.cuda.synchronize()
        for got, want in zip(outs[:7], (q, qs, ids, w, counts, offsets, srt)):
            assert torch.equal(got, want)
        if pad_q:
            assert torch.all(qw2[:, L.d_model:] == 7) and torch.all(sw2[:, L.d_model // 32:] == 7)
    else:
        y = getattr(m, entry)(layer, q, qs, ids, w, offsets, srt, y=yw[:, : L.d_model], ws=ws)
    torch.cuda.synchronize()
    if pad_y:
        assert torch.all(yw[:, L.d_model:] == 3.0)
    off_h, off_hs, _ = m.moe_ffn_workspace_layout(layer, T)

    rows = np.arange(T) if sample is None else np.asarray(sample)
    need = set(int(e) for e in ids_o[rows].reshape(-1) if e >= 0)
    if L.has_shared:
        need.add(L.n_experts)
    ex = (canonical_experts(L, seed, set_idx, need) if experts is None
          else {e: experts(e) for e in sorted(need)})
    k, slots = L.top_k, L.top_k + 1
    o_args = (ex, L.n_experts, k, L.has_shared, q_o[rows], qs_o[rows], ids_o[rows], w_o[rows])
    if bf16_mid:
        with oracle.bf16_intermediate():
            y_o, mid = oracle.ffn(*o_args, want_intermediates=True)
        h_pre = oracle.ffn(*o_args, want_intermediates=True)[1]["h"]
    else:
        y_o, mid = oracle.ffn(*o_args, want_intermediates=True)

    # stage 3: requantised intermediate read back from the documented workspace
    A = T * k
    n_h = A + (T if L.has_shared else 0)
    hraw = ws[off_h: off_h + n_h * L.d_ff * 2]
    hs = ws[off_hs: off_hs + n_h * (L.d_ff // 32) * 4].view(torch.float32).view(n_h, L.d_ff // 32)
    hs = hs.cpu().numpy()
    pos = np.empty(A, np.int64)
    valid = srt_o[: off_o[-1]]
    pos[valid] = np.arange(valid.size)
    gpu_rows, o_rows, wts = [], [], []
    for j, t in enumerate(rows):
        for i in range(slots):
            if i < k and ids_o[t, i] < 0:
                continue
            if i == k and not L.has_shared:
                continue
            gpu_rows.append(pos[t * k + i] if i < k else A + t)
            o_rows.append(j * slots + i)
            wts.append(w_o[t, i] if i < k else 1.0)
    gpu_rows, o_rows = np.array(gpu_rows), np.array(o_rows)
    # the hidden codes of the checked rows (rows of sentinel routes are never
    # written), stored as E2M1 digit planes or as exact bf16 values
    hb = np.zeros((n_h, L.d_ff), np.float32)
    if len(gpu_rows):
        if prefill_gemm(L, entry):
            raw = hraw.view(n_h, 2 * L.d_ff)[torch.from_numpy(gpu_rows).to(hraw.device)]
            hb[gpu_rows] = codes_from_digit_planes(raw.cpu().numpy(), L.d_ff)
        else:
            hb[gpu_rows] = hraw.view(torch.bfloat16).view(n_h, L.d_ff)[
                torch.from_numpy(gpu_rows).to(hraw.device)].float().cpu().numpy()
    flips = np.zeros((len(rows) * slots, L.d_ff), np.float64)
    if bf16_mid:
        flips[o_rows] = check_hidden_bf16(hb[gpu_rows], hs[gpu_rows], mid["hq"][o_rows],
                                          mid["hs"][o_rows], mid["h"][o_rows], h_pre[o_rows])
    else:
        def dh_fn(i):  # error bound of the i-th checked hidden row
            j, sl = divmod(int(o_rows[i]), slots)
            e = L.n_experts if sl == k else int(ids_o[rows[j], sl])
            return hidden_error_bound(ex[e]["gate_up_codes"], ex[e]["gate_up_scales"],
                                      q_o[rows[j]], qs_o[rows[j]])

        flips[o_rows] = check_hidden(hb[gpu_rows], hs[gpu_rows], mid["hq"][o_rows],
                                     mid["hs"][o_rows], mid["h"][o_rows], dh_fn=dh_fn)
    weight = np.zeros(len(rows) * slots)
    weight[o_rows] = wts
    col_max = {}

    def colmax(r):
        j, i = divmod(r, slots)
        e = L.n_experts if i == k else int(ids_o[rows[j], i])
        if e not in col_max:
            col_max[e] = down_col_absmax(ex[e]["down_codes"], ex[e]["down_scales"])
        return col_max[e]

    extra_slot = flip_bound(flips, weight, mid["hs"], colmax)
    extra = extra_slot.reshape(len(rows), slots).sum(axis=1)
    worst = assert_rows_close(y.cpu().numpy()[rows], y_o, extra=extra, what=entry)
    # what the GPU layer was given, for callers that check more (q_o and qs_o
    # equal the GPU's codes; ids and w are the routes the layer ran with)
    return dict(worst=worst, flips=int(np.count_nonzero(flips)), y=y, ex=ex, q_o=q_o,
                qs_o=qs_o, ids=ids.cpu().numpy(), w=w.cpu().numpy())
