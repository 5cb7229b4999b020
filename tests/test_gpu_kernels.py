"""GPU parity of the building blocks: pack, quantiser, router/grouping, k-row
matvec and block dots, through the C ABI, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import golden_lines
from parity import assert_rows_close

pytestmark = pytest.mark.gpu

m = pytest.importorskip("mxfp4_routed_expert_e2m1_amd")
DEV = "cuda"


def _sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------ pack
@pytest.mark.parametrize("n_out,d_in,inter", [(16, 128, 0), (64, 256, 1), (48, 384, 0),
                                              (1024, 256, 1), (4096, 4096, 1), (4096, 2048, 0)])
def test_pack_unpack_roundtrip(n_out, d_in, inter):
    key = synth.stream_key(n_out, d_in, inter)
    codes = synth.codes(key, n_out, d_in, DEV)
    scales = synth.scales(key + 1, n_out, d_in, DEV, exp_lo=-100, exp_hi=100)
    packed = m.moe_pack_mxfp4(codes, scales, inter)
    assert packed.numel() == m.moe_packed_bytes(n_out, d_in)
    c2, s2 = m.moe_unpack_mxfp4(packed, n_out, d_in, inter)
    _sync()
    assert torch.equal(c2, codes) and torch.equal(s2, scales)


def test_pack_padded_strides():
    n_out, d_in = 64, 512
    wide_c = torch.full((n_out, d_in // 2 + 40), 0xAB, dtype=torch.uint8, device=DEV)
    wide_s = torch.full((n_out, d_in // 32 + 3), 0xCD, dtype=torch.uint8, device=DEV)
    codes = synth.codes(5, n_out, d_in, DEV)
    scales = synth.scales(6, n_out, d_in, DEV)
    wide_c[:, : d_in // 2] = codes
    wide_s[:, : d_in // 32] = scales
    p1 = m.moe_pack_mxfp4(codes, scales, 1)
    p2 = m.moe_pack_mxfp4(wide_c[:, : d_in // 2], wide_s[:, : d_in // 32], 1)
    out_c = torch.full_like(wide_c, 0x11)
    out_s = torch.full_like(wide_s, 0x22)
    m.moe_unpack_mxfp4(p2, n_out, d_in, 1, out_c[:, : d_in // 2], out_s[:, : d_in // 32])
    _sync()
    assert torch.equal(p1, p2)
    assert torch.equal(out_c[:, : d_in // 2], codes) and torch.all(out_c[:, d_in // 2:] == 0x11)
    assert torch.equal(out_s[:, : d_in // 32], scales) and torch.all(out_s[:, d_in // 32:] == 0x22)


# ------------------------------------------------------------- quantiser
@pytest.mark.parametrize("rows,cols,pad", [(1, 4096, 0), (4, 256, 0), (16, 4096, 64),
                                           (4096, 4096, 0), (7, 2048, 32)])
def test_quant_bit_exact(rows, cols, pad):
    x = synth.normal(rows, cols, (rows, cols + pad))
    x *= np.float32(10.0) ** synth.normal(rows, 7, (rows, 1))   # per-row magnitudes
    x[:, 5 * 32:6 * 32] = 0.0 if cols > 192 else x[:, 5 * 32:6 * 32]  # a zero block
    xt = torch.from_numpy(x).to(DEV)[:, :cols]
    q_w = torch.zeros((rows, cols + 2 * pad), dtype=torch.int8, device=DEV)
    s_w = torch.zeros((rows, cols // 32 + pad // 8), dtype=torch.float32, device=DEV)
    q, s = m.moe_quant_act_q8(xt, q=q_w[:, :cols], scales=s_w[:, : cols // 32])
    _sync()
    q_o, s_o = oracle.quant_q8(x[:, :cols])
    np.testing.assert_array_equal(q.cpu().numpy(), q_o)
    np.testing.assert_array_equal(s.cpu().numpy(), s_o)
    if pad:
        assert torch.all(q_w[:, cols:] == 0) and torch.all(s_w[:, cols // 32:] == 0)


def test_quant_worked_blocks():
    xs, qs_, ds = [], [], []
    for line in golden_lines("quant_worked.txt"):
        name, d, x, q = [p.strip() for p in line.split("|")]
        xs.append([float(v) for v in x.split()])
        qs_.append([int(v) for v in q.split()])
        ds.append(float(d))
    x = np.array(xs, np.float32).reshape(1, -1)  # the four blocks in one row
    q, s = m.moe_quant_act_q8(torch.from_numpy(x).to(DEV))
    _sync()
    np.testing.assert_array_equal(q.cpu().numpy().reshape(-1), np.array(qs_).reshape(-1))
    np.testing.assert_array_equal(s.cpu().numpy().reshape(-1), np.float32(ds))


def test_quant_zero_rows_is_noop():
    x = torch.zeros((0, 64), device=DEV)
    m.moe_quant_act_q8(x)


# ---------------------------------------------------------- route / group
def _route_case(logits, k):
    lg = torch.from_numpy(logits).to(DEV)
    ids, w, counts, offsets, srt = m.moe_route_group(lg, k)
    _sync()
    ids_o, w_o = oracle.route(logits, k)
    c_o, off_o, srt_o = oracle.group(ids_o, logits.shape[1])
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_o)
    np.testing.assert_array_equal(counts.cpu().numpy(), c_o)
    np.testing.assert_array_equal(offsets.cpu().numpy(), off_o)
    np.testing.assert_array_equal(srt.cpu().numpy()[: ids_o.size], srt_o)
    np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=2e-6, atol=0)


@pytest.mark.parametrize("rows", [1, 2, 4, 8, 16, 512, 4096])
def test_route_group_dsv4(rows):
    _route_case(synth.router_logits(3, rows, rows, 256), 6)


@pytest.mark.parametrize("rows", [2, 16, 512])
def test_route_group_hot_experts(rows):
    _route_case(synth.router_logits(3, rows, rows, 256, hot_bias=2.0), 6)


def test_route_group_tiny_and_ties():
    _route_case(synth.router_logits(0, 0, 4, 8), 2)
    tied = np.round(synth.normal(9, 9, (300, 256)), 1).astype(np.float32)  # many exact ties
    _route_case(tied, 6)
    _route_case(np.zeros((5, 64), np.float32), 4)
    _route_case(synth.normal(9, 10, (33, 512)), 16)
    _route_case(synth.normal(9, 11, (3, 6)), 6)


def _all_ones_nan_rows(rows, n_experts, live):
    """Logits whose bits are all ones (a NaN whose order key is 0) for every
    expert but `live` finite ones per row, and those rows' expected picks."""
    rng = np.random.default_rng(17)
    bits = np.full((rows, n_experts), 0xFFFFFFFF, np.uint32)
    picks = []
    for r in range(rows):
        ex = rng.choice(n_experts, live, replace=False)
        vals = rng.standard_normal(live).astype(np.float32)
        bits[r, ex] = vals.view(np.uint32)
        picks.append([int(e) for e in ex[np.lexsort((ex, -vals))]])  # logit desc, index asc
    return bits.view(np.float32), picks


@pytest.mark.parametrize("rows", [1, 4, 512])
def test_route_group_all_ones_nan_logits_yield_sentinels(rows):
    """Fewer real logits than picks (outside the contract): the remaining
    picks are sentinels, never an expert past the row, and the grouping
    counts only the real ones."""
    E, k, live = 256, 6, 3
    lg, picks = _all_ones_nan_rows(rows, E, live)
    ids, w, counts, offsets, srt = m.moe_route_group(torch.from_numpy(lg).to(DEV), k)
    _sync()
    ids = ids.cpu().numpy()
    want = np.array([p + [-1] * (k - live) for p in picks], np.int32)
    np.testing.assert_array_equal(ids, want)
    c = np.bincount(want[want >= 0], minlength=E)
    np.testing.assert_array_equal(counts.cpu().numpy(), c)
    np.testing.assert_array_equal(offsets.cpu().numpy(), np.concatenate([[0], np.cumsum(c)]))
    flat = want.reshape(-1)
    order = [a for a in np.lexsort((np.arange(flat.size), flat)) if flat[a] >= 0]
    got = srt.cpu().numpy()
    np.testing.assert_array_equal(got[: len(order)], order)
    assert np.all(got[len(order): rows * k] == -1)


def test_route_group_zero_rows():
    lg = torch.zeros((0, 256), device=DEV)
    ids, w, counts, offsets, srt = m.moe_route_group(lg, 6)
    _sync()
    assert torch.all(counts == 0) and torch.all(offsets == 0)


def _prep_case(x, logits, k, pad=0):
    """moe_decode_prep against the oracle (quantiser, router, grouping) and
    bitwise against the two separate calls."""
    rows, cols = x.shape
    xw = torch.from_numpy(np.pad(x, ((0, 0), (0, pad)))).to(DEV)
    xt = xw[:, :cols]
    lg = torch.from_numpy(logits).to(DEV)
    q_w = torch.zeros((rows, cols + 2 * pad), dtype=torch.int8, device=DEV)
    s_w = torch.zeros((rows, cols // 32 + pad // 8), dtype=torch.float32, device=DEV)
    q, qs, ids, w, counts, offsets, srt = m.moe_decode_prep(
        xt, lg, k, q=q_w[:, :cols], scales=s_w[:, : cols // 32])
    q2, qs2 = m.moe_quant_act_q8(xt)
    ids2, w2, counts2, offsets2, srt2 = m.moe_route_group(lg, k)
    _sync()
    q_o, s_o = oracle.quant_q8(x)
    np.testing.assert_array_equal(q.cpu().numpy(), q_o)
    np.testing.assert_array_equal(qs.cpu().numpy(), s_o)
    ids_o, w_o = oracle.route(logits, k)
    c_o, off_o, srt_o = oracle.group(ids_o, logits.shape[1])
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_o)
    np.testing.assert_array_equal(counts.cpu().numpy(), c_o)
    np.testing.assert_array_equal(offsets.cpu().numpy(), off_o)
    np.testing.assert_array_equal(srt.cpu().numpy()[: ids_o.size], srt_o)
    np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=2e-6, atol=0)
    for a, b in ((q, q2), (qs, qs2), (ids, ids2), (w, w2), (counts, counts2),
                 (offsets, offsets2), (srt, srt2)):
        assert torch.equal(a, b)
    if pad:
        assert torch.all(q_w[:, cols:] == 0) and torch.all(s_w[:, cols // 32:] == 0)


@pytest.mark.parametrize("rows", [1, 2, 5, 16])
def test_decode_prep_dsv4(rows):
    x = synth.activations(2, 0, rows, 4096)
    _prep_case(x, synth.router_logits(3, rows, rows, 256), 6)


def test_decode_prep_hot_ties_shapes():
    _prep_case(synth.activations(2, 1, 16, 4096),
               synth.router_logits(3, 16, 16, 256, hot_bias=2.0), 6)
    tied = np.round(synth.normal(9, 12, (7, 256)), 1).astype(np.float32)
    x = synth.normal(9, 13, (7, 256))
    x[:, 64:96] = 0.0                                    # a zero block
    _prep_case(x, tied, 6, pad=64)
    _prep_case(synth.normal(9, 14, (3, 384)), synth.normal(9, 15, (3, 512)), 16)
    _prep_case(synth.normal(9, 16, (4, 256)), synth.router_logits(0, 0, 4, 8), 2)


# ------------------------------------------------------ matvec / block dots
def _matvec_inputs(n_out, d_in, rows, seed, exp=(-8, 0)):
    codes = synth.codes(synth.stream_key(seed, 1), n_out, d_in, DEV)
    scales = synth.scales(synth.stream_key(seed, 2), n_out, d_in, DEV, *exp)
    x = synth.normal(seed, 3, (rows, d_in))
    return codes, scales, x


@pytest.mark.parametrize("n_out,d_in,rows", [(16, 128, 3), (48, 384, 2), (256, 512, 16),
                                             (14336, 4096, 5)])
def test_matvec_parity(n_out, d_in, rows):
    codes, scales, x = _matvec_inputs(n_out, d_in, rows, 1)
    packed = m.moe_pack_mxfp4(codes, scales, 0)
    q, qs = m.moe_quant_act_q8(torch.from_numpy(x).to(DEV))
    y = m.moe_matvec_mxfp4(packed, n_out, d_in, q, qs)
    _sync()
    q_o, qs_o = oracle.quant_q8(x)
    y_o = oracle.matvec(codes.cpu().numpy(), scales.cpu().numpy(), q_o, qs_o)
    assert_rows_close(y.cpu().numpy(), y_o, what=f"matvec {n_out}x{d_in} rows={rows}")


@pytest.mark.parametrize("n_out,d_in,rows", [(14336, 4096, 5), (1024, 2048, 3), (512, 1024, 1)])
def test_matvec_bitwise_equals_exact_rows_oracle(n_out, d_in, rows):
    # the streaming matvec takes the oracle's exact-rows order (runs of 16
    # blocks folded with fmaf, runs added in order): every output bit equal
    codes, scales, x = _matvec_inputs(n_out, d_in, rows, 2)
    packed = m.moe_pack_mxfp4(codes, scales, 0)
    q, qs = m.moe_quant_act_q8(torch.from_numpy(x).to(DEV))
    y = m.moe_matvec_mxfp4(packed, n_out, d_in, q, qs)
    _sync()
    q_o, qs_o = oracle.quant_q8(x)
    with oracle.exact_rows():
        y_o = oracle.matvec(codes.cpu().numpy(), scales.cpu().numpy(), q_o, qs_o)
    np.testing.assert_array_equal(y.cpu().numpy(), y_o)


def test_matvec_k_rows_share_one_pass_bitwise():
    # a row's result does not depend on which other rows share the weight pass
    n_out, d_in = 14336, 4096
    codes, scales, x = _matvec_inputs(n_out, d_in, 5, 1)
    packed = m.moe_pack_mxfp4(codes, scales, 0)
    q, qs = m.moe_quant_act_q8(torch.from_numpy(x).to(DEV))
    full = {k: m.moe_matvec_mxfp4(packed, n_out, d_in, q[:k], qs[:k]) for k in range(1, 6)}
    singles = [m.moe_matvec_mxfp4(packed, n_out, d_in, q[t:t + 1], qs[t:t + 1]) for t in range(5)]
    _sync()
    for k, yk in full.items():
        for t in range(k):
            assert torch.equal(yk[t], singles[t][0]), (k, t)


def test_matvec_integer_exact_fixture_bitwise():
    # d = 1 in every block and u = 127: every partial is a multiple of 0.5 < 2^23,
    # so any summation order gives the exact value and results must match bitwise
    n_out, d_in, rows = 256, 1024, 7
    codes = synth.codes(77, n_out, d_in, DEV)
    scales = torch.full((n_out, d_in // 32), 127, dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(77)
    x = rng.integers(-127, 128, (rows, d_in)).astype(np.float32)
    x[:, ::32] = 127
    packed = m.moe_pack_mxfp4(codes, scales, 0)
    q, qs = m.moe_quant_act_q8(torch.from_numpy(x).to(DEV))
    y = m.moe_matvec_mxfp4(packed, n_out, d_in, q, qs)
    _sync()
    q_o, qs_o = oracle.quant_q8(x)
    assert np.all(qs_o == 1.0)
    y_o = oracle.matvec(codes.cpu().numpy(), scales.cpu().numpy(), q_o, qs_o)
    np.testing.assert_array_equal(y.cpu().numpy(), y_o)


def test_matvec_scale_fingerprint():
    # wide non-constant scales: a wrong scale address map changes the output
    n_out, d_in, rows = 512, 2048, 4
    codes, scales, x = _matvec_inputs(n_out, d_in, rows, 31, exp=(-40, 40))
    packed = m.moe_pack_mxfp4(codes, scales, 0)
    q, qs = m.moe_quant_act_q8(torch.from_numpy(x).to(DEV))
    y = m.moe_matvec_mxfp4(packed, n_out, d_in, q, qs)
    _sync()
    q_o, qs_o = oracle.quant_q8(x)
    y_o = oracle.matvec(codes.cpu().numpy(), scales.cpu().numpy(), q_o, qs_o)
    assert_rows_close(y.cpu().numpy(), y_o, what="scale fingerprint")


def test_matvec_padded_strides():
    n_out, d_in, rows = 128, 512, 3
    codes, scales, x = _matvec_inputs(n_out, d_in, rows, 4)
    packed = m.moe_pack_mxfp4(codes, scales, 0)
    q_w = torch.zeros((rows, d_in + 64), dtype=torch.int8, device=DEV)
    s_w = torch.zeros((rows, d_in // 32 + 12), dtype=torch.float32, device=DEV)
    q, qs = m.moe_quant_act_q8(torch.from_numpy(x).to(DEV), q=q_w[:, :d_in],
                               scales=s_w[:, : d_in // 32])
    y_w = torch.full((rows, n_out + 36), 7.0, device=DEV)
    m.moe_matvec_mxfp4(packed, n_out, d_in, q, qs, y=y_w[:, :n_out])
    _sync()
    q_o, qs_o = oracle.quant_q8(x)
    y_o = oracle.matvec(codes.cpu().numpy(), scales.cpu().numpy(), q_o, qs_o)
    assert_rows_close(y_w[:, :n_out].cpu().numpy(), y_o)
    assert torch.all(y_w[:, n_out:] == 7.0)


@pytest.mark.parametrize("n_out,d_in,rows", [(64, 512, 16), (32, 128, 1), (4096, 4096, 2)])
def test_block_dots_bit_exact(n_out, d_in, rows):
    codes, scales, x = _matvec_inputs(n_out, d_in, rows, 9)
    packed = m.moe_pack_mxfp4(codes, scales, 0)
    q, _ = m.moe_quant_act_q8(torch.from_numpy(x).to(DEV))
    dots = m.moe_debug_block_dots(packed, n_out, d_in, q)
    _sync()
    q_o, _ = oracle.quant_q8(x)
    np.testing.assert_array_equal(dots.cpu().numpy(), oracle.block_dots(codes.cpu().numpy(), q_o))


def test_block_dots_extremes():
    # max |dot| = 32 * 12 * 127 in both signs, every code value, q = +-127
    n_out, d_in = 32, 128
    codes = torch.empty((n_out, d_in // 2), dtype=torch.uint8)
    codes[:16] = 0x77
    codes[16:] = 0xFF
    codes[3] = torch.arange(64, dtype=torch.uint8) % 16 * 17   # every code, both nibbles
    codes = codes.to(DEV)
    scales = torch.full((n_out, d_in // 32), 127, dtype=torch.uint8, device=DEV)
    x = np.full((2, d_in), 127.0, np.float32)
    x[1] = -127.0
    packed = m.moe_pack_mxfp4(codes, scales, 0)
    q, _ = m.moe_quant_act_q8(torch.from_numpy(x).to(DEV))
    dots = m.moe_debug_block_dots(packed, n_out, d_in, q)
    _sync()
    want = oracle.block_dots(codes.cpu().numpy(), oracle.quant_q8(x)[0])
    assert want[0, 0, 0] == 48768 and want[0, 16, 0] == -48768
    np.testing.assert_array_equal(dots.cpu().numpy(), want)


@pytest.mark.parametrize("u", [240, 241])
def test_block_term_overflow_bound(u):
    # The contract's top E8M0 byte.  Every block holds the largest dot
    # (codes +6 -> 12 in half steps, q = 127: 32 * 127 * 12 = 48768) and the
    # activation scale is 2^-10, so the exact output 4 * 48768 * 2^(u-128-10)
    # is finite at both bytes.  The matrix core forms the block term
    # 48768 * 2^(u-128) before the activation scale: finite and exact at 240
    # (the output equals the oracle's bit for bit), above fp32's range at 241,
    # where the output overflows although the exact value does not -- the
    # reason the header stops the contract at 240.
    n_out, d_in = 16, 128
    codes = torch.full((n_out, d_in // 2), 0x77, dtype=torch.uint8, device=DEV)
    scales = torch.full((n_out, d_in // 32), u, dtype=torch.uint8, device=DEV)
    x = np.full((1, d_in), 127.0 * 2.0 ** -10, np.float32)
    packed = m.moe_pack_mxfp4(codes, scales, 0)
    q, qs = m.moe_quant_act_q8(torch.from_numpy(x).to(DEV))
    y = m.moe_matvec_mxfp4(packed, n_out, d_in, q, qs)
    _sync()
    q_o, qs_o = oracle.quant_q8(x)
    assert np.all(qs_o == np.float32(2.0 ** -10)) and np.all(q_o == 127)
    y_o = oracle.matvec(codes.cpu().numpy(), scales.cpu().numpy(), q_o, qs_o)
    exact = 4 * 48768 * 2.0 ** (u - 128 - 10)
    assert np.all(y_o == np.float32(exact)) and np.all(np.isfinite(y_o))
    if u <= 240:
        np.testing.assert_array_equal(y.cpu().numpy(), y_o)
    else:
        assert torch.all(torch.isinf(y))


def test_generator_cpu_gpu_identical():
    # the input generator gives the same bytes on both sides
    key = synth.stream_key(2, 0, 17, synth.GATE_UP_CODES)
    assert torch.equal(synth.codes(key, 256, 4096, DEV).cpu(), synth.codes(key, 256, 4096))
    assert torch.equal(synth.scales(key, 256, 4096, DEV).cpu(), synth.scales(key, 256, 4096))
