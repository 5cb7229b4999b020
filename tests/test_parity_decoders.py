"""The test-side decoder of the prefill GEMM's hidden-code workspace format
(E3M2 digit planes), checked on hand-built blocks on the CPU."""
import numpy as np
import pytest

from parity import codes_from_digit_planes, e3m2_value


def test_e3m2_values_follow_the_format_table():
    # OCP microscaling FP6 E3M2: bias 3, no infinities or NaNs, largest
    # normal 28, smallest subnormal 2^-4
    table = {0x00: 0.0, 0x01: 0.0625, 0x03: 0.1875, 0x04: 0.25, 0x0C: 1.0, 0x0D: 1.25,
             0x10: 2.0, 0x12: 3.0, 0x14: 4.0, 0x15: 5.0, 0x16: 6.0, 0x17: 7.0, 0x18: 8.0,
             0x1F: 28.0, 0x20: -0.0, 0x2C: -1.0, 0x38: -8.0, 0x3F: -28.0}
    for code, want in table.items():
        assert e3m2_value(code) == want, hex(code)


def _magnitude_code(v):
    # written out by hand for |v| in 0..8 (exponent field << 2 | mantissa)
    return {0: 0, 1: 3 << 2, 2: 4 << 2, 3: (4 << 2) | 2, 4: 5 << 2, 5: (5 << 2) | 1,
            6: (5 << 2) | 2, 7: (5 << 2) | 3, 8: 6 << 2}[v]


def _encode_row(codes):
    """One hidden row in the workspace format, built bit by bit."""
    d_ff = len(codes)
    out = np.zeros(2 * d_ff, np.uint8)
    for b in range(d_ff // 32):
        planes = [[0] * 192, [0] * 192]
        for e in range(32):
            q = int(codes[32 * b + e])
            d0 = (q + 8) % 16 - 8
            d1 = (q - d0) // 16
            for s, d in enumerate((d0, d1)):
                c = (32 if d < 0 else 0) | _magnitude_code(abs(d))
                for k in range(6):
                    planes[s][6 * e + k] = (c >> k) & 1
        pb = [bytes(sum(bits[8 * i + k] << k for k in range(8)) for i in range(24))
              for bits in planes]
        blk = pb[0][:16] + pb[1][:16] + pb[0][16:] + pb[1][16:]
        out[48 * b:48 * b + 48] = np.frombuffer(blk, np.uint8)
    return out


def test_decoder_round_trips_every_int8_code():
    codes = np.concatenate([np.arange(-128, 128), np.arange(127, -129, -1)]).astype(np.int32)
    raw = np.stack([_encode_row(codes), _encode_row(codes[::-1].copy())])
    got = codes_from_digit_planes(raw, len(codes))
    assert np.array_equal(got[0], codes) and np.array_equal(got[1], codes[::-1])


def test_decoder_rejects_a_code_that_is_not_a_digit():
    raw = _encode_row(np.zeros(32, np.int32))[None, :]
    raw[0, 0] = 0x01  # element 0 of plane 0 becomes 2^-4
    with pytest.raises(AssertionError):
        codes_from_digit_planes(raw, 32)
