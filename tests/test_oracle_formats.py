"""Pins for the oracle's number formats (FP4 E2M1, E4M3, E8M0, bf16) and the FP4 / MX FP4 input encoders."""
import math

import numpy as np
import torch

import oracle
from csa_synth import bf16_bits_from_f32, f32_from_bf16_bits, fp4_quantize


def test_e2m1_table_matches_golden(golden):
    rows = golden("e2m1_codes.txt")
    assert len(rows) == 16
    for row in rows:
        code, value, byte = row.split()
        code, value, byte = int(code), float(value), int(byte, 16)
        v = oracle.e2m1_value(code)
        assert v == value and math.copysign(1.0, v) == math.copysign(1.0, value)
        assert oracle.e2m1_to_e4m3(code) == byte
        # the E4M3 byte decodes to exactly the E2M1 value: the dequantisation is lossless
        assert oracle.e4m3_value(byte) == value


def test_e4m3_decoder_known_values():
    # fixed points of the OCP E4M3 definition: 1.0, max normal 448, min normal 2^-6,
    # min subnormal 2^-9, NaN encoding S.1111.111
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0xB8) == -1.0
    assert math.isnan(oracle.e4m3_value(0x7F))
    # monotone over the positive bytes
    vals = [oracle.e4m3_value(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


def test_fp4_dequantize_unpacks_low_nibble_first():
    # byte 0x72: low nibble 2 (1.0) is element 0, high nibble 7 (6.0) element 1
    codes = np.zeros((1, 16), dtype=np.uint8)
    codes[0, 0] = 0x72
    codes[0, 1] = 0x9B            # low 11 (-1.5), high 9 (-0.5)
    scales = np.array([[2.0]], dtype=np.float32)
    v = oracle.fp4_dequantize(codes, scales)
    assert v.shape == (1, 32)
    assert list(v[0, :4]) == [2.0, 12.0, -3.0, -1.0]
    assert np.all(v[0, 4:] == 0)


def test_fp4_encoder_rounding(golden):
    for row in golden("fp4_rounding.txt"):
        x, want = (float(t) for t in row.split())
        blk = torch.zeros(1, 32)
        blk[0, 0] = x
        blk[0, 1] = 6.0 if abs(x) <= 6 else abs(x)     # amax 6 -> scale 1 (if |x| <= 6)
        if abs(x) > 6:
            continue
        codes, scale = fp4_quantize(blk)
        assert float(scale[0, 0]) == 1.0
        got = oracle.fp4_dequantize(codes.numpy(), scale.numpy())[0, 0]
        assert got == want, (x, got, want)


def test_fp4_encoder_error_bound():
    # every value is within half a grid step (relative to the scale) of its code
    g = torch.Generator().manual_seed(5)
    x = torch.randn(64, 128, generator=g)
    codes, scale = fp4_quantize(x)
    deq = oracle.fp4_dequantize(codes.numpy(), scale.numpy())
    xs = x.numpy().astype(np.float64)
    s = np.repeat(scale.numpy().astype(np.float64), 32, axis=-1)
    err = np.abs(deq - xs) / s
    # the widest E2M1 gap is 2 (between 4 and 6), so the error is at most 1 step unit
    assert err.max() <= 1.0 + 1e-6
    # block amax maps to exactly +-6
    blocks = np.abs(deq).reshape(64, 4, 32).max(axis=-1)
    assert np.array_equal(blocks, scale.numpy().astype(np.float64) * 6.0)


def test_round_to_bf16_matches_bit_rounding():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),      # subnormals
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.0e38], np.float32),
    ])
    want = f32_from_bf16_bits(bf16_bits_from_f32(x)).astype(np.float64)
    got = oracle.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)
    # ties to even, by hand: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> 1
    assert oracle.round_to_bf16(np.array([1.0 + 2 ** -8]))[0] == 1.0
    assert oracle.round_to_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6


def test_bf16_bits_roundtrip():
    x = np.array([1.0, -2.5, 0.0078125, 3.140625], dtype=np.float32)   # all exact in bf16
    bits = bf16_bits_from_f32(x)
    assert list(bits) == [0x3F80, 0xC020, 0x3C00, 0x4049]
    assert np.array_equal(oracle.from_bf16_bits(bits), x.astype(np.float64))


# ---------------------------------------------------------------- MX FP4 (E8M0 block scales)
def test_e8m0_decoder_known_values(golden):
    rows = golden("e8m0_values.txt")
    assert len(rows) >= 8
    for row in rows:
        b, v = row.split()
        got = oracle.e8m0_value(int(b, 16))
        if v == "nan":
            assert math.isnan(got)
        else:
            assert got == float(v)


def test_fp4_to_e4m3_lossless_within_threshold():
    # §5: FP4 dequantises to FP8 E4M3 without loss while the block scale stays
    # within a threshold.  With a power-of-two scale 2^e that threshold is
    # -8 <= e <= 6: every E2M1 value times 2^e is an E4M3 value there, and
    # just outside it some code has no exact E4M3 form: 6 * 2^7 = 768 exceeds
    # E4M3's largest finite value 448, 0.5 * 2^-9 = 2^-10 is below its
    # smallest subnormal 2^-9, and 1.5 * 2^-9 would need a 2^-10 step.
    for e in range(-8, 7):
        for code in range(16):
            b = oracle.e2m1_scaled_to_e4m3(code, e)
            assert b is not None, (code, e)
            assert oracle.e4m3_value(b) == math.ldexp(oracle.e2m1_value(code), e)
    assert oracle.e2m1_scaled_to_e4m3(7, 7) is None          # 768 > 448
    assert oracle.e2m1_scaled_to_e4m3(1, -9) is None         # 2^-10 < 2^-9
    assert oracle.e2m1_scaled_to_e4m3(3, -9) is None         # 1.5 * 2^-9: needs a 2^-10 step


def test_mx4_dequantize_is_fp4_with_power_of_two_scales():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, size=(3, 64), dtype=np.uint8)
    sb = rng.integers(100, 160, size=(3, 4), dtype=np.uint8)
    pow2 = np.ldexp(np.float32(1.0), sb.astype(np.int32) - 127).astype(np.float32)
    np.testing.assert_array_equal(oracle.mx4_dequantize(codes, sb),
                                  oracle.fp4_dequantize(codes, pow2))


def test_mx4_encoder_worked_examples(golden):
    from csa_synth import mx4_quantize
    for row in golden("mx4_encoding.txt"):
        a, b, c = (t.strip() for t in row.split("|"))
        xs = [float(v) for v in a.split(",")]
        x = torch.zeros(1, 32)
        x[0, : len(xs)] = torch.tensor(xs)
        codes, sb = mx4_quantize(x)
        assert int(sb[0, 0]) == int(b), row
        got = oracle.mx4_dequantize(codes.numpy(), sb.numpy())[0]
        want = [float(v) for v in c.split(",")]
        assert list(got[: len(want)]) == want, row
        assert np.all(got[len(want):] == 0), row


def test_mx4_encoder_error_bound():
    # every decoded value is within half a grid step of the input clamped to
    # +-6 * 2^e (the largest step, between 4 and 6, is 2 * 2^e), and the
    # block's largest magnitude lands in [4, 8) * 2^e before saturation
    from csa_synth import mx4_quantize
    x = torch.randn(64, 128) * torch.exp(torch.randn(64, 1) * 3)
    codes, sb = mx4_quantize(x)
    deq = oracle.mx4_dequantize(codes.numpy(), sb.numpy())
    xs = x.numpy().astype(np.float64).reshape(64, 4, 32)
    step = np.ldexp(1.0, sb.numpy().astype(np.int64) - 127)[..., None]
    clamped = np.clip(xs, -6 * step, 6 * step)
    assert np.all(np.abs(deq.reshape(64, 4, 32) - clamped) <= step * (1 + 1e-12))
    amax = np.abs(xs).max(axis=-1, keepdims=True)
    assert np.all((amax >= 4 * step) & (amax < 8 * step))


def test_oracle_mx4_encoder_worked_examples(golden):
    # the oracle's own MX encoder (used to check the GPU encoder) on the same
    # hand-worked blocks as the input encoder
    for row in golden("mx4_encoding.txt"):
        a, b, c = (t.strip() for t in row.split("|"))
        xs = [float(v) for v in a.split(",")]
        x = np.zeros((1, 32))
        x[0, : len(xs)] = xs
        codes, sb = oracle.mx4_quantize(x)
        assert int(sb[0, 0]) == int(b), row
        got = oracle.mx4_dequantize(codes, sb)[0]
        want = [float(v) for v in c.split(",")]
        assert list(got[: len(want)]) == want, row


def test_oracle_mx4_encoder_matches_input_encoder():
    # two independent implementations of the same definition agree byte for
    # byte on float32 data with blocks spread over many binades, exact ties
    # and signed zeros
    from csa_synth import mx4_quantize
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((40, 128)) * np.exp2(rng.integers(-60, 60, (40, 4))).repeat(32, 1))
    x = x.astype(np.float32)
    x[0, :32] = 0.0
    x[0, :8] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]        # ties at scale 1 (amax 6)
    x[1, :32] = 0.0
    x[1, 3] = -0.0
    x[2, :32] = -0.0
    x[3, 32:64] = [-1e-30] * 31 + [4.0]                             # tiny values round to -0
    c1, s1 = oracle.mx4_quantize(x)
    c2, s2 = mx4_quantize(torch.from_numpy(x))
    np.testing.assert_array_equal(c1, c2.numpy())
    np.testing.assert_array_equal(s1, s2.numpy())
    assert (c1[3, 16] & 0x0F) == 0x8                                # -1e-30 -> code -0
    assert s1[0, 0] == 127 and list(c1[0, :4]) == [0x20, 0x42, 0x64, 0x76]   # 0,1 | 1,2 | 2,4 | 4,6
