"""Pins of the E4M3 codec: values the OCP FP8 specification tables give,
closed-form properties of rounding to nearest even, and a brute-force
nearest-value search."""
import numpy as np

from oracle.fp8 import MAX_E4M3, decode_e4m3, dequantize, encode_e4m3, quantize


def test_spec_values():
    # OCP 8-bit FP spec, E4M3: bias 7, max normal S.1111.110 = 448,
    # min normal S.0001.000 = 2^-6, max subnormal S.0000.111 = 0.875 * 2^-6,
    # min subnormal S.0000.001 = 2^-9, NaN S.1111.111, zeros S.0000.000
    table = {0x7E: 448.0, 0x08: 2.0 ** -6, 0x07: 0.875 * 2.0 ** -6, 0x01: 2.0 ** -9,
             0x38: 1.0, 0x40: 2.0, 0xC0: -2.0, 0x00: 0.0, 0x3C: 1.5, 0x77: 240.0}
    for code, val in table.items():
        assert decode_e4m3([code])[0] == val, hex(code)
    assert np.isnan(decode_e4m3([0x7F, 0xFF])).all()
    assert np.signbit(decode_e4m3([0x80])[0]) and decode_e4m3([0x80])[0] == 0.0
    finite = decode_e4m3(np.arange(256))
    assert np.isnan(finite).sum() == 2 and np.nanmax(finite) == MAX_E4M3


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(encode_e4m3(decode_e4m3(codes)), codes)


def test_ties_go_to_the_even_mantissa_and_saturation():
    # 1.0625 lies halfway between 1.0 (m=000) and 1.125 (m=001): -> 1.0;
    # 1.1875 between 1.125 (001) and 1.25 (010): -> 1.25
    assert decode_e4m3(encode_e4m3([1.0625, 1.1875, -1.0625]))[:].tolist() == [1.0, 1.25, -1.0]
    # halfway between the two smallest subnormals 2^-9 and 2^-8: -> 2^-8 (even)
    assert decode_e4m3(encode_e4m3([1.5 * 2.0 ** -9]))[0] == 2.0 ** -8
    # below half the smallest subnormal: zero, keeping the sign
    z = encode_e4m3([2.0 ** -11, -2.0 ** -11])
    assert z.tolist() == [0x00, 0x80]
    assert encode_e4m3([500.0, -1e9, np.inf, -np.inf]).tolist() == [0x7E, 0xFE, 0x7E, 0xFE]
    assert encode_e4m3([np.nan]).tolist() == [0x7F]


def test_encoder_equals_brute_force_nearest_on_random_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.uniform(-4, 3, 4000),
                        rng.uniform(-460, 460, 2000)])
    codes = encode_e4m3(x)
    allc = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = decode_e4m3(allc)
    for xi, ci in zip(x, codes):
        xc = min(max(xi, -448.0), 448.0)
        d = np.abs(vals - xc)
        best = allc[d == d.min()]
        if len(best) > 1:                               # a tie: the even mantissa, same sign
            best = [b for b in best if (b & 1) == 0 and bool(b >> 7) == (xi < 0)] or best
        assert decode_e4m3([ci])[0] == decode_e4m3([best[0]])[0], (xi, hex(ci))


def test_quantize_table_equals_the_encoder_value_by_value():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3000).astype(np.float16) * np.float16(20)
    for scale in (1.0, 0.0123, 7.0):
        inv = np.float32(1.0) / np.float32(scale)
        direct = np.array([encode_e4m3([float(np.float32(xi) * inv)])[0] for xi in x])
        assert np.array_equal(quantize(x, scale), direct)


def test_quantize_uses_the_fp32_reciprocal_of_the_scale():
    x = np.array([0.5, -3.0, 100.0], dtype=np.float16)
    scale = 0.3
    inv = np.float32(1.0) / np.float32(scale)
    exp = encode_e4m3((x.astype(np.float32) * inv).astype(np.float64))
    assert np.array_equal(quantize(x, scale), exp)
    assert np.allclose(dequantize(quantize(x, scale), scale), x, rtol=0.07)


def test_fp8_pool_stores_representable_rows_exactly():
    # rows made of E4M3 values times a power-of-two scale survive the pool unchanged
    from oracle import Fp8PoolModel
    rng = np.random.default_rng(1)
    finite = decode_e4m3(np.arange(0x7F))                # 0 .. 448, non-negative codes
    rows = rng.choice(finite[finite <= 64], size=(20, 2, 64)) * rng.choice([-1, 1], (20, 2, 64))
    k16 = (rows * 0.25).astype(np.float16)               # exact in fp16
    v16 = (rows * 2.0).astype(np.float16)
    pool = Fp8PoolModel(8, 2, 64, k_scale=0.25, v_scale=2.0)
    table = [5, 2]
    pool.write(k16, v16, [table[t // 16] * 16 + t % 16 for t in range(20)])
    k, v = pool.gather_values(table, 20)
    assert np.array_equal(k, k16.astype(np.float64)) and np.array_equal(v, v16.astype(np.float64))
