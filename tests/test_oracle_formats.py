"""Pins for the storage formats: the oracle's decoders against the published format
definitions, and the input generator's encoders against the oracle's decoders."""
import json
import os

import numpy as np

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_spot_values():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_spot_values.json")))
    for code, val in g["values"].items():
        got = oracle.e4m3_decode(np.array([int(code, 16)], np.uint8))[0]
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)
    for code in g["nan_codes"]:
        assert np.isnan(oracle.e4m3_decode(np.array([int(code, 16)], np.uint8))[0])


def test_e4m3_table_structure():
    vals = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = vals[np.isfinite(vals)]
    assert finite.size == 254                      # only 0x7F and 0xFF are NaN
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)                # monotone over positive codes
    assert np.array_equal(vals[0x80:0xFF], -vals[:0x7F])
    assert pos.max() == 448.0 and pos[1] == 2.0 ** -9


def test_encoder_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    back = W.e4m3_encode(vals)
    assert np.array_equal(back, codes)


def test_encoder_rounding_cases():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_spot_values.json")))
    for c in g["encode_cases"]:
        got = int(W.e4m3_encode(np.array([c["x"]], np.float32))[0])
        assert got == int(c["code"], 16), c


def test_encoder_is_nearest():
    """Every encoded value is a nearest representable value (brute force over the table)."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * rng.choice([1e-3, 1e-1, 1, 30, 300], 20000)).astype(np.float32)
    x = np.clip(x, -448, 448)
    codes = W.e4m3_encode(x)
    table = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = np.isfinite(table)
    err = np.abs(oracle.e4m3_decode(codes) - x.astype(np.float64))
    best = np.min(np.abs(table[fin][None, :] - x[:, None].astype(np.float64)), axis=1)
    assert np.all(err <= best)


def test_per_token_quantisation():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((50, 576)).astype(np.float32)
    codes, scale = W.fp8_quantize_tokens(x)
    deq = oracle.e4m3_decode(codes) * scale[:, None]
    amax = np.abs(x).max(1)
    np.testing.assert_allclose(scale, amax / 448, rtol=1e-7)
    assert np.all(np.abs(deq).max(1) <= amax * (1 + 1e-6))
    assert np.max(np.abs(deq - x) / amax[:, None]) <= 2.0 ** -4 * 1.0001   # half an ulp at 448 scale


def test_bf16_decode_and_encode():
    x = np.array([1.0, -2.5, 3.140625, 1e-3, 65504.0], np.float32)
    bits = W.bf16_bits(x)
    assert bits[0] == 0x3F80 and bits[1] == 0xC020
    back = oracle.bf16_to_f64(bits)
    assert back[0] == 1.0 and back[1] == -2.5 and back[2] == 3.140625
    # round to nearest even at the halfway point 1 + 2^-8
    assert W.bf16_bits(np.array([1.0 + 2.0 ** -8], np.float32))[0] == 0x3F80
    assert W.bf16_bits(np.array([1.0 + 3 * 2.0 ** -8], np.float32))[0] == 0x3F82
