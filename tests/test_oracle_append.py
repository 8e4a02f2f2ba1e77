"""Pins for the KV-append oracle: the E4M3 nearest-value encoder against the published
format (golden cases, the round trip of every code, the halfway points of every pair of
neighbours, PyTorch's own float8_e4m3fn conversion), the per-token quantiser against its
error bound, and the paged scatter against the block-table gather."""
import json
import os

import numpy as np
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_nearest_golden_cases():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_spot_values.json")))
    for c in g["encode_cases"]:
        got = int(oracle.e4m3_nearest(np.array([c["x"]], np.float32))[0])
        assert got == int(c["code"], 16), c


def test_nearest_round_trips_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_nearest(vals), codes)


def test_nearest_halfway_points_go_to_even_code():
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mid = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (vals[:-1] + vals[1:]) / 2)  # exact in f32
    got = oracle.e4m3_nearest(mid).astype(np.int64)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.e4m3_nearest(-mid).astype(np.int64), want | 0x80)
    # one float32 ulp either side of a halfway point decides by distance
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    assert np.array_equal(oracle.e4m3_nearest(up).astype(np.int64), lo + 1)
    assert np.array_equal(oracle.e4m3_nearest(dn).astype(np.int64), lo)


def test_nearest_matches_torch_float8_in_range():
    """Within +-448 the format's round-to-nearest-even conversion is PyTorch's own."""
    rng = np.random.default_rng(11)
    y = (rng.standard_normal(200000) * rng.choice([1e-4, 1e-2, 1, 20, 200], 200000)).astype(np.float32)
    y = np.clip(y, -448, 448)
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_nearest(y), want)


def test_nearest_saturates():
    y = np.array([448.0, 449.0, 464.0, 480.0, 1e30, -1e30, -500.0], np.float32)
    assert list(oracle.e4m3_nearest(y)) == [0x7E] * 5 + [0xFE] * 2


def test_quantize_token_bounds():
    rng = np.random.default_rng(12)
    for mult in (1e-30, 1e-3, 1.0, 1e4):
        x = (rng.standard_normal(576) * mult).astype(np.float32)
        bits = W.bf16_bits(x)
        xv = oracle.bf16_to_f64(bits)
        codes, scale = oracle.quantize_token_fp8(bits)
        amax = np.abs(xv).max()
        assert scale == np.float32(np.float32(amax) / np.float32(448))
        deq = oracle.e4m3_decode(codes) * np.float64(scale)
        # the largest element lands on +-448 (its quotient is within an f32 ulp of 448)
        i = int(np.argmax(np.abs(xv)))
        assert codes[i] & 0x7F == 0x7E
        # relative error of E4M3 rounding: at most half a step (2^-4 of the binade) plus
        # the f32 division's rounding; absolute floor half the smallest subnormal
        err = np.abs(deq - xv)
        bound = np.maximum(np.abs(xv) * 2.0 ** -4, 2.0 ** -10 * scale) * (1 + 1e-6)
        assert np.all(err <= bound)
        assert np.all(np.signbit(oracle.e4m3_decode(codes)) == np.signbit(xv))


def test_quantize_zero_token():
    codes, scale = oracle.quantize_token_fp8(np.zeros(128, np.uint16))
    assert scale == 1.0 and np.all(codes == 0)


def _small_layout(rng, bs, nb, lens, new):
    perm = rng.permutation(nb)
    need = [-(-(c + n) // bs) for c, n in zip(lens, new)]
    width = max(need) + 1
    bt = np.full((len(lens), width), -1, np.int32)
    k = 0
    for s, m in enumerate(need):
        bt[s, :m] = perm[k:k + m]
        k += m
    q_start = np.concatenate([[0], np.cumsum(new)[:-1]]).astype(np.int32)
    return bt, np.array(lens, np.int32), np.array(new, np.int32), q_start


def test_append_gqa_then_gather():
    rng = np.random.default_rng(13)
    bs, hkv, d = 16, 2, 8
    lens, new = [0, 5, 16, 31], [3, 20, 1, 0]
    nb = 20
    bt, cl, nl, qs = _small_layout(rng, bs, nb, lens, new)
    kp = rng.integers(0, 1 << 16, (nb, hkv, bs, d), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, (nb, hkv, bs, d), dtype=np.uint16)
    n = int(nl.sum())
    kn = rng.integers(0, 1 << 16, (n, hkv, d), dtype=np.uint16)
    vn = rng.integers(0, 1 << 16, (n, hkv, d), dtype=np.uint16)
    k2, v2 = oracle.append_gqa(kp, vp, bt, cl, nl, qs, kn, vn)
    touched = np.zeros((nb, bs), bool)
    for s in range(len(lens)):
        for j in range(int(nl[s])):
            p = int(cl[s]) + j
            b, r = int(bt[s, p // bs]), p % bs
            assert np.array_equal(k2[b, :, r], kn[qs[s] + j])
            assert np.array_equal(v2[b, :, r], vn[qs[s] + j])
            touched[b, r] = True
    for b in range(nb):
        for r in range(bs):
            if not touched[b, r]:
                assert np.array_equal(k2[b, :, r], kp[b, :, r])
                assert np.array_equal(v2[b, :, r], vp[b, :, r])
    assert touched.sum() == n


def test_append_skips_out_of_range_blocks():
    bs = 4
    bt = np.array([[1, 99, -1]], np.int32)
    kp = np.zeros((2, 1, bs, 2), np.uint16)
    kn = np.arange(1, 13, dtype=np.uint16).reshape(6, 1, 2)
    k2, _ = oracle.append_gqa(kp, kp, bt, np.array([2]), np.array([6]), np.array([0]), kn, kn)
    assert np.array_equal(k2[1, 0, 2:], kn[:2, 0])     # positions 2, 3 in block 1
    assert np.all(k2[0] == 0) and np.all(k2[1, 0, :2] == 0)


def test_append_fp8_rows():
    rng = np.random.default_rng(14)
    bs, D, nb = 8, 40, 9
    lens, new = [3, 0, 8], [7, 2, 9]
    bt, cl, nl, qs = _small_layout(rng, bs, nb, lens, new)
    pool = rng.integers(0, 256, (nb, bs, D), dtype=np.uint8)
    sc = rng.random((nb, bs)).astype(np.float32)
    n = int(nl.sum())
    x = W.bf16_bits(rng.standard_normal((n, D)).astype(np.float32))
    p2, s2 = oracle.append_fp8(pool, sc, bt, cl, nl, qs, x)
    for s in range(3):
        for j in range(int(nl[s])):
            p = int(cl[s]) + j
            b, r = int(bt[s, p // bs]), p % bs
            codes, scale = oracle.quantize_token_fp8(x[qs[s] + j])
            assert np.array_equal(p2[b, r], codes) and s2[b, r] == scale
    changed = np.any(p2 != pool, axis=2) | (s2 != sc)
    assert changed.sum() == n
