"""Pins for the oracle's MXFP4 indexer keys and the packed per-block layout: E2M1 / E8M0
decoding against the OCP MX spot values, the nearest-value encoder's halfway points and
saturation, the shared-exponent rule against an independent floor(log2), closed forms of
the group quantiser, the byte layout of a packed block, and FP4 indexer scores against a
brute-force loop."""
import json
import math
import os

import numpy as np

import oracle
import workloads as W

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_spot_values.json")))
E2M1 = {int(k, 16): v for k, v in GOLDEN["e2m1"].items()}


def test_e2m1_and_e8m0_spot_values():
    got = oracle.e2m1_decode(np.arange(16))
    for c, v in E2M1.items():
        assert got[c] == v and math.copysign(1, got[c]) == math.copysign(1, v), c
    for c, v in GOLDEN["e8m0"].items():
        assert oracle.e8m0_decode(np.array([int(c)]))[0] == v, c
    assert np.isnan(oracle.e8m0_decode(np.array(GOLDEN["e8m0_nan"]))).all()


def test_mxfp4_decode_nibble_order_and_scale():
    dc = GOLDEN["decode_case"]
    packed = np.array([[int(b, 16) for b in dc["packed"]]], np.uint8)
    # one group of 32 needs 16 bytes: pad with zero codes
    packed = np.concatenate([packed, np.zeros((1, 14), np.uint8)], axis=1)
    got = oracle.mxfp4_decode(packed, np.array([[dc["scale"]]], np.uint8))
    assert list(got[0, :4]) == dc["elements"] and np.all(got[0, 4:] == 0)


def test_e2m1_nearest_golden_cases_and_round_trip():
    for c in GOLDEN["encode_cases"]:
        assert int(oracle.e2m1_nearest(np.array([c["x"]]))[0]) == int(c["code"], 16), c
    vals = oracle.e2m1_decode(np.arange(16))
    assert np.array_equal(oracle.e2m1_nearest(vals), np.arange(16, dtype=np.uint8))


def test_e2m1_nearest_halfway_points_and_neighbours():
    pos = oracle.e2m1_decode(np.arange(8))
    mid = (pos[:-1] + pos[1:]) / 2
    lo = np.arange(7)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(oracle.e2m1_nearest(mid).astype(int), want)
    assert np.array_equal(oracle.e2m1_nearest(-mid).astype(int), want | 0x8)
    assert np.array_equal(oracle.e2m1_nearest(np.nextafter(mid, np.inf)).astype(int), lo + 1)
    assert np.array_equal(oracle.e2m1_nearest(np.nextafter(mid, 0)).astype(int), lo)
    assert list(oracle.e2m1_nearest(np.array([6.0, 7.0, 7.99, 1e9, -1e9]))) == [7, 7, 7, 7, 15]


def test_shared_exponent_is_floor_log2_minus_two():
    rng = np.random.default_rng(3)
    amax = np.concatenate([np.exp2(rng.uniform(-30, 30, 2000)), np.exp2(np.arange(-20, 21, dtype=np.float64)),
                           [1.0, 3.999, 4.0, 6.0, 7.99, 8.0]])
    for a in amax:
        assert oracle.mx_shared_exponent(float(a)) == math.floor(math.log2(float(a))) - 2 + 127, a
    assert oracle.mx_shared_exponent(0.0) == 127
    assert oracle.mx_shared_exponent(2.0 ** -130) == 2           # clamped: codes stay in [2, 252]


def _bits(x):
    return W.bf16_bits(np.asarray(x, np.float32))


def test_quantize_group_closed_forms():
    rng = np.random.default_rng(4)
    # values exactly on the grid of a power-of-two scale, with the group max at 6 X or 4 X,
    # quantise back to the same codes
    for k in (-3, 0, 5):
        codes = rng.integers(0, 16, 128).astype(np.uint8)
        codes[0::32] = 7                                   # every group holds +6
        codes[1::64] = 14                                  # and some hold -4
        x = oracle.e2m1_decode(codes) * 2.0 ** k
        packed, scales = oracle.quantize_token_mxfp4(_bits(x))
        assert np.all(scales == 127 + k)
        back = np.empty(128, np.uint8)
        back[0::2], back[1::2] = packed & 0xF, packed >> 4
        zero = oracle.e2m1_decode(codes) == 0
        assert np.array_equal(back[~zero], codes[~zero]) and np.all((back[zero] & 7) == 0)
    # random groups: the largest element decodes to 4 X or 6 X; errors within the grid
    # spacing (X/2 below 2X, X in [2X, 4X), 2X above: bound X), saturation past 6 X
    for _ in range(50):
        x = W.bf16_bits_to_f32(_bits(rng.standard_normal(128) * rng.choice([1e-3, 1, 50]))).astype(np.float64)
        packed, scales = oracle.quantize_token_mxfp4(_bits(x))
        dq = oracle.mxfp4_decode(packed[None], scales[None])[0]
        X = np.repeat(np.ldexp(1.0, scales.astype(int) - 127), 32)
        for g in range(4):
            i = np.argmax(np.abs(x[32 * g:32 * g + 32])) + 32 * g
            assert abs(dq[i]) in (4 * X[i], 6 * X[i])
        assert np.all(np.abs(dq - x) <= np.maximum(X, np.abs(x) - 6 * X) + 1e-300)
        assert np.all(np.sign(dq[dq != 0]) == np.sign(x[dq != 0]))
    # an all-zero group: scale code 127, zero codes
    packed, scales = oracle.quantize_token_mxfp4(_bits(np.zeros(128)))
    assert np.all(scales == 127) and np.all(packed == 0)


def test_packed_block_layout_and_append():
    assert (oracle.PACKED_LATENT, oracle.PACKED_LATENT_SCALE, oracle.PACKED_KEYS, oracle.PACKED_KEY_SCALES,
            oracle.PACKED_BLOCK_BYTES) == (0, 36864, 37120, 41216, 41472)
    rng = np.random.default_rng(5)
    nb = 6
    pool = rng.integers(0, 256, (nb, oracle.PACKED_BLOCK_BYTES)).astype(np.uint8)
    bt = np.array([[4, 1, -1], [2, 5, -1]], np.int32)
    cached, new, qs = np.array([60, 0]), np.array([6, 3]), np.array([0, 6])
    lat = _bits(rng.standard_normal((9, 576)))
    keys = _bits(rng.standard_normal((9, 128)))
    p1 = oracle.append_packed(pool, bt, cached, new, qs, lat, "latent")
    p2 = oracle.append_packed(p1, bt, cached, new, qs, keys, "keys")
    l_, ls, k_, ks = oracle.packed_fields(p2)
    changed = np.zeros_like(pool, bool)
    for i in range(9):
        s = 0 if i < 6 else 1
        t = int(cached[s]) + i - int(qs[s])
        b, r = int(bt[s, t // 64]), t % 64
        c, sc = oracle.quantize_token_fp8(lat[i])
        pk, ksc = oracle.quantize_token_mxfp4(keys[i])
        assert np.array_equal(l_[b, r], c) and ls[b, r] == sc
        assert np.array_equal(k_[b, r], pk) and np.array_equal(ks[b, r], ksc)
        # the byte ranges of this row, by the stated offsets
        changed[b, 576 * r:576 * r + 576] = True
        changed[b, 36864 + 4 * r:36864 + 4 * r + 4] = True
        changed[b, 37120 + 64 * r:37120 + 64 * r + 64] = True
        changed[b, 41216 + 4 * r:41216 + 4 * r + 4] = True
    assert np.array_equal(p2[~changed], pool[~changed])


def test_indexer_scores_mxfp4_brute_force():
    rng = np.random.default_rng(6)
    n, H, d, L = 3, 2, 64, 9
    q = _bits(rng.standard_normal((n, H, d)))
    w = rng.standard_normal((n, H)).astype(np.float32)
    x = _bits(rng.standard_normal((L, d)))
    packed = np.empty((L, d // 2), np.uint8)
    scales = np.empty((L, d // 32), np.uint8)
    for t in range(L):
        packed[t], scales[t] = oracle.quantize_token_mxfp4(x[t])
    pos = np.array([0, 4, 8])
    got = oracle.indexer_scores_mxfp4(q, w, packed, scales, pos)
    qf = W.bf16_bits_to_f32(q).astype(np.float64)
    for i in range(n):
        for t in range(L):
            if t > pos[i]:
                assert got[i, t] == -np.inf
                continue
            kt = []
            for j in range(d):           # decode element j from the golden table, by hand
                byte = int(packed[t, j // 2])
                code = byte & 0xF if j % 2 == 0 else byte >> 4
                kt.append(E2M1[code] * 2.0 ** (int(scales[t, j // 32]) - 127))
            ref = math.fsum(float(w[i, h]) * max(0.0, math.fsum(qf[i, h, j] * kt[j] for j in range(d)))
                            for h in range(H))
            assert abs(got[i, t] - ref) <= 1e-12 * max(1.0, abs(ref))
