"""Pins of the oracle quantizer and packer ([P1 para 1, 3, 4, 5]; [P1] =
ihal.it/?p=61653).  CPU only."""
import os

import numpy as np
import pytest

import oracle
from oracle import quantize_groups, quantize_k, quantize_v, pack_codes, unpack_codes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_quant_cases():
    lines = [l.strip() for l in open(os.path.join(GOLDEN, "quant_groups.txt"))
             if l.strip() and not l.startswith("#")]
    cases = []
    for head, exp in zip(lines[0::2], lines[1::2]):
        name, bits, vals = [p.strip() for p in head.split("|")]
        s, z, codes = [p.strip() for p in exp.split("|")]
        cases.append((name, int(bits), np.array(vals.split(), np.float64),
                      float(s), float(z), np.array(codes.split(), np.int64)))
    return cases


@pytest.mark.parametrize("case", _read_quant_cases(), ids=lambda c: c[0])
def test_hand_fixtures(case):
    name, bits, vals, s, z, codes = case
    x16 = vals.astype(np.float16)
    assert np.all(x16.astype(np.float64) == vals), "fixture values must be fp16-exact"
    q, sc, ze = quantize_groups(x16[None], bits)
    assert float(sc[0]) == s
    assert float(ze[0]) == z
    np.testing.assert_array_equal(q[0], codes)


def _random_groups(rng, n, spread=1.0):
    x = rng.standard_normal((n, 32)) * spread
    # some groups with an outlier that widens the step ([P1 para 3])
    x[::7, 3] *= 40.0
    return x.astype(np.float16)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_levels_are_exactly_two_to_the_b(bits):
    rng = np.random.default_rng(0)
    x16 = _random_groups(rng, 500)
    q, s, z = quantize_groups(x16, bits)
    L = 2 ** bits - 1
    assert q.max() <= L
    xh = q * s.astype(np.float64)[:, None] + z.astype(np.float64)[:, None]
    for g in range(x16.shape[0]):
        lv = z[g].astype(np.float64) + np.arange(L + 1) * float(s[g])
        assert np.all(np.isin(xh[g], lv))
    if bits == 2:
        # a group holding exactly the four levels uses all four codes
        ramp = np.tile(np.array([0.0, 1.0, 2.0, 3.0]) * 0.5 - 1.0, 8).astype(np.float16)
        qq, ss, zz = quantize_groups(ramp[None], 2)
        assert sorted(set(qq[0].tolist())) == [0, 1, 2, 3]


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_constant_group_round_trips(bits):
    for val in [0.0, -3.25, 7.5, 1e-3, 60000.0, -2.0 ** -20]:
        x16 = np.full((1, 32), val, np.float16)
        q, s, z = quantize_groups(x16, bits)
        assert float(s[0]) == 0.0
        assert np.all(q == 0)
        xh = q * s.astype(np.float64)[:, None] + z.astype(np.float64)[:, None]
        assert np.array_equal(xh, x16.astype(np.float64))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_error_at_most_half_scale(bits):
    rng = np.random.default_rng(1)
    x16 = np.concatenate([_random_groups(rng, 2000), _random_groups(rng, 500, 300.0)])
    q, s, z = quantize_groups(x16, bits)
    sf = s.astype(np.float64)[:, None]
    assert np.all(sf >= 2.0 ** -14)           # the bound is stated for normal scales
    xh = q * sf + z.astype(np.float64)[:, None]
    err = np.abs(x16.astype(np.float64) - xh)
    L = 2 ** bits - 1
    # s/2 plus the two fp32 roundings (difference, quotient) of t = (x - z)/s
    assert np.all(err <= sf * (0.5 + L * 2.0 ** -22))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_nearest_level_by_brute_force(bits):
    rng = np.random.default_rng(2)
    x16 = _random_groups(rng, 300)
    q, s, z = quantize_groups(x16, bits)
    L = 2 ** bits - 1
    lv = z.astype(np.float64)[:, None, None] + np.arange(L + 1)[None, None, :] * s.astype(np.float64)[:, None, None]
    dist = np.abs(x16.astype(np.float64)[:, :, None] - lv)        # [g, 32, L+1]
    best = dist.min(axis=2)
    chosen = np.take_along_axis(dist, q[:, :, None].astype(np.int64), axis=2)[:, :, 0]
    sf = s.astype(np.float64)[:, None]
    assert np.all(chosen <= best + sf * L * 2.0 ** -21)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_codes_hit_both_ends(bits):
    rng = np.random.default_rng(3)
    x16 = _random_groups(rng, 400)
    q, s, z = quantize_groups(x16, bits)
    nonconst = s.astype(np.float64) > 0
    assert np.all(q[nonconst].min(axis=1) == 0)
    assert np.all(q[nonconst].max(axis=1) == 2 ** bits - 1)


def test_axis_pins_keys_per_channel_values_per_token():
    rng = np.random.default_rng(4)
    B, H, T, d = 2, 3, 64, 64
    # keys constant over tokens within each channel, different across channels
    kc = rng.standard_normal((B, H, 1, d)) * 10
    k16 = np.broadcast_to(kc, (B, H, T, d)).astype(np.float16)
    codes, s, z = quantize_k(k16, 2)
    kh = oracle.dequantize_k(codes, s, z)
    assert np.array_equal(kh, k16.astype(np.float64))
    # grouping the same keys along channels (the wrong axis) loses them
    codes_t, s_t, z_t = quantize_v(k16, 2)
    kh_t = oracle.dequantize_v(codes_t, s_t, z_t)
    assert not np.array_equal(kh_t, k16.astype(np.float64))
    # values constant over channels within each token
    vc = rng.standard_normal((B, H, T, 1)) * 10
    v16 = np.broadcast_to(vc, (B, H, T, d)).astype(np.float16)
    codes, s, z = quantize_v(v16, 2)
    assert np.array_equal(oracle.dequantize_v(codes, s, z), v16.astype(np.float64))
    codes_c, s_c, z_c = quantize_k(v16, 2)
    assert not np.array_equal(oracle.dequantize_k(codes_c, s_c, z_c), v16.astype(np.float64))


def test_group_shapes_and_membership():
    # key group (b, h, g, c) is channel c over tokens 32g..32g+31; value
    # group (b, h, t, j) is token t over channels 32j..32j+31
    rng = np.random.default_rng(5)
    k16 = rng.standard_normal((1, 2, 96, 64)).astype(np.float16)
    codes, s, z = quantize_k(k16, 4)
    assert s.shape == (1, 2, 3, 64) and codes.shape == k16.shape
    q1, s1, z1 = quantize_groups(k16[0, 1, 32:64, 17][None], 4)
    assert s1[0] == s[0, 1, 1, 17] and z1[0] == z[0, 1, 1, 17]
    np.testing.assert_array_equal(q1[0], codes[0, 1, 32:64, 17])
    codes, s, z = quantize_v(k16, 4)
    assert s.shape == (1, 2, 96, 2)
    q1, s1, z1 = quantize_groups(k16[0, 0, 70, 32:64][None], 4)
    assert s1[0] == s[0, 0, 70, 1]
    np.testing.assert_array_equal(q1[0], codes[0, 0, 70, 32:64])


def _read_pack_cases():
    cases = []
    for l in open(os.path.join(GOLDEN, "pack_words.txt")):
        l = l.strip()
        if not l or l.startswith("#"):
            continue
        bits, codes, words = [p.strip() for p in l.split("|")]
        cases.append((int(bits), np.array(codes.split(), np.uint8),
                      np.array([int(w, 16) for w in words.split()], np.uint32)))
    return cases


@pytest.mark.parametrize("case", _read_pack_cases())
def test_pack_hand_fixtures(case):
    bits, codes, words = case
    np.testing.assert_array_equal(pack_codes(codes, bits), words)
    np.testing.assert_array_equal(unpack_codes(words, bits, codes.size), codes)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_pack_bit_positions_brute_force(bits):
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 2 ** bits, size=(3, 5, 64), dtype=np.uint8)
    words = pack_codes(codes, bits)
    assert words.shape == (3, 5, 64 * bits // 32)
    # build the whole stream as one Python integer and read every field back
    stream = 0
    for i, w in enumerate(words.reshape(-1).tolist()):
        stream |= int(w) << (32 * i)
    for f, c in enumerate(codes.reshape(-1).tolist()):
        assert (stream >> (f * bits)) & (2 ** bits - 1) == c
    np.testing.assert_array_equal(unpack_codes(words, bits, 64), codes)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_value_pack_block_order_brute_force(bits):
    """Value codes: 32-token blocks, channel-major inside a block, one bit
    stream; element (t, c) of a unit sits at stream index
    (t // 32) * 32 * d + c * 32 + t % 32."""
    rng = np.random.default_rng(7)
    d, T = 64, 96
    codes = rng.integers(0, 2 ** bits, size=(2, 1, T, d), dtype=np.uint8)
    words = oracle.pack_v_codes(codes, bits)
    assert words.shape == (2, 1, T // 32, d * bits)
    for b in range(2):
        stream = 0
        for i, w in enumerate(words[b, 0].reshape(-1).tolist()):
            stream |= int(w) << (32 * i)
        for t in range(T):
            for c in range(d):
                f = (t // 32) * 32 * d + c * 32 + t % 32
                assert (stream >> (f * bits)) & (2 ** bits - 1) == codes[b, 0, t, c]
    np.testing.assert_array_equal(oracle.unpack_v_codes(words, bits, d), codes)


def test_value_pack_hand_word():
    # 2-bit, one 32-token block, d = 32: channel 0's tokens 0..15 fill word
    # 0; token 1 of channel 0 has code 3 -> bits 2..3 -> 0x0000000C; token 16
    # of channel 1 (stream index 32 + 16 = 48 -> word 3, bits 0..1) has code 1
    codes = np.zeros((1, 1, 32, 32), np.uint8)
    codes[0, 0, 1, 0] = 3
    codes[0, 0, 16, 1] = 1
    words = oracle.pack_v_codes(codes, 2)[0, 0, 0]
    assert words[0] == 0x0000000C and words[3] == 0x00000001
    assert np.count_nonzero(words) == 2
