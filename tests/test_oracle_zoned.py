"""Pins of the mixed-width (TriZone) oracle ([P3 sec 2.2, bit-allocation
pipeline] and [P3 sec 2.2, TriZone packed decoding]; [P3] = RDKV summary,
gist.science/it/paper/2605.08317).  CPU only."""
import numpy as np
import pytest

import oracle
from oracle import zoned_pack, zoned_layout, zoned_decode_attention, attention_fp64
from workloads import zoned_inputs

PROBS_V = {0: 0.5, 2: 0.2, 4: 0.15, 8: 0.1, 16: 0.05}
PROBS_K = {2: 0.4, 4: 0.3, 8: 0.2, 16: 0.1}


def _small(seed, T=200, C=8, B=1, Hkv=2, Hq=4, d=64, pv=PROBS_V, pk=PROBS_K):
    return zoned_inputs(B, Hq, Hkv, d, T, C, seed, pv, pk, ("lognormal", 0.04, 3.0, 1.0))


def _zoned(inp, **kw):
    return zoned_decode_attention(inp["q"], inp["k"], inp["v"], inp["v_bits"],
                                  inp["k_bits"], inp["k_new"], inp["v_new"], 0.125, **kw)


def test_all_sixteen_bit_is_unquantized_attention():
    inp = _small(0)
    inp["v_bits"][:] = 16
    inp["k_bits"][:] = 16
    o = _zoned(inp)
    B, Hq, d = inp["q"].shape
    for b in range(B):
        for h in range(Hq):
            kv = h // 2
            k = np.concatenate([inp["k"][b, kv], inp["k_new"][b, kv]]).astype(np.float64)
            v = np.concatenate([inp["v"][b, kv], inp["v_new"][b, kv]]).astype(np.float64)
            ref = attention_fp64(inp["q"][b, h][None].astype(np.float64), k, v, 0.125)
            np.testing.assert_allclose(o[b, h], ref[0], rtol=1e-11, atol=1e-13)


def test_width_zero_is_eviction():
    inp = _small(1, T=256)
    keep = inp["v_bits"][0, 0] != 0
    assert (~keep).sum() > 50
    o = _zoned(inp)
    # same cache with the evicted tokens deleted (all units share the cut)
    inp2 = dict(inp)
    mask = np.ones(256, bool)
    mask[~keep] = False
    vb = inp["v_bits"].copy()
    vb[:, :, ~mask] = 0
    inp["v_bits"] = vb
    o_masked = _zoned(inp)
    inp2["k"] = inp["k"][:, :, mask]
    inp2["v"] = inp["v"][:, :, mask]
    inp2["v_bits"] = vb[:, :, mask]
    o_deleted = _zoned(inp2)
    np.testing.assert_allclose(o_masked, o_deleted, rtol=1e-12, atol=1e-14)
    # byte image identical too: evicted tokens leave no trace
    b1 = zoned_pack(inp["k"], inp["v"], inp["v_bits"], inp["k_bits"], inp["k_new"], inp["v_new"])
    b2 = zoned_pack(inp2["k"], inp2["v"], inp2["v_bits"], inp2["k_bits"], inp2["k_new"], inp2["v_new"])
    assert np.array_equal(b1, b2)
    # and evicting changes the result compared with keeping those tokens
    assert not np.allclose(o, _zoned(dict(inp2, v_bits=np.full_like(inp2["v_bits"], 2))))


def test_single_width_equals_uniform_layout():
    # every token at value width 2 and every key channel at width 2: the
    # segments are the token order, so the result is the uniform
    # (per-channel K, per-token V) 2-bit cache with no recent zone, plus the
    # fp16 new tokens
    inp = _small(2, T=192, C=0)
    inp["v_bits"][:] = 2
    inp["k_bits"][:] = 2
    o = _zoned(inp)
    kc, ks, kz = oracle.quantize_k(inp["k"], 2)
    vc, vs, vz = oracle.quantize_v(inp["v"], 2)
    cache = dict(B=1, Hq=4, Hkv=2, d=64, bits=2, T_q=192, R=0, rope_theta=0.0,
                 k_codes=oracle.pack_codes(kc, 2), v_codes=oracle.pack_v_codes(vc, 2),
                 k_scale=ks, k_zero=kz, v_scale=vs, v_zero=vz,
                 k_recent=np.zeros((1, 2, 0, 64), np.float16), v_recent=np.zeros((1, 2, 0, 64), np.float16))
    ref = oracle.kivi_decode_attention(inp["q"], cache, 0.125)
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-13)
    # and the key words of the blob are exactly the uniform layout's words
    blob = zoned_pack(inp["k"], inp["v"], inp["v_bits"], inp["k_bits"], inp["k_new"], inp["v_new"])
    units, total = zoned_layout(inp["v_bits"], inp["k_bits"], 64, 0)
    lay = units[1]
    g1 = lay["base"] + lay["seg"][2]["offset"] + 1 * lay["seg"][2]["group_bytes"]
    words = blob[g1:g1 + 32 * lay["W_K"] * 4].view(np.uint32).reshape(32, lay["W_K"])
    np.testing.assert_array_equal(words, cache["k_codes"][0, 1, 32:64])


def test_segments_key_classes_and_zones():
    inp = _small(3, T=300, C=8)
    blob = zoned_pack(inp["k"], inp["v"], inp["v_bits"], inp["k_bits"], inp["k_new"], inp["v_new"])
    units, total = zoned_layout(inp["v_bits"], inp["k_bits"], 64, 8)
    assert blob.size == total and total % 256 == 0
    for u, lay in enumerate(units):
        b, h = divmod(u, 2)
        vb, kb = inp["v_bits"][b, h], inp["k_bits"][b, h]
        # segments: kept tokens by width, token order preserved
        for w in (2, 4, 8, 16):
            np.testing.assert_array_equal(lay["seg"][w]["tokens"], np.flatnonzero(vb == w))
            assert lay["seg"][w]["P"] % 32 == 0 and lay["seg"][w]["P"] - lay["seg"][w]["n"] < 32
        assert sum(lay["seg"][w]["n"] for w in (2, 4, 8, 16)) == (vb != 0).sum()
        assert sum(lay["m"].values()) == 64
        # zone C = raw bytes of the new tokens
        zc = lay["base"] + lay["zone_c"]
        assert np.array_equal(blob[zc:zc + 8 * 64 * 2].view(np.float16).reshape(8, 64), inp["k_new"][b, h])
        assert np.array_equal(blob[zc + 1024:zc + 2048].view(np.float16).reshape(8, 64), inp["v_new"][b, h])
        # zone B = raw fp16 values of the 16-bit tokens, masked slots zero
        zb = lay["base"] + lay["zone_b"]
        rows = blob[zb:zb + lay["seg"][16]["P"] * 128].view(np.float16).reshape(-1, 64)
        n16 = lay["seg"][16]["n"]
        assert np.array_equal(rows[:n16], inp["v"][b, h][vb == 16])
        assert np.all(rows[n16:] == 0)
        # 16-bit key channels: raw fp16 in the last key-class block
        if lay["m"][16] and lay["seg"][4]["n"]:
            g0 = lay["base"] + lay["seg"][4]["offset"]
            kr = blob[g0:g0 + 32 * lay["W_K"] * 4].view(np.uint32).reshape(32, lay["W_K"])
            raw_words = kr[:, lay["W_K"] - lay["kwords"][16]:]
            halves = np.stack([raw_words & 0xFFFF, raw_words >> 16], 2).reshape(32, -1)[:, :lay["m"][16]]
            n = min(32, lay["seg"][4]["n"])
            expect = inp["k"][b, h][lay["seg"][4]["tokens"][:n]][:, lay["classes"][16]].view(np.uint16)
            np.testing.assert_array_equal(halves[:n].astype(np.uint16), expect)


def test_hand_built_key_row():
    # one token, d = 64: channels 0..31 at width 2 would need a full test of
    # the row layout; here 4 channels at width 4 (the rest 16-bit) and a
    # group of two valid tokens with hand-computable codes
    d = 64
    k = np.zeros((1, 1, 2, d), np.float16)
    k[0, 0, :, :] = np.arange(d, dtype=np.float16)       # 16-bit channels: 0..63
    k[0, 0, 0, :4] = [0.0, 1.0, 2.0, 3.0]
    k[0, 0, 1, :4] = [15.0, 16.0, 17.0, 18.0]            # range 15 per channel
    v = np.zeros((1, 1, 2, d), np.float16)
    vb = np.full((1, 1, 2), 16, np.int8)
    kb = np.full((1, 1, d), 16, np.int8)
    kb[0, 0, :4] = 4
    blob = zoned_pack(k, v, vb, kb, np.zeros((1, 1, 0, d), np.float16), np.zeros((1, 1, 0, d), np.float16))
    units, _ = zoned_layout(vb, kb, d, 0)
    lay = units[0]
    assert lay["W_K"] == 1 + 30            # 4 channels x 4 bits, then 60 fp16 = 30 words
    row = blob[:32 * lay["W_K"] * 4].view(np.uint32).reshape(32, lay["W_K"])
    # scale = 15/15 = 1, zero = channel min: token 0 -> codes 0, token 1 -> 15
    assert row[0, 0] == 0x0000 and row[1, 0] == 0xFFFF
    assert np.all(row[2:] == 0)                          # masked slots
    # fp16 channel 4 and 5 of token 0: 4.0 = 0x4400, 5.0 = 0x4500
    assert row[0, 1] == (0x4500 << 16 | 0x4400)


def test_directional_values_per_token_under_peaked_attention():
    # [P1 para 5, 6]: with peaked attention, per-token value grouping gives a
    # lower attention-output error than per-channel grouping (directional
    # check on synthetic data)
    rng = np.random.default_rng(9)
    T, d = 1024, 128
    v = rng.standard_normal((1, 1, T, d)).astype(np.float16)
    logits = rng.standard_normal(T) * 4.0
    p = np.exp(logits - logits.max())
    p /= p.sum()
    exact = p @ v[0, 0].astype(np.float64)
    c, s, z = oracle.quantize_v(v, 2)
    e_tok = np.linalg.norm(p @ oracle.dequantize_v(c, s, z)[0, 0] - exact)
    c, s, z = oracle.quantize_k(v, 2)
    e_ch = np.linalg.norm(p @ oracle.dequantize_k(c, s, z)[0, 0] - exact)
    assert e_tok < e_ch


def test_key_width_zero_is_a_zeroed_channel():
    """A key channel of width 0 ([P3 sec 2.1]: weight = logit change when the
    channel is zeroed) equals that channel stored raw with every old token's
    key component set to 0, bit for bit; the new tokens keep the channel."""
    inp = _small(3, pk={0: 0.3, 2: 0.3, 4: 0.2, 16: 0.2})
    ev = inp["k_bits"] == 0
    assert ev.sum() > 5 and (~ev).sum() > 5
    o = _zoned(inp)
    k2, kb2 = inp["k"].copy(), inp["k_bits"].copy()
    for b, h in np.ndindex(ev.shape[:2]):
        k2[b, h][:, ev[b, h]] = 0
        kb2[b, h][ev[b, h]] = 16
    np.testing.assert_array_equal(o, _zoned(dict(inp, k=k2, k_bits=kb2)))
    # evicting differs from keeping the channel at full precision
    kb3 = np.where(ev, 16, inp["k_bits"]).astype(inp["k_bits"].dtype)
    assert not np.allclose(o, _zoned(dict(inp, k_bits=kb3)))
    # every key channel evicted: old tokens all score 0 against every query
    o0 = _zoned(dict(inp, k_bits=np.zeros_like(inp["k_bits"])))
    k4 = np.zeros_like(inp["k"])
    np.testing.assert_array_equal(o0, _zoned(dict(inp, k=k4, k_bits=np.full_like(inp["k_bits"], 16))))


# ------------------------------------------------------------ sink window

def test_sink_tokens_are_new_tokens_at_the_front():
    # A sink of S tokens is the same cache as: those tokens evicted from the
    # old cache and placed (fp16, all channels) before the new tokens.  Both
    # the byte image and the attention must agree exactly.
    inp = _small(21, T=150, C=5)
    S = 9
    kw = dict(sink=S)
    o = _zoned(inp, **kw)
    alt = dict(inp)
    vb = inp["v_bits"].copy()
    vb[:, :, :S] = 0
    alt["v_bits"] = vb
    alt["k_new"] = np.concatenate([inp["k"][:, :, :S], inp["k_new"]], axis=2)
    alt["v_new"] = np.concatenate([inp["v"][:, :, :S], inp["v_new"]], axis=2)
    np.testing.assert_allclose(o, _zoned(alt), rtol=1e-12, atol=1e-14)
    b1 = zoned_pack(inp["k"], inp["v"], inp["v_bits"], inp["k_bits"], inp["k_new"], inp["v_new"], sink=S)
    b2 = zoned_pack(alt["k"], alt["v"], alt["v_bits"], alt["k_bits"], alt["k_new"], alt["v_new"])
    assert np.array_equal(b1, b2)
    # the sink overrides eviction: a sink changes the result when its tokens
    # were evicted
    assert (inp["v_bits"][:, :, :S] == 0).any()
    assert not np.allclose(o, _zoned(inp))


def test_whole_cache_as_sink_is_unquantized_attention():
    inp = _small(22, T=40, C=3)
    o = _zoned(inp, sink=40)
    B, Hq, d = inp["q"].shape
    for b in range(B):
        for h in range(Hq):
            kv = h // 2
            k = np.concatenate([inp["k"][b, kv], inp["k_new"][b, kv]]).astype(np.float64)
            v = np.concatenate([inp["v"][b, kv], inp["v_new"][b, kv]]).astype(np.float64)
            ref = attention_fp64(inp["q"][b, h][None].astype(np.float64), k, v, 0.125)
            np.testing.assert_allclose(o[b, h], ref[0], rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------- outlier list

def test_outlier_rule_hand_worked():
    iso = oracle.zoned.isolate_outliers
    # mean of (0, 1, 2, 100) = 25.75: the largest (100) is farther -> slot 3;
    # then mean(0, 1, 2) = 1: both ends 1 away -> the largest (slot 2); then
    # two values remain -> stop
    assert iso(np.array([0, 1, 2, 100], np.float16), 1) == [3]
    assert iso(np.array([0, 1, 2, 100], np.float16), 2) == [2, 3]
    assert iso(np.array([0, 1, 2, 100], np.float16), 4) == [2, 3]
    # a low spike: mean(-50, 3, 4, 5) = -9.5: -50 is 40.5 away, 5 is 14.5
    assert iso(np.array([3, -50, 4, 5], np.float16), 1) == [1]
    # equal values at the maximum: mean(9, 2, 9, 3, 3, 3) = 29/6, the 9s are
    # 25/6 away, the 2 is 17/6 -> the first 9 (slot 0) goes
    assert iso(np.array([9, 2, 9, 3, 3, 3], np.float16), 1) == [0]
    # mean(7, 1, 7, 0) = 3.75: the 0 (3.75 away) beats the 7s (3.25)
    assert iso(np.array([7, 1, 7, 0], np.float16), 1) == [3]
    # constant groups and groups of two lose nothing
    assert iso(np.full(5, 3, np.float16), 3) == []
    assert iso(np.array([1, 9], np.float16), 1) == []


def test_outlier_taken_out_of_the_range():
    # a group with one spike: the other entries quantize exactly as the group
    # without the spike, and the spike comes back exactly
    rng = np.random.default_rng(23)
    x = rng.standard_normal(32).astype(np.float16)
    x[11] = np.float16(60.0)
    codes, sc, z, out = oracle.zoned._quantize_channel(x, 2, 1)
    assert out == [11]
    keep = np.arange(32) != 11
    c_ref, s_ref, z_ref = oracle.quantize_groups(x[keep][None], 2)
    assert np.array_equal(codes[keep], c_ref[0]) and codes[11] == 0
    assert sc == s_ref[0] and z == z_ref[0]
    # the step shrinks: every kept entry within half the new step
    xh = codes[keep] * np.float64(sc) + np.float64(z)
    assert np.abs(xh - x[keep].astype(np.float64)).max() <= np.float64(sc) / 2 * (1 + 1e-3) + 1e-6
    _, sc0, _, _ = oracle.zoned._quantize_channel(x, 2, 0)
    assert sc < sc0 / 5


def test_outlier_attention_and_layout():
    inp = _small(24, T=130, C=4, d=64)
    k = inp["k"].copy()
    # spikes at known places of kept tokens
    kept = np.flatnonzero(inp["v_bits"][0, 0] != 0)
    qch = np.flatnonzero((inp["k_bits"][0, 0] > 0) & (inp["k_bits"][0, 0] < 16))
    for i, t in enumerate(kept[:6]):
        k[0, 0, t, qch[i]] = np.float16(80.0 if i % 2 else -80.0)
    inp["k"] = k
    o1 = _zoned(inp, k_out=1)
    # against the definition: dequantize each group by hand
    d = 64
    lay = oracle.zoned._unit_layout(inp["v_bits"][0, 0], inp["k_bits"][0, 0], d, 4, 0, 1)
    kq = oracle.zoned._quantize_unit_keys(inp["k"][0, 0], lay)
    spikes = {(int(t), int(qch[i])) for i, t in enumerate(kept[:6])}
    found = set()
    qchan = np.concatenate([lay["classes"][w] for w in (2, 4, 8)])
    for w in (2, 4, 8, 16):
        for codes, scale, zero, raw, t, outl in kq[w]:
            for slot, pc, val in outl:
                found.add((int(t[slot]), int(qchan[pc])))
                assert val == inp["k"][0, 0, t[slot], qchan[pc]]
    assert spikes <= found
    # no group's step grows (a subset's range is never wider), and the step
    # of every spiked group shrinks by more than half
    lay0 = oracle.zoned._unit_layout(inp["v_bits"][0, 0], inp["k_bits"][0, 0], d, 4, 0, 0)
    kq0 = oracle.zoned._quantize_unit_keys(inp["k"][0, 0], lay0)
    pos = {int(c): i for i, c in enumerate(qchan)}
    for w in (2, 4, 8, 16):
        for g, (c1, s1, z1, r1, t1, outl) in enumerate(kq[w]):
            s0 = kq0[w][g][1]
            assert np.all(s1.astype(np.float64) <= s0.astype(np.float64))
            for tok, ch in spikes:
                if tok in set(t1.tolist()):
                    assert float(s1[pos[ch]]) < 0.5 * float(s0[pos[ch]])
    assert np.all(np.isfinite(o1))
    # the dequantized keys hold the spikes exactly
    kh, _ = oracle.zoned._dequant_unit(inp["k"][0, 0], inp["v"][0, 0], inp["v_bits"][0, 0],
                                       inp["k_bits"][0, 0], lay)
    toks = np.concatenate([lay["seg"][w]["tokens"] for w in (2, 4, 8, 16)])
    row = {int(t): i for i, t in enumerate(toks)}
    for tok, ch in spikes:
        assert kh[row[tok], ch] == float(inp["k"][0, 0, tok, ch])
    # byte image: the side list sits after the key zeros of every group
    blob = zoned_pack(inp["k"], inp["v"], inp["v_bits"], inp["k_bits"], inp["k_new"], inp["v_new"], k_out=1)
    units, total = zoned_layout(inp["v_bits"], inp["k_bits"], d, 4, 0, 1)
    assert blob.size == total
    sg = units[0]["seg"][2]
    go = units[0]["base"] + sg["offset"]
    o = go + units[0]["k_codes_bytes"] + 2 * units[0]["k_sz_bytes"]
    offs = blob[o:o + 66].view(np.uint16)
    n = int(offs[32])
    assert n == len(kq[2][0][5])
    assert np.all(np.diff(offs.astype(int)) >= 0)


def test_outlier_list_empty_is_the_plain_layout():
    # groups of at most two valid slots lose nothing: attention equals the
    # plain layout's exactly
    inp = _small(25, T=40, C=2)
    vb = np.zeros_like(inp["v_bits"])
    vb[:, :, [3, 17]] = 4                               # two kept tokens per unit
    inp["v_bits"] = vb
    np.testing.assert_array_equal(_zoned(inp, k_out=2), _zoned(inp))
