"""Pins of the oracle attention, RoPE and KIVI-cache reader ([P1 para 2, 6,
7, 8]; [P1] = ihal.it/?p=61653).  CPU only."""
import numpy as np
import pytest
import torch

import oracle
from oracle import attention_fp64, rope_rotate, kivi_decode_attention
from workloads import kivi_inputs


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_matches_library_sdpa():
    rng = np.random.default_rng(0)
    q, k, v = _rand(rng, 4, 64), _rand(rng, 300, 64) * 3, _rand(rng, 300, 64)
    scale = 1 / 8.0
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(k)[None, None].expand(1, 4, 300, 64),
        torch.from_numpy(v)[None, None].expand(1, 4, 300, 64), scale=scale)[0, :, 0, :].numpy()
    np.testing.assert_allclose(attention_fp64(q, k, v, scale), ref, rtol=1e-12, atol=1e-12)


def test_special_cases():
    rng = np.random.default_rng(1)
    v = _rand(rng, 1, 32)
    # one key: the output is that value
    np.testing.assert_allclose(attention_fp64(_rand(rng, 3, 32), _rand(rng, 1, 32), v, 0.5),
                               np.repeat(v, 3, 0), rtol=1e-14)
    # zero query: uniform weights -> mean of the values
    k, v = _rand(rng, 50, 32), _rand(rng, 50, 32)
    np.testing.assert_allclose(attention_fp64(np.zeros((2, 32)), k, v, 0.3),
                               np.repeat(v.mean(0, keepdims=True), 2, 0), rtol=1e-12)
    # identical tokens: the output is the shared value
    kk = np.repeat(_rand(rng, 1, 32), 40, 0)
    vv = np.repeat(_rand(rng, 1, 32), 40, 0)
    np.testing.assert_allclose(attention_fp64(_rand(rng, 2, 32), kk, vv, 1.0),
                               vv[:2], rtol=1e-12)
    # no keys: zeros
    assert np.all(attention_fp64(_rand(rng, 2, 32), np.zeros((0, 32)), np.zeros((0, 32)), 1.0) == 0)


def test_permutation_invariance_and_split_merge():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 3, 64), _rand(rng, 257, 64) * 2, _rand(rng, 257, 64)
    o = attention_fp64(q, k, v, 0.125)
    perm = rng.permutation(257)
    np.testing.assert_allclose(attention_fp64(q, k[perm], v[perm], 0.125), o, rtol=1e-12)
    # splitting the keys and merging partial softmax states (log-sum-exp)
    # gives the single-pass result
    parts = np.array_split(np.arange(257), 5)
    ms, ls, os_ = [], [], []
    for idx in parts:
        lg = 0.125 * q @ k[idx].T
        m = lg.max(1, keepdims=True)
        p = np.exp(lg - m)
        ms.append(m), ls.append(p.sum(1, keepdims=True)), os_.append(p @ v[idx])
    M = np.max(np.concatenate(ms, 1), 1, keepdims=True)
    L = sum(l * np.exp(m - M) for m, l in zip(ms, ls))
    O = sum(oo * np.exp(m - M) for m, oo in zip(ms, os_))
    np.testing.assert_allclose(O / L, o, rtol=1e-12)


def test_gqa_head_mapping():
    rng = np.random.default_rng(3)
    inp = kivi_inputs(1, 4, 2, 64, 64, 0, seed=3)
    cache = _cache_from(inp, 4, rope=0.0, Hq=4)
    o = kivi_decode_attention(inp["q"], cache, 0.125)
    # head h reads KV head h // 2: rebuild as MHA with KV heads repeated
    rep = {k: (np.repeat(v, 2, axis=1) if k in ("k", "v", "k_recent", "v_recent") else v)
           for k, v in inp.items()}
    cache_mha = _cache_from(rep, 4, rope=0.0, Hq=4)
    o_mha = kivi_decode_attention(inp["q"], cache_mha, 0.125)
    np.testing.assert_allclose(o, o_mha, rtol=1e-11, atol=1e-13)


def test_rope_properties():
    rng = np.random.default_rng(4)
    d, theta = 64, 500000.0
    x = _rand(rng, 10, d)
    # position 0 is the identity
    np.testing.assert_allclose(rope_rotate(x, np.zeros(10), theta), x, rtol=0, atol=0)
    pos = rng.integers(0, 40000, size=10)
    y = rope_rotate(x, pos, theta)
    # rotations preserve each pair's norm
    np.testing.assert_allclose(np.hypot(y[:, 0::2], y[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]), rtol=1e-12)
    # the score of a rotated query/key pair depends only on the offset
    a, b = _rand(rng, 1, d), _rand(rng, 1, d)
    s1 = rope_rotate(a, [100], theta) @ rope_rotate(b, [130], theta).T
    s2 = rope_rotate(a, [5000], theta) @ rope_rotate(b, [5030], theta).T
    np.testing.assert_allclose(s1, s2, rtol=1e-9)
    # complex-number formulation: pair (a, b) as a + ib times exp(i pos w)
    w = theta ** (-2.0 * np.arange(d // 2) / d)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * pos[:, None] * w[None, :])
    np.testing.assert_allclose(y[:, 0::2], z.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[:, 1::2], z.imag, rtol=1e-12, atol=1e-12)
    # first pair has frequency 1 (theta^0): angle equals the position
    np.testing.assert_allclose(rope_rotate(np.array([[1.0, 0.0] + [0.0] * (d - 2)]), [2.0], theta)[0, :2],
                               [np.cos(2.0), np.sin(2.0)], rtol=1e-14)


def _cache_from(inp, bits, rope, Hq=None):
    B, Hkv, T_q, d = inp["k"].shape
    R = inp["k_recent"].shape[2]
    kc, ks, kz = oracle.quantize_k(inp["k"], bits)
    vc, vs, vz = oracle.quantize_v(inp["v"], bits)
    return dict(B=B, Hq=Hq or inp["q"].shape[1], Hkv=Hkv, d=d, bits=bits, T_q=T_q,
                R=R, rope_theta=rope, k_codes=oracle.pack_codes(kc, bits),
                v_codes=oracle.pack_v_codes(vc, bits), k_scale=ks, k_zero=kz,
                v_scale=vs, v_zero=vz, k_recent=inp["k_recent"], v_recent=inp["v_recent"])


def test_fp16_only_cache_is_plain_attention():
    # T_q = 0, every token in the fp16 recent zone: plain attention over the
    # fp16 values (the unquantized reference)
    inp = kivi_inputs(2, 4, 2, 64, 0, 96, seed=5)
    cache = _cache_from(inp, 2, rope=0.0)
    o = kivi_decode_attention(inp["q"], cache, 0.125)
    for b in range(2):
        for h in range(4):
            ref = attention_fp64(inp["q"][b, h][None].astype(np.float64),
                                 inp["k_recent"][b, h // 2].astype(np.float64),
                                 inp["v_recent"][b, h // 2].astype(np.float64), 0.125)
            np.testing.assert_allclose(o[b, h], ref[0], rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("rope", [0.0, 500000.0])
def test_packed_reader_equals_dequantized_tensors(rope):
    inp = kivi_inputs(1, 4, 2, 64, 128, 32, seed=6, outliers=("fixed", (5, 37), 50.0))
    cache = _cache_from(inp, 2, rope=rope)
    o = kivi_decode_attention(inp["q"], cache, 0.125)
    kc, ks, kz = oracle.quantize_k(inp["k"], 2)
    vc, vs, vz = oracle.quantize_v(inp["v"], 2)
    K = np.concatenate([oracle.dequantize_k(kc, ks, kz), inp["k_recent"].astype(np.float64)], 2)
    V = np.concatenate([oracle.dequantize_v(vc, vs, vz), inp["v_recent"].astype(np.float64)], 2)
    for h in range(4):
        k = K[0, h // 2]
        if rope:
            k = rope_rotate(k, np.arange(160), rope)
        ref = attention_fp64(inp["q"][0, h][None].astype(np.float64), k, V[0, h // 2], 0.125)
        np.testing.assert_allclose(o[0, h], ref[0], rtol=1e-11, atol=1e-13)
    # rows= computes only the requested rows
    o2 = kivi_decode_attention(inp["q"], cache, 0.125, rows=[(0, 3)])
    np.testing.assert_allclose(o2[0, 3], o[0, 3], rtol=1e-12, atol=1e-14)
    assert np.isnan(o2[0, 0]).all()


def test_directional_claim_keys_per_channel_lower_error():
    # [P1 para 4]: with outlier channels, per-channel key grouping
    # reconstructs keys better than per-token grouping (directional check on
    # synthetic data, not a reproduction of the page's numbers)
    inp = kivi_inputs(1, 1, 4, 128, 1024, 0, seed=7, outliers=("lognormal", 0.04, 3.0, 1.0))
    k = inp["k"]
    kc, ks, kz = oracle.quantize_k(k, 2)
    e_ch = np.abs(oracle.dequantize_k(kc, ks, kz) - k.astype(np.float64)).mean()
    tc, ts, tz = oracle.quantize_v(k, 2)
    e_tok = np.abs(oracle.dequantize_v(tc, ts, tz) - k.astype(np.float64)).mean()
    assert e_ch < e_tok
