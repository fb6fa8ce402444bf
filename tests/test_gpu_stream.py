"""GPU parity of the streaming append (kivi_append) and of decode over a
cache whose buffers have spare capacity: the library's quantized zone and
fp16 window equal the oracle's streamed state bit for bit, and attention
over the streamed cache matches the oracle's fp64 attention."""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import dev, host, check_attention, say

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def dqa():
    import dequant_decode_attention_amd as m
    return m


def _tokens(B, H, T, d, seed):
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((B, H, T, d)) * rng.lognormal(0, 1, (1, H, 1, d))).astype(np.float16)
    v = rng.standard_normal((B, H, T, d)).astype(np.float16)
    return k, v


def _empty_gpu_cache(dqa, B, Hq, Hkv, d, bits, T_cap, R_cap, rope):
    z = lambda *s, dt=torch.float16: torch.zeros(s, dtype=dt, device="cuda:0")
    return dqa.KiviCache(Hq, bits, z(B, Hkv, T_cap, d * bits // 32, dt=torch.int32), z(B, Hkv, T_cap // 32, d),
                         z(B, Hkv, T_cap // 32, d), z(B, Hkv, T_cap, d * bits // 32, dt=torch.int32),
                         z(B, Hkv, T_cap, d // 32), z(B, Hkv, T_cap, d // 32), z(B, Hkv, R_cap, d),
                         z(B, Hkv, R_cap, d), rope_theta=rope, T_q=0, R=0)


def _check_state(cache, st, bits):
    T_q, R = st["k_codes"].shape[2], st["k_recent"].shape[2]
    assert (cache.T_q, cache.R) == (T_q, R)
    t = cache.tensors
    B, H = st["k_codes"].shape[:2]
    got = {n: host(t[n]) for n in t}
    assert np.array_equal(got["k_codes"][:, :, :T_q].view(np.uint32), oracle.pack_codes(st["k_codes"], bits))
    assert np.array_equal(got["k_scale"][:, :, :T_q // 32], st["k_scale"])
    assert np.array_equal(got["k_zero"][:, :, :T_q // 32], st["k_zero"])
    vw = oracle.pack_v_codes(st["v_codes"], bits)
    assert np.array_equal(got["v_codes"][:, :, :T_q].view(np.uint32).reshape(vw.shape), vw)
    assert np.array_equal(got["v_scale"][:, :, :T_q], st["v_scale"])
    assert np.array_equal(got["v_zero"][:, :, :T_q], st["v_zero"])
    assert np.array_equal(got["k_recent"][:, :, :R], st["k_recent"])
    assert np.array_equal(got["v_recent"][:, :, :R], st["v_recent"])


def _oracle_cache(st, Hq, bits, rope):
    B, H, T_q, d = st["k_codes"].shape
    return dict(B=B, Hq=Hq, Hkv=H, d=d, bits=bits, T_q=T_q, R=st["k_recent"].shape[2], rope_theta=rope,
                k_codes=oracle.pack_codes(st["k_codes"], bits), v_codes=oracle.pack_v_codes(st["v_codes"], bits),
                k_scale=st["k_scale"], k_zero=st["k_zero"], v_scale=st["v_scale"], v_zero=st["v_zero"],
                k_recent=st["k_recent"], v_recent=st["v_recent"])


CASES = [
    # B, Hq, Hkv, d, bits, R_max, T, chunk pattern, rope
    (2, 8, 2, 128, 2, 128, 300, (1, 7, 33, 64, 5, 40), 5e5),
    (1, 4, 1, 64, 4, 64, 260, (32, 1, 100, 3), 1e4),
    (2, 4, 2, 128, 8, 0, 150, (17, 31, 50), 0.0),
    (1, 4, 4, 128, 2, 31, 200, (9,), 1e4),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}x{c[3]}-b{c[4]}-Rmax{c[5]}-T{c[6]}")
def test_append_matches_oracle_stream_and_decodes(dqa, case):
    B, Hq, Hkv, d, bits, R_max, T, pattern, rope = case
    say("kivi_append", case[:7])
    k, v = _tokens(B, Hkv, T, d, seed=T + bits)
    T_cap = ((T + 31) // 32 + 1) * 32
    cache = _empty_gpu_cache(dqa, B, Hq, Hkv, d, bits, T_cap, 160, rope)
    st = oracle.empty_stream(B, Hkv, d)
    t, i, flushed = 0, 0, 0
    while t < T:
        n = min(pattern[i % len(pattern)], T - t)
        i += 1
        flushed += dqa.kivi_append(cache, dev(k[:, :, t:t + n]), dev(v[:, :, t:t + n]), R_max)
        st = oracle.kivi_append(st, k[:, :, t:t + n], v[:, :, t:t + n], bits, R_max)
        t += n
        if i % 3 == 0 or t == T:
            torch.cuda.synchronize()
            _check_state(cache, st, bits)
    assert flushed * 32 == cache.T_q
    # decode over the streamed cache (buffers with spare capacity)
    rng = np.random.default_rng(T)
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    scale = 1.0 / math.sqrt(d)
    got = host(dqa.decode_attention_qkv(dev(q), cache, scale))
    ref = oracle.kivi_decode_attention(q, _oracle_cache(st, Hq, bits, rope), scale)
    check_attention(got, ref, TOL, f"T_q={cache.T_q} R={cache.R}")


def test_append_one_token_per_step_flush_points(dqa):
    """One token per step with R_max = 128: the library flushes exactly where
    the oracle does, and the window rows move in place."""
    B, Hq, Hkv, d, bits = 1, 2, 2, 64, 2
    say("kivi_append one token per step")
    k, v = _tokens(B, Hkv, 200, d, seed=11)
    cache = _empty_gpu_cache(dqa, B, Hq, Hkv, d, bits, 128, 128, 0.0)
    st = oracle.empty_stream(B, Hkv, d)
    for t in range(200):
        dqa.kivi_append(cache, dev(k[:, :, t:t + 1]), dev(v[:, :, t:t + 1]), 128)
        st = oracle.kivi_append(st, k[:, :, t:t + 1], v[:, :, t:t + 1], bits, 128)
        assert (cache.T_q, cache.R) == (st["k_codes"].shape[2], st["k_recent"].shape[2])
        if t in (127, 128, 129, 160, 199):
            torch.cuda.synchronize()
            _check_state(cache, st, bits)


def test_append_full_config_flush(dqa):
    """Llama-3.1-8B shape (batch 4, 8 KV heads, d 128, 2 bits): a full window
    of 128 tokens plus one new token flushes one group per (batch, KV head)
    into a cache that already holds 32736 quantized tokens; the new group and
    the window equal the oracle's quantization of the same tokens."""
    B, Hq, Hkv, d, bits = 4, 32, 8, 128, 2
    say("kivi_append llama3.1-8b-gqa-32k flush")
    T_q0 = 32768 - 32
    cache = _empty_gpu_cache(dqa, B, Hq, Hkv, d, bits, 32768, 128, 5e5)
    k, v = _tokens(B, Hkv, 129, d, seed=13)
    cache.T_q = T_q0
    cache.tensors["k_recent"].copy_(dev(k[:, :, :128]))
    cache.tensors["v_recent"].copy_(dev(v[:, :, :128]))
    cache.R = 128
    assert dqa.kivi_append(cache, dev(k[:, :, 128:]), dev(v[:, :, 128:]), 128) == 1
    torch.cuda.synchronize()
    assert (cache.T_q, cache.R) == (32768, 97)
    kc, ks, kz = oracle.quantize_k(k[:, :, :32], bits)
    vc, vs, vz = oracle.quantize_v(v[:, :, :32], bits)
    t = {n: host(x) for n, x in cache.tensors.items()}
    assert np.array_equal(t["k_codes"][:, :, T_q0:].view(np.uint32), oracle.pack_codes(kc, bits))
    assert np.array_equal(t["k_scale"][:, :, T_q0 // 32:], ks) and np.array_equal(t["k_zero"][:, :, T_q0 // 32:], kz)
    vw = oracle.pack_v_codes(vc, bits)
    assert np.array_equal(t["v_codes"][:, :, T_q0:].view(np.uint32).reshape(vw.shape), vw)
    assert np.array_equal(t["v_scale"][:, :, T_q0:], vs) and np.array_equal(t["v_zero"][:, :, T_q0:], vz)
    assert np.array_equal(t["k_recent"][:, :, :97], k[:, :, 32:129])
    assert np.array_equal(t["v_recent"][:, :, :97], v[:, :, 32:129])
    # nothing before the new group was touched
    assert not t["k_codes"][:, :, :T_q0].any() and not t["k_scale"][:, :, :T_q0 // 32].any()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_append_in_window_flush_every_width(dqa, bits, d):
    """One token per step into a 32-row window: every flush quantizes the
    window's oldest group in place and moves the rest of the window (the
    in-window flush path), for each width and head dim; state bit-exact with
    the oracle's stream after each flush and at the end."""
    B, Hq, Hkv, T = 2, 4, 2, 120
    say("kivi_append in-window flush", bits, d)
    k, v = _tokens(B, Hkv, T, d, seed=100 + bits + d)
    cache = _empty_gpu_cache(dqa, B, Hq, Hkv, d, bits, 128, 64, 0.0)
    st = oracle.empty_stream(B, Hkv, d)
    flushes = 0
    for t in range(T):
        f = dqa.kivi_append(cache, dev(k[:, :, t:t + 1]), dev(v[:, :, t:t + 1]), 32)
        st = oracle.kivi_append(st, k[:, :, t:t + 1], v[:, :, t:t + 1], bits, 32)
        flushes += f
        if f or t == T - 1:
            torch.cuda.synchronize()
            _check_state(cache, st, bits)
    assert flushes == 3 and (cache.T_q, cache.R) == (96, 24)


def test_append_capacity_zero_keeps_row_stride(dqa):
    """A direct C caller passes R_cap = 0 (the recent buffers hold exactly R
    rows) and T_cap = the quantized capacity: a flush that shrinks R must
    leave the rows of every (batch, KV head) at the old stride, so that the
    next decode (and append) reads them where they are.  Four units, so a
    wrong stride would misplace the rows of all but the first."""
    import ctypes
    B, Hq, Hkv, d, bits = 2, 4, 2, 64, 2
    say("kivi_append R_cap = 0 through the C ABI")
    k, v = _tokens(B, Hkv, 161, d, seed=21)
    cache = _empty_gpu_cache(dqa, B, Hq, Hkv, d, bits, 64, 128, 1e4)
    st = oracle.empty_stream(B, Hkv, d)
    # 160 tokens with R_max = 128: one group quantized, the window full
    dqa.kivi_append(cache, dev(k[:, :, :160]), dev(v[:, :, :160]), 128)
    st = oracle.kivi_append(st, k[:, :, :160], v[:, :, :160], bits, 128)
    assert (cache.T_q, cache.R) == (32, 128)
    c = cache.struct()
    c.R_cap = 0                                  # "R rows", i.e. 128
    kn, vn = dev(k[:, :, 160:]), dev(v[:, :, 160:])
    n = dqa.lib.kivi_append_workspace_bytes(ctypes.byref(c), 1)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    assert dqa.lib.kivi_append(ctypes.byref(c), dqa._ptr(kn), dqa._ptr(vn), 1, 128, dqa._ptr(ws), n,
                               dqa._stream(kn.device)) == 0
    st = oracle.kivi_append(st, k[:, :, 160:], v[:, :, 160:], bits, 128)
    assert (c.T_q, c.R, c.T_cap, c.R_cap) == (64, 97, 64, 128)
    cache.T_q, cache.R = c.T_q, c.R
    torch.cuda.synchronize()
    _check_state(cache, st, bits)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    scale = 1.0 / math.sqrt(d)
    # decode through the same descriptor the append updated
    qd = dev(q)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda:0")
    nws = dqa.lib.decode_attention_workspace_bytes(ctypes.byref(c))
    dws = torch.zeros(nws, dtype=torch.uint8, device="cuda:0")
    assert dqa.lib.decode_attention_qkv(dqa._ptr(qd), ctypes.byref(c), ctypes.c_float(scale), dqa._ptr(dws),
                                        nws, dqa._ptr(out), dqa._stream(qd.device)) == 0
    torch.cuda.synchronize()
    ref = oracle.kivi_decode_attention(q, _oracle_cache(st, Hq, bits, 1e4), scale)
    check_attention(host(out), ref, TOL, "after the R_cap = 0 flush")
