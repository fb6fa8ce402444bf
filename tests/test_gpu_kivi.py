"""GPU parity of the uniform-layout path against the oracle: quantize +
pack bit-exact, decode attention within relative L2 1e-3 of the oracle's
fp64 attention over its own dequantized cache."""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import say, dev, host, check_attention, oracle_cache, gpu_cache
from workloads import kivi_inputs, CONFIGS

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def dqa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dequant_decode_attention_amd as m
    return m


def _special_k(rng, B, H, T, d):
    """Keys with constant groups, outlier channels, tiny ranges, ties."""
    k = rng.standard_normal((B, H, T, d)).astype(np.float32)
    k[..., 5] *= 50.0
    k[:, :, :32, 7] = 3.25                       # constant key group
    if T >= 64:                                  # a group with few distinct levels
        k[:, :, 32:64, 9] = 1000.0 + rng.integers(0, 4, size=(B, H, 32)) * 0.5
    k[..., 11] *= 1e-3                           # tiny range
    k[:, :, :, 13] = np.round(k[:, :, :, 13] * 2) / 2   # values on half-integers
    return k.astype(np.float16)


SHAPES = [(1, 1, 256, 64, 2), (2, 3, 96, 128, 2), (2, 3, 96, 128, 4), (2, 3, 96, 128, 8),
          (1, 2, 64, 64, 4), (3, 1, 32, 128, 8), (1, 1, 0, 128, 2)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_quantize_pack_bit_exact(dqa, shape):
    B, H, T, d, bits = shape
    rng = np.random.default_rng(hash(shape) % 2 ** 32)
    k = _special_k(rng, B, H, T, d)
    v = k.transpose(0, 1, 2, 3).copy()
    v[..., :32] = rng.standard_normal((B, H, T, 32)).astype(np.float16)
    v[:, :, :3, 32:64] = -2.5                    # constant value groups
    say("quantize_pack_k/v", shape)
    gk = dqa.quantize_pack_k(dev(k), bits)
    gv = dqa.quantize_pack_v(dev(v), bits)
    torch.cuda.synchronize()
    kc, ks, kz = oracle.quantize_k(k, bits)
    vc, vs, vz = oracle.quantize_v(v, bits)
    np.testing.assert_array_equal(host(gk[0]).view(np.uint32), oracle.pack_codes(kc, bits))
    np.testing.assert_array_equal(host(gk[1]).view(np.uint16), ks.view(np.uint16))
    np.testing.assert_array_equal(host(gk[2]).view(np.uint16), kz.view(np.uint16))
    np.testing.assert_array_equal(host(gv[0]).view(np.uint32), oracle.pack_v_codes(vc, bits).reshape(host(gv[0]).shape))
    np.testing.assert_array_equal(host(gv[1]).view(np.uint16), vs.view(np.uint16))
    np.testing.assert_array_equal(host(gv[2]).view(np.uint16), vz.view(np.uint16))


def _tie_group(rng, bits):
    """32 fp16 values whose quotients (x - min) / scale sit exactly on
    half-integers (ties, rounded half to even) or one fp16 step away from
    them, with min 0 and max 2^bits - 1 so that the scale is exactly 1."""
    L = (1 << bits) - 1
    k = rng.integers(0, L, size=30)
    step = np.float16(np.spacing(np.float16(L)))          # fp16 step at the top of the range
    off = rng.choice(np.array([0.0, -1.0, 1.0]), size=30) * np.maximum(step, 2.0 ** -10)
    vals = np.concatenate([[0.0, float(L)], k + 0.5 + off]).astype(np.float16)
    return vals[rng.permutation(32)]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_quantize_rounding_ties(dqa, bits, d):
    """Quotients on and next to the rounding boundaries: the codes must be
    those of the IEEE division rounded half to even (the kernels take a
    reciprocal product and fall back to the division near a boundary)."""
    rng = np.random.default_rng(1000 * bits + d)
    T = 64
    k = np.empty((2, 1, T, d), np.float16)
    for b in range(2):
        for t0 in range(0, T, 32):
            for c in range(d):
                k[b, 0, t0:t0 + 32, c] = _tie_group(rng, bits)
    v = np.empty((2, 1, T, d), np.float16)
    for b in range(2):
        for t in range(T):
            for g in range(d // 32):
                v[b, 0, t, 32 * g:32 * g + 32] = _tie_group(rng, bits)
    say("quantize ties", bits, d)
    gk = dqa.quantize_pack_k(dev(k), bits)
    gv = dqa.quantize_pack_v(dev(v), bits)
    torch.cuda.synchronize()
    kc, ks, kz = oracle.quantize_k(k, bits)
    vc, vs, vz = oracle.quantize_v(v, bits)
    assert np.all(ks.astype(np.float32) == 1.0) and np.all(vs.astype(np.float32) == 1.0)
    np.testing.assert_array_equal(host(gk[0]).view(np.uint32), oracle.pack_codes(kc, bits))
    np.testing.assert_array_equal(host(gv[0]).view(np.uint32), oracle.pack_v_codes(vc, bits).reshape(host(gv[0]).shape))
    np.testing.assert_array_equal(host(gk[1]).view(np.uint16), ks.view(np.uint16))
    np.testing.assert_array_equal(host(gv[2]).view(np.uint16), vz.view(np.uint16))


@pytest.mark.parametrize("name", ["llama2-13b-decode-layer", "llama3.1-8b-gqa-32k"])
def test_quantize_full_config_sampled_units(dqa, name):
    """Full-size quantization on the GPU; the oracle re-quantizes sampled
    (batch, KV head) units and compares them bit for bit."""
    cfg = CONFIGS[name]
    inp = kivi_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T_q"], 0,
                      seed=cfg["seed"], outliers=cfg["outliers"])
    for bits in cfg["bits"]:
        say("quantize full", name, bits)
        gk = dqa.quantize_pack_k(dev(inp["k"]), bits)
        gv = dqa.quantize_pack_v(dev(inp["v"]), bits)
        torch.cuda.synchronize()
        rng = np.random.default_rng(0)
        for _ in range(3):
            b, h = int(rng.integers(cfg["B"])), int(rng.integers(cfg["Hkv"]))
            kc, ks, kz = oracle.quantize_k(inp["k"][b:b + 1, h:h + 1], bits)
            vc, vs, vz = oracle.quantize_v(inp["v"][b:b + 1, h:h + 1], bits)
            np.testing.assert_array_equal(host(gk[0][b, h]).view(np.uint32), oracle.pack_codes(kc, bits)[0, 0])
            np.testing.assert_array_equal(host(gk[1][b, h]).view(np.uint16), ks[0, 0].view(np.uint16))
            np.testing.assert_array_equal(host(gk[2][b, h]).view(np.uint16), kz[0, 0].view(np.uint16))
            np.testing.assert_array_equal(host(gv[0][b, h]).view(np.uint32), oracle.pack_v_codes(vc, bits)[0, 0].reshape(host(gv[0][b, h]).shape))
            np.testing.assert_array_equal(host(gv[1][b, h]).view(np.uint16), vs[0, 0].view(np.uint16))
            np.testing.assert_array_equal(host(gv[2][b, h]).view(np.uint16), vz[0, 0].view(np.uint16))


DECODE_CASES = [
    # B, Hq, Hkv, d, T_q, R, bits, rope
    (1, 1, 1, 64, 256, 0, 2, 0.0),          # tiny-kivi shape
    (2, 8, 2, 128, 320, 37, 2, 500000.0),   # GQA 4, ragged recent zone, RoPE
    (2, 8, 2, 128, 320, 37, 4, 500000.0),
    (1, 4, 4, 128, 128, 128, 8, 10000.0),   # MHA, full recent zone
    (2, 4, 2, 64, 96, 5, 2, 500000.0),      # d 64, G 2
    (1, 4, 1, 64, 64, 0, 4, 0.0),           # d 64, G 4
    (3, 2, 2, 128, 32, 1, 2, 0.0),          # single tile + one recent token
    (1, 4, 1, 128, 0, 100, 2, 500000.0),    # only recent tokens
    (1, 4, 1, 128, 4096, 0, 2, 500000.0),   # many tiles -> many splits
    (2, 2, 1, 128, 0, 0, 2, 0.0),           # empty cache -> zeros
    (1, 4, 1, 128, 32768, 128, 2, 500000.0),  # one unit: split cap, recent tiles in 4 waves
    (2, 4, 1, 64, 192, 70, 8, 10000.0),     # d 64, 8 bits, RoPE, 3 ragged recent tiles
    (1, 4, 2, 128, 640, 31, 4, 0.0),        # G 2, 4 bits, no RoPE, ragged recent zone
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_attention_parity(dqa, case):
    B, Hq, Hkv, d, T_q, R, bits, rope = case
    inp = kivi_inputs(B, Hq, Hkv, d, T_q, R, seed=T_q + R + d,
                      outliers=("lognormal", 0.04, 3.0, 1.0))
    scale = 1.0 / math.sqrt(d)
    ref = oracle.kivi_decode_attention(inp["q"], oracle_cache(inp, bits, Hq, rope), scale)
    say("decode_attention_qkv", case)
    cache = gpu_cache(dqa, inp, bits, Hq, rope)
    out = dqa.decode_attention_qkv(dev(inp["q"]), cache, scale)
    torch.cuda.synchronize()
    got = host(out)
    if T_q + R == 0:
        assert np.all(got == 0)
        return
    check_attention(got, ref, TOL, str(case))
    # a second call reuses the workspace (its counters were reset) and is
    # bit-identical: the split merge runs in a fixed order
    out2 = dqa.decode_attention_qkv(dev(inp["q"]), cache, scale)
    torch.cuda.synchronize()
    assert np.array_equal(host(out2), got)


@pytest.mark.parametrize("bits,d", [(2, 128), (4, 128), (2, 64), (4, 64)])
def test_rope_table_copy_equals_in_kernel_build(dqa, bits, d):
    """A cache's built in-tile rotation table (kivi_rope_table) gives outputs
    bit-identical to the kernel's own evaluation of the rotations (same
    arithmetic), and a table built for another theta, or another code width,
    is ignored (its header does not match)."""
    B, Hq, Hkv, T_q, R, rope = 2, 8, 2, 320, 37, 500000.0
    inp = kivi_inputs(B, Hq, Hkv, d, T_q, R, seed=T_q + R + d, outliers=("lognormal", 0.04, 3.0, 1.0))
    scale = 1.0 / math.sqrt(d)
    say("rope table", bits, d)
    with_table = gpu_cache(dqa, inp, bits, Hq, rope)
    assert with_table.rope_table is not None
    built = gpu_cache(dqa, inp, bits, Hq, rope, rope_table=False)
    assert built.rope_table is None
    q = dev(inp["q"])
    a = host(dqa.decode_attention_qkv(q, with_table, scale))
    b = host(dqa.decode_attention_qkv(q, built, scale))
    assert np.array_equal(a, b)
    ref = oracle.kivi_decode_attention(inp["q"], oracle_cache(inp, bits, Hq, rope), scale)
    check_attention(a, ref, TOL, f"rope table {bits} {d}")
    # the kernel reads the table it is given: contents altered behind a
    # valid header change the output
    altered = with_table.rope_table.clone()
    altered[4:] = 0
    with_table.rope_table = altered
    assert not np.array_equal(host(dqa.decode_attention_qkv(q, with_table, scale)), b)
    for other in (dqa.kivi_rope_table(1e4, d, bits, q.device), dqa.kivi_rope_table(rope, d, 6 - bits, q.device)):
        with_table.rope_table = other
        c = host(dqa.decode_attention_qkv(q, with_table, scale))
        assert np.array_equal(c, b)


@pytest.mark.parametrize("T_q,R", [(4096, 77), (64, 5)])
def test_decode_two_phase_equals_one_call(dqa, T_q, R):
    """decode_attention_qkv is exactly _partial then _merge (bit-identical),
    with many splits and with a single split."""
    B, Hq, Hkv, d, bits = 2, 8, 2, 128, 4
    inp = kivi_inputs(B, Hq, Hkv, d, T_q, R, seed=7, outliers=("lognormal", 0.04, 3.0, 1.0))
    say("decode two-phase", T_q, R)
    cache = gpu_cache(dqa, inp, bits, Hq, 500000.0)
    q = dev(inp["q"])
    ref = host(dqa.decode_attention_qkv(q, cache, 0.088))
    ws = cache.workspace(q.device)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=q.device)
    dqa.decode_attention_qkv_partial(q, cache, 0.088, out, ws)
    dqa.decode_attention_qkv_merge(cache, out, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), ref)


def test_merge_counters_reset_and_shared_workspace(dqa):
    """The workgroup that finishes a (batch, KV head) last merges its splits
    and sets the unit's counter back to zero: after every call the counter
    area is zero again, and one workspace serves caches of different shapes
    (different unit counts and split counts) in turn."""
    cases = [(2, 8, 2, 128, 4096, 40, 2, 500000.0), (1, 4, 1, 128, 8192, 0, 4, 10000.0),
             (3, 8, 4, 64, 2048, 100, 2, 0.0), (2, 8, 2, 128, 4096, 40, 2, 500000.0)]
    caches = []
    for case in cases:
        B, Hq, Hkv, d, T_q, R, bits, rope = case
        inp = kivi_inputs(B, Hq, Hkv, d, T_q, R, seed=T_q + R, outliers=("lognormal", 0.04, 3.0, 1.0))
        caches.append((case, inp, gpu_cache(dqa, inp, bits, Hq, rope)))
    n = max(c.workspace_bytes() for _, _, c in caches)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda:0")
    for case, inp, cache in caches:
        B, Hq, Hkv, d, T_q, R, bits, rope = case
        say("decode on a shared workspace", case)
        scale = 1.0 / math.sqrt(d)
        out = host(dqa.decode_attention_qkv(dev(inp["q"]), cache, scale, workspace=ws))
        counters = host(ws[:16384 * 4]).view(np.uint32)
        assert not counters.any(), np.nonzero(counters)
        ref = oracle.kivi_decode_attention(inp["q"], oracle_cache(inp, bits, Hq, rope), scale)
        check_attention(out, ref, TOL, f"shared workspace {case}")


@pytest.mark.parametrize("name,bits", [("llama3.1-8b-gqa-32k", 2), ("llama3.1-8b-gqa-32k", 4), ("llama2-13b-decode-layer", 2), ("tiny-kivi", 2)])
def test_decode_full_config_every_unit(dqa, name, bits):
    """Full-size decode in the launch configuration the bench times; the
    oracle computes every (batch, KV head) unit's output rows, one unit at a
    time."""
    cfg = CONFIGS[name]
    inp = kivi_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T_q"], cfg["R"],
                      seed=cfg["seed"], outliers=cfg["outliers"])
    scale = 1.0 / math.sqrt(cfg["d"])
    say("decode full", name, bits)
    cache = gpu_cache(dqa, inp, bits, cfg["Hq"], cfg["rope_theta"])
    out = host(dqa.decode_attention_qkv(dev(inp["q"]), cache, scale))
    units = [(b, u) for b in range(cfg["B"]) for u in range(cfg["Hkv"])]
    for b, u in units:
        sub = {k: v[b:b + 1, u:u + 1] for k, v in inp.items() if k != "q"}
        G = cfg["Hq"] // cfg["Hkv"]
        sub["q"] = inp["q"][b:b + 1, u * G:(u + 1) * G]
        ref = oracle.kivi_decode_attention(sub["q"], oracle_cache(sub, bits, G, cfg["rope_theta"]), scale)
        got = out[b, u * G:(u + 1) * G][None]
        check_attention(got, ref, TOL, f"{name} bits={bits} unit=({b},{u})")
