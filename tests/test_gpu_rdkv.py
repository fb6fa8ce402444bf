"""GPU parity of the RDKV allocator.

* Token and channel weights against the oracle's fp64 values, elementwise
  within a relative 2e-4: the GPU computes fp32 logits from exact fp16
  products (fp32 accumulation over d <= 128 terms), exponentials to about
  one ulp, and fp32 sums over at most G*T terms; all terms are positive, so
  the relative error of a sum stays below the largest relative error of its
  terms plus the accumulation error (about 1e-5 at the sizes here).
* Widths: the allocation is an integer decision taken from the weights.
  Given the same float32 weights, the GPU and the oracle must agree exactly
  (both compare exact float64 breakpoints).  From their own weights they may
  differ only on units whose breakpoint lies within the weight tolerance of
  the critical multiplier.
* At the full mixed-width cache size (16k tokens, 32 query heads): every
  query row's attention sums to 1, so each KV head's token weights sum to
  G*T; the last 16 tokens' weights need only the last 16 query rows and are
  checked against the oracle directly; the allocation is exact on the GPU's
  own weights.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import say, dev, host, check_attention
from workloads import rdkv_inputs, zoned_inputs, CONFIGS

pytestmark = pytest.mark.gpu
WTOL = 2e-4
OUTL = ("lognormal", 0.04, 3.0, 1.0)


@pytest.fixture(scope="module")
def dqa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dequant_decode_attention_amd as m
    return m


def _rel(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float((np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)).max())


TOKEN_CASES = [
    # B, Hq, Hkv, T, d
    (1, 1, 1, 1, 64),
    (1, 4, 2, 37, 64),
    (1, 2, 1, 129, 128),
    (1, 3, 1, 200, 128),
    (2, 8, 2, 300, 128),
    (1, 8, 2, 1000, 128),
    (1, 4, 4, 640, 64),
    (1, 3, 3, 64, 128),      # one key tile exactly, head ratio 1
    (2, 6, 3, 128, 128),     # one query tile exactly, 6 units
    (1, 4, 1, 129, 64),      # one row past a tile
    (3, 12, 3, 257, 128),    # 9 units, ragged
]


@pytest.mark.parametrize("case", TOKEN_CASES, ids=lambda c: "x".join(map(str, c)))
def test_token_weights(dqa, case):
    B, Hq, Hkv, T, d = case
    inp = rdkv_inputs(B, Hq, Hkv, d, T, seed=T + Hq, outliers=OUTL)
    scale = d ** -0.5
    say("rdkv_token_weights", case)
    got = host(dqa.rdkv_token_weights(dev(inp["q"]), dev(inp["k"]), scale))
    torch.cuda.synchronize()
    ref = oracle.token_weights(inp["q"], inp["k"], scale)
    err = _rel(got, ref)
    say("  max rel", err)
    assert err <= WTOL
    again = host(dqa.rdkv_token_weights(dev(inp["q"]), dev(inp["k"]), scale))
    assert np.array_equal(got, again)           # no atomics: bit-for-bit repeatable


CHANNEL_CASES = [
    (1, 4, 2, 37, 64, 0.5),
    (2, 8, 2, 300, 128, 0.3),
    (1, 4, 1, 513, 128, 0.0),       # nothing evicted
    (1, 4, 1, 100, 128, 1.0),       # everything evicted: key norms 0
]


@pytest.mark.parametrize("case", CHANNEL_CASES, ids=lambda c: "x".join(map(str, c)))
def test_channel_weights(dqa, case):
    B, Hq, Hkv, T, d, p_evict = case
    inp = rdkv_inputs(B, Hq, Hkv, d, T, seed=7 * T + d, outliers=OUTL)
    rng = np.random.default_rng(T)
    keep = (rng.random((B, Hkv, T)) >= p_evict).astype(np.int8) * 4
    say("rdkv_channel_weights", case)
    got = host(dqa.rdkv_channel_weights(dev(inp["q"]), dev(inp["k"]), dev(keep)))
    ref = oracle.channel_weights(inp["q"], inp["k"], keep)
    if p_evict == 1.0:
        assert np.all(got == 0)
    else:
        assert _rel(got, ref) <= 1e-5


def _alloc_weights(kind, rows, n, rng):
    if kind == "lognormal":
        return rng.lognormal(0, 2, (rows, n)).astype(np.float32)
    if kind == "zeros":
        w = rng.exponential(1.0, (rows, n)).astype(np.float32)
        w[rng.random((rows, n)) < 0.3] = 0
        return w
    if kind == "ties":           # few distinct values, powers of two apart
        return (2.0 ** rng.integers(-6, 6, (rows, n))).astype(np.float32)
    if kind == "uniform":
        return np.ones((rows, n), np.float32)
    raise ValueError(kind)


ALLOC_CASES = [
    # kind, rows, n, budgets as fractions of 16 n (1.0 = everything fits)
    ("lognormal", 3, 5000, (0.0, 0.05, 0.16, 0.5, 0.999, 1.0)),
    ("zeros", 2, 4097, (0.1, 0.3, 0.69, 0.7)),
    ("ties", 2, 9000, (0.1, 0.25, 0.6)),
    ("uniform", 1, 4096, (0.0, 0.125, 0.126, 0.5)),
    ("lognormal", 4, 1, (0.0, 0.5, 1.0)),
    ("lognormal", 1, 131072, (0.1625, 0.325)),
]


@pytest.mark.parametrize("case", ALLOC_CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}")
def test_allocate_exact(dqa, case):
    kind, rows, n, fracs = case
    rng = np.random.default_rng(n + rows)
    w = _alloc_weights(kind, rows, n, rng)
    wd = dev(w)
    for f in fracs:
        budget = int(f * 16 * n)
        say("rdkv_allocate", kind, rows, n, budget)
        got = host(dqa.rdkv_allocate(wd, budget))
        ref = oracle.allocate(w.astype(np.float64), budget)
        assert np.array_equal(got, ref), (budget, int((got != ref).sum()))
        assert np.all(got.astype(np.int64).sum(axis=1) <= budget)


def test_allocate_sanitizes_weights(dqa):
    # NaN, negative and -0 weights count as weight 0
    rng = np.random.default_rng(11)
    w = rng.exponential(1.0, (2, 300)).astype(np.float32)
    w[0, :10] = np.nan
    w[0, 10:20] = -3.0
    w[1, :5] = -0.0
    clean = np.where(w > 0, w, 0).astype(np.float32)
    say("rdkv_allocate sanitize")
    got = host(dqa.rdkv_allocate(dev(w), 2000))
    assert np.array_equal(got, oracle.allocate(clean.astype(np.float64), 2000))


def _near_tie_only(got, ref, w, budget):
    """Units where two width maps differ must sit near the critical
    breakpoint of the oracle's allocation (within the weight tolerance)."""
    diff = np.flatnonzero(got.ravel() != ref.ravel())
    if diff.size == 0:
        return True
    lam = oracle.multiplier(w.astype(np.float64), budget)
    for u in diff:
        bps = [float(w.ravel()[u]) * f for f, _ in oracle.rdkv.BREAKPOINTS]
        if min(abs(b - lam) for b in bps) > 4 * WTOL * max(lam, 1e-30):
            return False
    return True


WIDTH_CASES = [
    # B, Hq, Hkv, T, d, mean value width, mean key width
    (1, 4, 2, 200, 128, 2.6, 5.2),
    (2, 8, 2, 333, 64, 4.0, 3.0),
    (1, 4, 1, 64, 128, 16.0, 16.0),     # everything fits at full width
    (1, 4, 1, 64, 128, 0.0, 2.0),       # every token evicted
]


@pytest.mark.parametrize("case", WIDTH_CASES, ids=lambda c: "x".join(map(str, c)))
def test_widths_pipeline(dqa, case):
    B, Hq, Hkv, T, d, vm, km = case
    inp = rdkv_inputs(B, Hq, Hkv, d, T, seed=T * d, outliers=OUTL)
    scale = d ** -0.5
    vbud = oracle.budget_bits(vm, Hkv * T)
    kbud = oracle.budget_bits(km, Hkv * d)
    say("rdkv_widths", case)
    q, k = dev(inp["q"]), dev(inp["k"])
    vb, kb = (host(t) for t in dqa.rdkv_widths(q, k, scale, vbud, kbud))
    # each phase exactly as the oracle would allocate the GPU's own weights
    wt = host(dqa.rdkv_token_weights(q, k, scale))
    assert np.array_equal(vb, oracle.allocate(wt.reshape(B, -1).astype(np.float64), vbud).reshape(vb.shape))
    wc = host(dqa.rdkv_channel_weights(q, k, dev(vb)))
    assert np.array_equal(kb, oracle.allocate(wc.reshape(B, -1).astype(np.float64), kbud).reshape(kb.shape))
    # against the oracle's own pipeline: equal except at near-ties
    rvb, rkb = oracle.rdkv_widths(inp["q"], inp["k"], scale, vm, km)
    rwt = oracle.token_weights(inp["q"], inp["k"], scale)
    for b in range(B):
        assert _near_tie_only(vb[b], rvb[b], rwt[b], vbud)
        assert vb[b].astype(int).sum() <= vbud and kb[b].astype(int).sum() <= kbud
    if np.array_equal(vb, rvb):
        rwc = oracle.channel_weights(inp["q"], inp["k"], vb)
        for b in range(B):
            assert _near_tie_only(kb[b], rkb[b], rwc[b], kbud)


def test_maps_drive_the_zoned_cache(dqa):
    """The allocator's maps go straight into the zoned layout: plan, pack and
    decode run on them and match the oracle's zoned attention."""
    B, Hq, Hkv, T, d, C = 1, 8, 2, 300, 128, 8
    inp = rdkv_inputs(B, Hq, Hkv, d, T, seed=5, outliers=OUTL)
    z = zoned_inputs(B, Hq, Hkv, d, T, C, seed=6, v_width_probs={2: 1.0}, k_width_probs={2: 1.0})
    say("rdkv maps -> zoned decode")
    vb, kb = dqa.rdkv_widths(dev(inp["q"]), dev(inp["k"]), d ** -0.5,
                             oracle.budget_bits(2.6, Hkv * T), oracle.budget_bits(5.2, Hkv * d))
    vb, kb = host(vb), host(kb)
    plan = dqa.zoned_plan(vb, kb, C, d, "cuda:0")
    blob = dqa.zoned_pack(plan, dev(inp["k"]), dev(z["v"]), dev(z["k_new"]), dev(z["v_new"]))
    qd = z["q"]
    out = host(dqa.decode_attention_zoned(dev(qd), plan, blob, d ** -0.5))
    ref = oracle.zoned_decode_attention(qd, inp["k"], z["v"], vb, kb, z["k_new"], z["v_new"], d ** -0.5)
    check_attention(out, ref, 1e-3, "rdkv maps -> zoned decode")


def test_full_size_invariants(dqa):
    cfg = CONFIGS["mixed-width-zoned-16k"]
    B, Hq, Hkv, d, T = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T_old"]
    G = Hq // Hkv
    inp = rdkv_inputs(B, Hq, Hkv, d, T, seed=4, outliers=cfg["outliers"])
    scale = d ** -0.5
    vm, km = cfg["rdkv_mean_widths"]
    vbud, kbud = oracle.budget_bits(vm, Hkv * T), oracle.budget_bits(km, Hkv * d)
    say("rdkv full size", B, Hq, Hkv, T, d)
    q, k = dev(inp["q"]), dev(inp["k"])
    wt = host(dqa.rdkv_token_weights(q, k, scale))
    sums = wt.astype(np.float64).sum(axis=2)
    assert np.abs(sums / (G * T) - 1).max() <= 1e-4
    tail = np.arange(T - 16, T)
    ref_tail = oracle.token_weight_rows(inp["q"], inp["k"], scale, tail)[..., T - 16:]
    assert _rel(wt[..., T - 16:], ref_tail) <= WTOL
    # a slice three quarters into the sequence, for one (batch, KV head):
    # its weights need every query position from the slice on
    m, b0, h0 = 3 * T // 4, 1, 5
    ref_mid = oracle.token_weight_rows(inp["q"][b0:b0 + 1, h0 * G:(h0 + 1) * G], inp["k"][b0:b0 + 1, h0:h0 + 1],
                                       scale, np.arange(m, T))[0, 0, m:m + 64]
    assert _rel(wt[b0, h0, m:m + 64], ref_mid) <= WTOL
    vb, kb = (host(t) for t in dqa.rdkv_widths(q, k, scale, vbud, kbud))
    assert np.array_equal(vb, oracle.allocate(wt.reshape(B, -1).astype(np.float64), vbud).reshape(vb.shape))
    wc = host(dqa.rdkv_channel_weights(q, k, dev(vb)))
    ref_wc = oracle.channel_weights(inp["q"], inp["k"], vb)
    assert _rel(wc, ref_wc) <= 1e-5
    assert np.array_equal(kb, oracle.allocate(wc.reshape(B, -1).astype(np.float64), kbud).reshape(kb.shape))
    for b in range(B):
        assert vb[b].astype(int).sum() <= vbud and kb[b].astype(int).sum() <= kbud
