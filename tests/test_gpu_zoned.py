"""GPU parity of the mixed-width zoned path: the packed blob is bit-exact
against the oracle's byte image; decode attention is within relative L2
1e-3 of the oracle's fp64 attention over its own dequantized values."""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import say, dev, host, check_attention
from workloads import zoned_inputs, CONFIGS

pytestmark = pytest.mark.gpu
TOL = 1e-3
PV = {0: 0.5, 2: 0.2, 4: 0.15, 8: 0.1, 16: 0.05}
PK = {2: 0.4, 4: 0.3, 8: 0.2, 16: 0.1}


@pytest.fixture(scope="module")
def dqa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dequant_decode_attention_amd as m
    return m


def _marked_blob(plan):
    """A blob buffer pre-filled with 0xA5, so that a byte the packer leaves
    unwritten differs from the oracle's image (whose padding is zero)."""
    return torch.full((plan.blob_bytes,), 0xA5, dtype=torch.uint8, device="cuda:0")


def _run(dqa, inp, d):
    plan = dqa.zoned_plan(inp["v_bits"], inp["k_bits"], inp["k_new"].shape[2], d, "cuda:0")
    blob = dqa.zoned_pack(plan, dev(inp["k"]), dev(inp["v"]),
                          dev(inp["k_new"]) if inp["k_new"].shape[2] else None,
                          dev(inp["v_new"]) if inp["v_new"].shape[2] else None, out=_marked_blob(plan))
    return plan, blob


CASES = [
    # B, Hq, Hkv, d, T_old, C, v-probs, k-probs
    (1, 4, 1, 128, 300, 8, PV, PK),
    (2, 8, 2, 64, 513, 64, PV, PK),
    (1, 2, 2, 128, 200, 0, PV, PK),
    (1, 4, 1, 128, 96, 33, {16: 1.0}, {16: 1.0}),           # all 16-bit: unquantized
    (1, 4, 2, 128, 128, 5, {2: 1.0}, {2: 1.0}),             # single width class
    (1, 4, 1, 64, 64, 4, {0: 1.0}, PK),                     # everything evicted: zone C only
    (2, 4, 2, 128, 1000, 64, {0: .3, 8: .7}, {8: .5, 16: .5}),
    (1, 4, 2, 128, 300, 16, PV, {0: .25, 2: .25, 4: .2, 8: .15, 16: .15}),   # evicted key channels
    (1, 4, 1, 64, 100, 4, PV, {0: 1.0}),                                    # every key channel evicted
    (2, 4, 2, 64, 150, 8, PV, {0: .85, 2: .1, 16: .05}),    # key rows of 1-3 words: 16-byte pieces span slots
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}x{c[3]}-T{c[4]}-C{c[5]}")
def test_zoned_pack_and_decode(dqa, case):
    B, Hq, Hkv, d, T, C, pv, pk = case
    inp = zoned_inputs(B, Hq, Hkv, d, T, C, seed=T + C, v_width_probs=pv, k_width_probs=pk,
                       outliers=("lognormal", 0.04, 3.0, 1.0))
    say("zoned_pack/decode", case[:6])
    plan, blob = _run(dqa, inp, d)
    ref_blob = oracle.zoned_pack(inp["k"], inp["v"], inp["v_bits"], inp["k_bits"], inp["k_new"], inp["v_new"])
    got_blob = host(blob)
    assert got_blob.size == ref_blob.size
    if not np.array_equal(got_blob, ref_blob):
        bad = np.flatnonzero(got_blob != ref_blob)
        pytest.fail(f"blob differs at {bad.size} bytes, first {bad[:8]}")
    scale = 1.0 / math.sqrt(d)
    out = host(dqa.decode_attention_zoned(dev(inp["q"]), plan, blob, scale))
    ref = oracle.zoned_decode_attention(inp["q"], inp["k"], inp["v"], inp["v_bits"], inp["k_bits"],
                                        inp["k_new"], inp["v_new"], scale)
    if np.all(inp["v_bits"] == 0) and C == 0:
        assert np.all(out == 0)
        return
    check_attention(out, ref, TOL)
    out2 = host(dqa.decode_attention_zoned(dev(inp["q"]), plan, blob, scale))
    assert np.array_equal(out2, out)


def test_zoned_full_config_sampled(dqa):
    cfg = CONFIGS["mixed-width-zoned-16k"]
    inp = zoned_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T_old"], cfg["C"], seed=4,
                       v_width_probs=cfg["v_width_probs"], k_width_probs=cfg["k_width_probs"],
                       outliers=cfg["outliers"])
    say("zoned full mixed-width-zoned-16k")
    plan, blob = _run(dqa, inp, cfg["d"])
    scale = 1.0 / math.sqrt(cfg["d"])
    out = host(dqa.decode_attention_zoned(dev(inp["q"]), plan, blob, scale))
    got_blob = host(blob)
    units, total = oracle.zoned_layout(inp["v_bits"], inp["k_bits"], cfg["d"], cfg["C"])
    assert got_blob.size == total
    G = cfg["Hq"] // cfg["Hkv"]
    for b, h in [(b, h) for b in range(cfg["B"]) for h in range(cfg["Hkv"])]:
        # every unit; the oracle packs and attends one unit at a time
        sl = lambda x: x[b:b + 1, h:h + 1]
        ref_blob = oracle.zoned_pack(sl(inp["k"]), sl(inp["v"]), sl(inp["v_bits"]), sl(inp["k_bits"]),
                                     sl(inp["k_new"]), sl(inp["v_new"]))
        lay = units[b * cfg["Hkv"] + h]
        assert np.array_equal(got_blob[lay["base"]:lay["base"] + lay["size"]], ref_blob)
        ref = oracle.zoned_decode_attention(inp["q"][b:b + 1, h * G:(h + 1) * G], sl(inp["k"]), sl(inp["v"]),
                                            sl(inp["v_bits"]), sl(inp["k_bits"]), sl(inp["k_new"]),
                                            sl(inp["v_new"]), scale)
        check_attention(out[b, h * G:(h + 1) * G][None], ref, TOL, f"mixed-width-zoned-16k unit ({b},{h})")


SINK_OUT_CASES = [
    # B, Hq, Hkv, d, T_old, C, sink, k_out, v-probs, k-probs
    (1, 4, 1, 128, 300, 8, 4, 0, PV, PK),                        # sink only
    (1, 4, 2, 64, 200, 0, 0, 1, PV, PK),                         # outliers only
    (2, 8, 2, 128, 513, 16, 16, 2, PV, PK),
    (1, 4, 1, 128, 100, 4, 0, 4, {2: .5, 4: .5}, {2: .5, 8: .5}),
    (1, 4, 2, 64, 70, 3, 70, 1, PV, PK),                         # the whole old cache as sink
    (1, 4, 1, 128, 300, 16, 8, 3, PV, {0: .2, 2: .3, 4: .2, 8: .2, 16: .1}),   # with evicted channels
    (2, 2, 2, 64, 257, 5, 33, 4, PV, PK),                        # head ratio 1, d 64, longest side list
    (1, 4, 2, 128, 90, 0, 2, 2, {8: 1.0}, {2: .5, 4: .5}),       # head ratio 2, one width
]


@pytest.mark.parametrize("case", SINK_OUT_CASES,
                         ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}x{c[3]}-T{c[4]}-C{c[5]}-S{c[6]}-o{c[7]}")
def test_zoned_sink_and_outliers(dqa, case):
    B, Hq, Hkv, d, T, C, S, ko, pv, pk = case
    inp = zoned_inputs(B, Hq, Hkv, d, T, C, seed=3 * T + S + ko, v_width_probs=pv, k_width_probs=pk,
                       outliers=("lognormal", 0.04, 3.0, 1.0))
    # key spikes inside the groups, so that the side lists hold real outliers
    rng = np.random.default_rng(T)
    k = inp["k"].copy()
    idx = rng.integers(0, [B, Hkv, T, d], size=(max(1, T // 10), 4))
    k[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]] = np.float16(90.0)
    inp["k"] = k
    say("zoned sink/outliers", case[:8])
    plan = dqa.zoned_plan(inp["v_bits"], inp["k_bits"], C, d, "cuda:0", sink=S, k_out=ko)
    blob = dqa.zoned_pack(plan, dev(inp["k"]), dev(inp["v"]),
                          dev(inp["k_new"]) if C else None, dev(inp["v_new"]) if C else None,
                          out=_marked_blob(plan))
    ref_blob = oracle.zoned_pack(inp["k"], inp["v"], inp["v_bits"], inp["k_bits"], inp["k_new"],
                                 inp["v_new"], sink=S, k_out=ko)
    got_blob = host(blob)
    assert got_blob.size == ref_blob.size
    if not np.array_equal(got_blob, ref_blob):
        bad = np.flatnonzero(got_blob != ref_blob)
        pytest.fail(f"blob differs at {bad.size} bytes, first {bad[:8]}")
    scale = 1.0 / math.sqrt(d)
    out = host(dqa.decode_attention_zoned(dev(inp["q"]), plan, blob, scale))
    ref = oracle.zoned_decode_attention(inp["q"], inp["k"], inp["v"], inp["v_bits"], inp["k_bits"],
                                        inp["k_new"], inp["v_new"], scale, sink=S, k_out=ko)
    check_attention(out, ref, TOL)
