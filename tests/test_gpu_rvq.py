"""GPU parity of the residual-VQ path.  Indices are bit-exact against the
oracle except where the oracle's exact distances of the two codewords
differ by less than the GPU arithmetic's error bound (a documented tie);
after such a tie the comparison continues from the GPU's prefix.  Decode
attention over the GPU's indices is within relative L2 1e-3 of the oracle's
fp64 attention over the reconstructed cache."""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import say, dev, host, check_attention
from workloads import rvq_inputs, CONFIGS

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module")
def dqa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dequant_decode_attention_amd as m
    return m


def _error_bound(r, cb):
    """Per-codeword bound on |GPU key - exact key| (key = |c|^2 - 2 r.c):
    the two-fp16 split of -2r keeps 22 bits (2^-21 sum|r c| plus 2^-25 |c|_1
    for underflow of the low half); fp32 accumulation of the products and
    of |c|^2 over at most 300 roundings; the fp32 norm over 128 terms."""
    r = r.astype(np.float64)
    c = cb.astype(np.float64)
    S = np.abs(r)[None, :] @ np.abs(c).T                     # [1, Kc]
    c2 = (c * c).sum(1)[None, :]
    return (2.0 ** -21 * S + 2.0 ** -25 * np.abs(c).sum(1)[None, :]
            + 300 * 2.0 ** -24 * (c2 + 2 * S) + 128 * 2.0 ** -24 * c2)[0]


def check_indices(x16, cbs, gpu_idx):
    """Walk every vector's stages along the GPU's choices; returns the
    number of documented ties (raises on any other mismatch)."""
    ties = 0
    N = cbs.shape[0]
    for i in range(x16.shape[0]):
        r = x16[i].astype(np.float32)
        for s in range(N):
            d = oracle.rvq_stage_distances(r[None], cbs[s])[0]
            o = int(np.argmin(d))
            g = int(gpu_idx[i, s])
            if g != o:
                e = _error_bound(r, cbs[s])
                assert d[g] - d[o] <= e[g] + e[o], (i, s, g, o, d[g] - d[o], e[g] + e[o])
                ties += 1
            r = (r - cbs[s][g].astype(np.float32)).astype(np.float32)
    return ties


def test_exact_small_integer_codebooks_and_ties(dqa):
    """Integer data: every key is exact on both sides, so indices must match
    bit for bit, including lowest-index tie breaks on duplicated codewords."""
    rng = np.random.default_rng(0)
    N, Kc, d = 3, 128, 128
    cbs = rng.integers(-3, 4, size=(N, Kc, d)).astype(np.float16)
    cbs[0, 77] = cbs[0, 5]
    cbs[0, 100] = cbs[0, 5]
    cbs[1, 64:] = cbs[1, :64]                               # every stage-1 codeword twice
    x = rng.integers(-3, 4, size=(300, d)).astype(np.float16)
    x[:10] = cbs[0, 5]
    say("rvq_encode exact", x.shape, cbs.shape)
    g = host(dqa.rvq_encode(dev(x), dev(cbs)))
    ref, _ = oracle.rvq_encode(x, cbs)
    np.testing.assert_array_equal(g, ref)
    assert np.all(g[:10, 0] == 5)
    assert np.all(g[:, 1] < 64)


@pytest.mark.parametrize("n,N,Kc", [(300, 4, 128), (257, 2, 1024), (64, 1, 64), (1000, 8, 256)])
def test_encode_random(dqa, n, N, Kc):
    inp = rvq_inputs(1, 1, 1, 128, n, N, Kc, seed=n + N + Kc)
    x = inp["k"][0, 0]
    say("rvq_encode", n, N, Kc)
    g = host(dqa.rvq_encode(dev(x), dev(inp["k_cb"])))
    ties = check_indices(x, inp["k_cb"], g)
    ref, _ = oracle.rvq_encode(x, inp["k_cb"])
    print(f"documented ties: {ties}; exact-match fraction {np.mean(g == ref):.6f}", flush=True)
    assert ties <= max(1, n * N // 1000)


def test_full_config_encode_and_decode(dqa):
    cfg = CONFIGS["rvq-llama3.2-3b-8k"]
    inp = rvq_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T"], cfg["N"], cfg["Kc"], seed=5)
    B, Hkv, T, d, N = cfg["B"], cfg["Hkv"], cfg["T"], cfg["d"], cfg["N"]
    say("rvq full rvq-llama3.2-3b-8k encode")
    ki = dqa.rvq_encode(dev(inp["k"].reshape(-1, d)), dev(inp["k_cb"])).reshape(B, Hkv, T, N)
    vi = dqa.rvq_encode(dev(inp["v"].reshape(-1, d)), dev(inp["v_cb"])).reshape(B, Hkv, T, N)
    kih, vih = host(ki), host(vi)
    rng = np.random.default_rng(0)
    rows = rng.choice(B * Hkv * T, size=48, replace=False)
    ties = check_indices(inp["k"].reshape(-1, d)[rows], inp["k_cb"], kih.reshape(-1, N)[rows])
    ties += check_indices(inp["v"].reshape(-1, d)[rows], inp["v_cb"], vih.reshape(-1, N)[rows])
    print(f"rvq-llama3.2-3b-8k sampled vectors: documented ties {ties}", flush=True)
    say("rvq full rvq-llama3.2-3b-8k decode")
    scale = 1.0 / math.sqrt(d)
    out = host(dqa.rvq_decode_attention(dev(inp["q"]), ki, vi, dev(inp["k_cb"]), dev(inp["v_cb"]), scale))
    G = cfg["Hq"] // Hkv
    for b, h in [(b, h) for b in range(B) for h in range(Hkv)]:     # every unit
        ref = oracle.rvq_decode_attention(inp["q"][b:b + 1, h * G:(h + 1) * G], kih[b:b + 1, h:h + 1],
                                          vih[b:b + 1, h:h + 1], inp["k_cb"], inp["v_cb"], scale)
        check_attention(out[b, h * G:(h + 1) * G][None], ref, TOL, f"rvq-llama3.2-3b-8k decode unit ({b},{h})")


# key logits through the per-unit table when G * N * Kc <= 16384 floats, by
# gathered codewords otherwise: the last two cases take the gather path, the
# one before sits at the table's limit
@pytest.mark.parametrize("B,Hq,Hkv,T,N,Kc", [(1, 3, 1, 100, 4, 64), (2, 8, 2, 33, 2, 128),
                                             (1, 4, 4, 1, 1, 64), (2, 2, 1, 700, 8, 64),
                                             (1, 4, 1, 90, 4, 1024), (1, 4, 1, 150, 8, 1024),
                                             (1, 2, 1, 77, 4, 4096)])
def test_decode_attention_small(dqa, B, Hq, Hkv, T, N, Kc):
    inp = rvq_inputs(B, Hq, Hkv, 128, T, N, Kc, seed=T)
    rng = np.random.default_rng(T)
    ki = rng.integers(0, Kc, size=(B, Hkv, T, N)).astype(np.int16)
    vi = rng.integers(0, Kc, size=(B, Hkv, T, N)).astype(np.int16)
    scale = 1.0 / math.sqrt(128)
    say("rvq_decode_attention", B, Hq, Hkv, T, N, Kc)
    out = host(dqa.rvq_decode_attention(dev(inp["q"]), dev(ki), dev(vi), dev(inp["k_cb"]),
                                        dev(inp["v_cb"]), scale))
    ref = oracle.rvq_decode_attention(inp["q"], ki, vi, inp["k_cb"], inp["v_cb"], scale)
    check_attention(out, ref, TOL)


# long splits: up to three tiles per wave, so the value-row ring runs across
# tiles and the value indices are read two tiles ahead (table path at G = 3,
# gather path at G = 2); and four stages whose value indices are not 8-byte
# aligned (read one at a time)
@pytest.mark.parametrize("B,Hq,Hkv,T,N,Kc,v_offset", [(1, 3, 1, 40000, 4, 1024, 0),
                                                      (1, 2, 1, 40000, 4, 4096, 0),
                                                      (1, 4, 2, 3000, 4, 256, 1),
                                                      (2, 3, 1, 500, 3, 512, 0)])
def test_decode_attention_long_splits_and_index_alignment(dqa, B, Hq, Hkv, T, N, Kc, v_offset):
    inp = rvq_inputs(B, Hq, Hkv, 128, T, N, Kc, seed=T + N)
    rng = np.random.default_rng(T + Kc)
    ki = rng.integers(0, Kc, size=(B, Hkv, T, N)).astype(np.int16)
    vi = rng.integers(0, Kc, size=(B, Hkv, T, N)).astype(np.int16)
    # v_idx at v_offset int16 elements past an aligned allocation
    buf = torch.zeros(vi.size + v_offset, dtype=torch.int16, device="cuda")
    buf[v_offset:] = dev(vi.reshape(-1))
    v_dev = buf[v_offset:].view(vi.shape)
    assert (v_dev.data_ptr() % 8 == 0) == (v_offset == 0)
    scale = 1.0 / math.sqrt(128)
    say("rvq_decode_attention long/aligned", B, Hq, Hkv, T, N, Kc, v_offset)
    out = host(dqa.rvq_decode_attention(dev(inp["q"]), dev(ki), v_dev, dev(inp["k_cb"]),
                                        dev(inp["v_cb"]), scale))
    ref = oracle.rvq_decode_attention(inp["q"], ki, vi, inp["k_cb"], inp["v_cb"], scale)
    check_attention(out, ref, TOL)


def test_decode_attention_workspace_reuse(dqa):
    """One workspace for several calls: new queries over the same cache (the
    key-logit tables are rebuilt every call), another shape, and back; the
    table path and the gather path; each call against the oracle."""
    Kc, N = 512, 4
    shapes = [(2, 6, 2, 3000), (2, 6, 2, 3000), (1, 3, 1, 700), (2, 6, 2, 3000)]
    cases = []
    for i, (B, Hq, Hkv, T) in enumerate(shapes):
        inp = rvq_inputs(B, Hq, Hkv, 128, T, N, Kc, seed=100 + (i if i != 3 else 0))
        rng = np.random.default_rng(T)
        ki = rng.integers(0, Kc, size=(B, Hkv, T, N)).astype(np.int16)
        vi = rng.integers(0, Kc, size=(B, Hkv, T, N)).astype(np.int16)
        cases.append((inp, ki, vi))
    big = max(dqa.lib.rvq_decode_attention_workspace_bytes(B, Hq, Hkv, T, 128) for B, Hq, Hkv, T in shapes)
    for kc_gather in (False, True):
        ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
        for i, (inp, ki, vi) in enumerate(cases):
            kcb, vcb = inp["k_cb"], inp["v_cb"]
            if kc_gather:   # G * N * Kc above the table's limit: keys by gathered codewords
                kcb = np.ascontiguousarray(np.concatenate([kcb] * 9, axis=1))
                vcb = np.ascontiguousarray(np.concatenate([vcb] * 9, axis=1))
            scale = 1.0 / math.sqrt(128)
            say("rvq_decode_attention workspace reuse", i, shapes[i], "gather" if kc_gather else "table")
            out = host(dqa.rvq_decode_attention(dev(inp["q"]), dev(ki), dev(vi), dev(kcb), dev(vcb),
                                                scale, workspace=ws))
            ref = oracle.rvq_decode_attention(inp["q"], ki, vi, kcb, vcb, scale)
            check_attention(out, ref, TOL, f"reuse call {i}")


@pytest.mark.parametrize("B,Hq,Hkv,T,N,Kc", [(2, 6, 2, 3000, 4, 512), (1, 3, 1, 40000, 4, 1024),
                                             (1, 4, 4, 1, 1, 64), (2, 2, 1, 700, 8, 64)])
def test_decode_attention_table_built_alone(dqa, B, Hq, Hkv, T, N, Kc):
    """The path a workgroup takes when its (batch, KV head)'s other
    workgroups do not set their table flags within the poll bound: with the
    bound at 0 every workgroup builds the whole key-logit table itself (the
    flags are still set, so the calls after it find a consistent state)."""
    inp = rvq_inputs(B, Hq, Hkv, 128, T, N, Kc, seed=T + 1)
    rng = np.random.default_rng(T + 1)
    ki = rng.integers(0, Kc, size=(B, Hkv, T, N)).astype(np.int16)
    vi = rng.integers(0, Kc, size=(B, Hkv, T, N)).astype(np.int16)
    scale = 1.0 / math.sqrt(128)
    ref = oracle.rvq_decode_attention(inp["q"], ki, vi, inp["k_cb"], inp["v_cb"], scale)
    n = dqa.lib.rvq_decode_attention_workspace_bytes(B, Hq, Hkv, T, 128)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    args = (dev(inp["q"]), dev(ki), dev(vi), dev(inp["k_cb"]), dev(inp["v_cb"]), scale)
    prev = dqa.rvq_decode_set_table_polls(0)
    try:
        say("rvq_decode_attention table built alone", B, Hq, Hkv, T, N, Kc)
        alone = host(dqa.rvq_decode_attention(*args, workspace=ws))
    finally:
        dqa.rvq_decode_set_table_polls(prev)
    check_attention(alone, ref, TOL, "table built alone")
    say("rvq_decode_attention after it, shared table", B, Hq, Hkv, T, N, Kc)
    shared = host(dqa.rvq_decode_attention(*args, workspace=ws))
    check_attention(shared, ref, TOL, "shared table after")


def test_decode_attention_two_rounds_of_workgroups(dqa):
    """Keys by gathered codewords at 8 (batch, KV head) units x 86 splits:
    more workgroups than are resident at once, so the splits of one unit
    run in two rounds and its merge waits on the last; three calls, each
    against the oracle (a merge that reads a split's state before it has
    arrived shows as one wrong head)."""
    B, Hq, Hkv, T, N, Kc = 2, 12, 4, 8192, 4, 4608
    inp = rvq_inputs(B, Hq, Hkv, 128, T, N, Kc, seed=100)
    rng = np.random.default_rng(T)
    ki = rng.integers(0, Kc, size=(B, Hkv, T, N)).astype(np.int16)
    vi = rng.integers(0, Kc, size=(B, Hkv, T, N)).astype(np.int16)
    scale = 1.0 / math.sqrt(128)
    ref = oracle.rvq_decode_attention(inp["q"], ki, vi, inp["k_cb"], inp["v_cb"], scale)
    args = (dev(inp["q"]), dev(ki), dev(vi), dev(inp["k_cb"]), dev(inp["v_cb"]), scale)
    for call in range(3):
        say("rvq_decode_attention two rounds", call)
        check_attention(host(dqa.rvq_decode_attention(*args)), ref, TOL, f"two rounds call {call}")
