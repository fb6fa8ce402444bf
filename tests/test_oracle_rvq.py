"""Pins of the residual-VQ oracle ([P2 sec 2, key components: RSimVQ, prefill
and decoding phases]; [P2] = VQKV summary, gist.science/it/paper/2603.16435).
CPU only."""
import numpy as np
import pytest
from scipy.spatial.distance import cdist

from oracle import rvq_encode, rvq_reconstruct, rvq_decode_attention, rvq_stage_distances, attention_fp64
from workloads import rvq_inputs


def test_stage_distances_against_scipy():
    rng = np.random.default_rng(0)
    r = rng.standard_normal((20, 16)).astype(np.float32)
    cb = rng.standard_normal((50, 16)).astype(np.float16)
    np.testing.assert_allclose(rvq_stage_distances(r, cb),
                               cdist(r.astype(np.float64), cb.astype(np.float64), "sqeuclidean"),
                               rtol=1e-12)


def test_brute_force_nearest_tiny_codebooks():
    rng = np.random.default_rng(1)
    N, Kc, d = 3, 8, 6
    cbs = (rng.standard_normal((N, Kc, d)) * [[[1.0]], [[0.5]], [[0.25]]]).astype(np.float16)
    x = rng.standard_normal((40, d)).astype(np.float16)
    idx, res = rvq_encode(x, cbs)
    for i in range(40):
        r = x[i].astype(np.float32)
        for s in range(N):
            # exhaustive search with an independent distance formula
            best = min(range(Kc), key=lambda j: (float(np.sum((r.astype(np.float64) - cbs[s, j].astype(np.float64)) ** 2)), j))
            assert idx[i, s] == best
            r = (r - cbs[s, best].astype(np.float32)).astype(np.float32)
        np.testing.assert_array_equal(res[i], r)


def test_single_stage_is_plain_vq_and_reconstruction():
    rng = np.random.default_rng(2)
    cb = rng.standard_normal((1, 64, 32)).astype(np.float16)
    x = rng.standard_normal((100, 32)).astype(np.float16)
    idx, res = rvq_encode(x, cb)
    d = cdist(x.astype(np.float64), cb[0].astype(np.float64), "sqeuclidean")
    np.testing.assert_array_equal(idx[:, 0], d.argmin(1))
    # reconstruction plus final residual gives back the input
    np.testing.assert_allclose(rvq_reconstruct(idx, cb) + res, x.astype(np.float64), rtol=0, atol=1e-6)


def test_exact_codeword_then_min_norm():
    rng = np.random.default_rng(3)
    cbs = rng.standard_normal((3, 16, 8)).astype(np.float16)
    x = cbs[0, [5, 9, 0]]
    idx, res = rvq_encode(x, cbs)
    np.testing.assert_array_equal(idx[:, 0], [5, 9, 0])
    # zero residual: each later stage picks its minimum-norm codeword
    for s in (1, 2):
        assert np.all(idx[:, s] == np.argmin((cbs[s].astype(np.float64) ** 2).sum(1)))


def test_ties_go_to_lowest_index_small_integers():
    # small-integer codebooks make every distance exact in fp32 and fp64;
    # duplicated codewords tie exactly
    rng = np.random.default_rng(4)
    cb = rng.integers(-4, 5, size=(2, 12, 8)).astype(np.float16)
    cb[0, 7] = cb[0, 2]
    cb[0, 11] = cb[0, 2]
    x = np.concatenate([cb[0, [2]], rng.integers(-4, 5, size=(30, 8)).astype(np.float16)])
    idx, _ = rvq_encode(x, cb)
    assert idx[0, 0] == 2
    for i in range(x.shape[0]):
        dist = ((x[i].astype(np.int64) - cb[0].astype(np.int64)) ** 2).sum(1)
        assert idx[i, 0] == np.flatnonzero(dist == dist.min())[0]


def test_prefix_continuation():
    inp = rvq_inputs(1, 2, 1, 32, 40, 3, 16, seed=5)
    x = inp["k"][0, 0]
    idx, _ = rvq_encode(x, inp["k_cb"])
    idx2, _ = rvq_encode(x, inp["k_cb"], prefix=idx[:, :1])
    np.testing.assert_array_equal(idx, idx2)
    alt = (idx[:, :1] + 1) % 16
    idx3, _ = rvq_encode(x, inp["k_cb"], prefix=alt)
    np.testing.assert_array_equal(idx3[:, 0], alt[:, 0])


def test_decode_attention_over_reconstruction():
    inp = rvq_inputs(1, 6, 2, 32, 50, 2, 16, seed=6)
    ki = np.stack([np.stack([rvq_encode(inp["k"][0, h], inp["k_cb"])[0] for h in range(2)])])
    vi = np.stack([np.stack([rvq_encode(inp["v"][0, h], inp["v_cb"])[0] for h in range(2)])])
    o = rvq_decode_attention(inp["q"], ki, vi, inp["k_cb"], inp["v_cb"], 0.2)
    for h in range(6):
        k = rvq_reconstruct(ki[0, h // 3], inp["k_cb"])
        v = rvq_reconstruct(vi[0, h // 3], inp["v_cb"])
        ref = attention_fp64(inp["q"][0, h][None].astype(np.float64), k, v, 0.2)
        np.testing.assert_allclose(o[0, h], ref[0], rtol=1e-11, atol=1e-13)
