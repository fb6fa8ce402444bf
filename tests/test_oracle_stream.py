"""Pins of the oracle's streaming append ([P1 para 8, residual buffer]):
the window of full-precision tokens and the flush of its oldest groups.
CPU only."""
import numpy as np
import pytest

from oracle import empty_stream, flush_count, kivi_append, quantize_k, quantize_v, GROUP


def _tokens(B, H, T, d, seed):
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((B, H, T, d)) * rng.lognormal(0, 1, (1, H, 1, d))).astype(np.float16)
    v = rng.standard_normal((B, H, T, d)).astype(np.float16)
    return k, v


def _stream(k, v, bits, R_max, chunks):
    st = empty_stream(k.shape[0], k.shape[1], k.shape[3])
    t = 0
    for n in chunks:
        st = kivi_append(st, k[:, :, t:t + n], v[:, :, t:t + n], bits, R_max)
        t += n
        T_q, R = st["k_codes"].shape[2], st["k_recent"].shape[2]
        # window bound and token accounting after every append
        assert T_q % GROUP == 0 and T_q + R == t
        assert R <= R_max or R < GROUP
    return st, t


@pytest.mark.parametrize("bits,R_max,seed", [(2, 128, 1), (4, 64, 2), (8, 0, 3), (2, 31, 4), (4, 32, 5)])
def test_streaming_equals_batch_quantization(bits, R_max, seed):
    """Whatever the chunking, the quantized zone equals quantize_k / quantize_v
    of the first T_q tokens, and the window holds the remaining tokens."""
    B, H, T, d = 2, 3, 333, 64
    k, v = _tokens(B, H, T, d, seed)
    rng = np.random.default_rng(seed + 100)
    chunks = []
    while sum(chunks) < T:
        chunks.append(int(min(rng.integers(0, 45), T - sum(chunks))))
    st, t = _stream(k, v, bits, R_max, chunks)
    T_q = st["k_codes"].shape[2]
    assert t == T
    kc, ks, kz = quantize_k(k[:, :, :T_q], bits)
    vc, vs, vz = quantize_v(v[:, :, :T_q], bits)
    for a, b in [(st["k_codes"], kc), (st["k_scale"], ks), (st["k_zero"], kz),
                 (st["v_codes"], vc), (st["v_scale"], vs), (st["v_zero"], vz)]:
        assert a.dtype == b.dtype and np.array_equal(a, b)
    assert np.array_equal(st["k_recent"], k[:, :, T_q:]) and np.array_equal(st["v_recent"], v[:, :, T_q:])
    # nothing flushable is left behind: a further whole group would exceed the bound
    R = T - T_q
    assert not (R > R_max and R >= GROUP)


def test_hand_counted_flushes_one_token_at_a_time():
    """R_max = 128, one token per step: the window first reaches 129 tokens at
    step 129 and then every 32 steps; each time its oldest 32 go."""
    k, v = _tokens(1, 1, 230, 32, 7)
    st = empty_stream(1, 1, 32)
    expect = {1: 0, 128: 0, 129: 32, 160: 32, 161: 64, 192: 64, 193: 96, 225: 128, 230: 128}
    for t in range(1, 231):
        st = kivi_append(st, k[:, :, t - 1:t], v[:, :, t - 1:t], 2, 128)
        if t in expect:
            assert st["k_codes"].shape[2] == expect[t], t
            assert st["k_recent"].shape[2] == t - expect[t], t


def test_flush_count_closed_form():
    """Groups flushed: none at or below the bound; otherwise the fewest whole
    groups that bring the window to the bound, as long as a whole group is
    there."""
    assert flush_count(0, 0) == 0 and flush_count(31, 0) == 0 and flush_count(32, 0) == 1
    assert flush_count(100, 16) == 3                   # 100 -> 68 -> 36 -> 4
    assert flush_count(128, 128) == 0 and flush_count(129, 128) == 1
    assert flush_count(128 + 64, 128) == 2
    for rows in range(0, 300):
        for R_max in (0, 1, 31, 32, 64, 128):
            f = flush_count(rows, R_max)
            left = rows - 32 * f
            assert left >= 0 and not (left > R_max and left >= 32)
            assert f == 0 or (left + 32 > R_max)       # one group fewer would leave too many


def test_empty_append_is_identity():
    k, v = _tokens(1, 2, 40, 64, 9)
    st = kivi_append(empty_stream(1, 2, 64), k, v, 4, 128)
    st2 = kivi_append(st, k[:, :, :0], v[:, :, :0], 4, 128)
    for name in st:
        assert np.array_equal(st[name], st2[name])
