"""Pins for the RDKV allocation oracle (token and channel weights, the
Lagrangian width assignment).  CPU only."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle

WIDTHS = (0, 2, 4, 8, 16)


def _h(n):
    return sum(1.0 / i for i in range(1, n + 1))


# ---------------------------------------------------------------- weights

def test_uniform_attention_gives_harmonic_sums():
    # q = 0: every causal row is uniform, a_{tau,t} = 1/(tau+1), so
    # w_t = G * (H_T - H_t) with H the harmonic numbers.
    rng = np.random.default_rng(1)
    B, Hkv, G, T, d = 1, 2, 3, 9, 8
    q = np.zeros((B, Hkv * G, T, d), np.float16)
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    w = oracle.token_weights(q, k, 0.5)
    want = np.array([G * (_h(T) - _h(t)) for t in range(T)])
    np.testing.assert_allclose(w[0, 0], want, rtol=1e-12)
    np.testing.assert_allclose(w[0, 1], want, rtol=1e-12)
    assert abs(w.sum() - B * Hkv * G * T) < 1e-9


def test_two_tokens_sigmoid_form():
    # T = 2: row 0 sees only token 0; row 1 splits as a logistic function
    # of the scaled logit difference.
    q = np.zeros((1, 2, 2, 4), np.float16)
    k = np.zeros((1, 1, 2, 4), np.float16)
    q[0, 0, 1] = [1, 2, 0, 0]
    q[0, 1, 1] = [0, 0, -1, 0.5]
    k[0, 0, 0] = [0.5, 0, 1, 0]
    k[0, 0, 1] = [0, 1, 0, 2]
    scale = 0.75
    w = oracle.token_weights(q, k, scale)[0, 0]
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))
    want1 = 0.0
    want0 = 2.0                      # both heads' row 0
    for h in range(2):
        q1 = q[0, h, 1].astype(np.float64)
        dlt = scale * (q1 @ k[0, 0, 1].astype(np.float64) - q1 @ k[0, 0, 0].astype(np.float64))
        want1 += sig(dlt)
        want0 += sig(-dlt)
    np.testing.assert_allclose(w, [want0, want1], rtol=1e-12)


def test_grouped_heads_read_their_own_kv_head():
    # group 0's queries are zero (uniform rows over random keys), group 1's
    # are not: KV head 0 must come out harmonic, KV head 1 must not.
    rng = np.random.default_rng(2)
    B, Hkv, G, T, d = 1, 2, 2, 7, 8
    q = rng.standard_normal((B, Hkv * G, T, d)).astype(np.float16) * 2
    q[:, :G] = 0
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16) * 2
    w = oracle.token_weights(q, k, 1.0)
    want = np.array([G * (_h(T) - _h(t)) for t in range(T)])
    np.testing.assert_allclose(w[0, 0], want, rtol=1e-12)
    assert np.abs(w[0, 1] - want).max() > 0.1
    np.testing.assert_allclose(w[0, 1].sum(), G * T, rtol=1e-12)


def test_row_subset_matches_tail_of_full_weights():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 4, 20, 16)).astype(np.float16)
    k = rng.standard_normal((2, 2, 20, 16)).astype(np.float16)
    full = oracle.token_weights(q, k, 0.25)
    part = oracle.token_weight_rows(q, k, 0.25, np.arange(14, 20))
    np.testing.assert_allclose(part[..., 14:], full[..., 14:], rtol=1e-12)


def test_channel_weights_hand_worked():
    # d = 4, G = 2, T = 4.  Channel 1: the group's query entries 3 (head 0)
    # and 4 (head 1) give norm 5; the kept keys 1, 2, 2 give norm 3; the
    # evicted token holds 100 and must not count.  w = 5 * 3 / sqrt(4).
    q = np.zeros((1, 2, 4, 4), np.float16)
    k = np.zeros((1, 1, 4, 4), np.float16)
    q[0, 0, 2, 1] = 3
    q[0, 1, 0, 1] = 4
    k[0, 0, :, 1] = [1, 100, 2, 2]
    keep = np.array([[[2, 0, 4, 16]]], np.int8)
    # channel 3: query entries 1 at every position of both heads (norm
    # sqrt(8)); kept keys all 0.5 (norm sqrt(3)/2)
    q[0, :, :, 3] = 1
    k[0, 0, :, 3] = 0.5
    w = oracle.channel_weights(q, k, keep)
    np.testing.assert_allclose(w[0, 0], [0, 7.5, 0, np.sqrt(8) * np.sqrt(3) / 2 / 2],
                               rtol=1e-12)


# ------------------------------------------------------------- allocation

def _exact_argmin(w, lam):
    w, lam = Fraction(float(w)), Fraction(float(lam))
    costs = [w * Fraction(1, 2 ** b) + lam * b for b in WIDTHS]
    return WIDTHS[costs.index(min(costs))]          # first = smaller width


def test_width_rule_is_the_exact_argmin():
    rng = np.random.default_rng(4)
    w = np.concatenate([rng.exponential(1.0, 200), [0.0, 1.0, 2.0, 0.5]]).astype(np.float32)
    lams = [0.0] + [float(x) for x in rng.exponential(0.05, 40)]
    # every breakpoint is a tie between two widths
    lams += [float(np.float64(wi) * f) for wi in w[-4:] for f, _ in oracle.rdkv.BREAKPOINTS]
    for lam in lams:
        got = oracle.widths_at(w, lam)
        want = [_exact_argmin(wi, lam) for wi in w]
        assert list(got) == want, lam


def _objective(w, b):
    return sum(Fraction(float(wi)) * Fraction(1, 2 ** int(bi)) for wi, bi in zip(w, b))


def test_lagrangian_solution_is_optimal_for_its_own_total():
    # Everett: the widths at any multiplier minimize the objective among all
    # assignments whose total does not exceed theirs (brute force, 5^5).
    rng = np.random.default_rng(5)
    for trial in range(12):
        w = rng.exponential(1.0, 5).astype(np.float32)
        budget = int(rng.integers(0, 81))
        b = oracle.allocate(w, budget)
        tot = int(b.sum())
        assert tot <= budget
        best = min(_objective(w, c) for c in itertools.product(WIDTHS, repeat=5)
                   if sum(c) <= tot)
        assert _objective(w, b) == best


def test_multiplier_is_the_smallest_that_fits():
    rng = np.random.default_rng(6)
    for trial in range(20):
        w = rng.exponential(1.0, 7).astype(np.float32)
        w[rng.integers(0, 7)] = w[rng.integers(0, 7)]          # a repeated weight
        budget = int(rng.integers(0, 113))
        lam = oracle.multiplier(w, budget)
        assert oracle.widths_at(w, lam).astype(int).sum() <= budget
        cands = sorted({0.0} | {float(np.float64(x) * f) for x in w
                                for f, _ in oracle.rdkv.BREAKPOINTS})
        for c in cands:
            if c < lam:
                assert oracle.widths_at(w, c).astype(int).sum() > budget


def test_hand_worked_allocation():
    # w = 1, 2, 4.  Breakpoints (3w/8, 3w/32, ...): at lam = 3/8 unit 1 drops
    # to 0 and unit 3 ties 2-vs-4 and takes 2, total 4 <= 6; just below
    # (lam = 3/16, unit 2's second breakpoint) the total is 2 + 2 + 4 = 8.
    w = np.array([1.0, 2.0, 4.0])
    assert oracle.multiplier(w, 6) == 0.375
    assert list(oracle.allocate(w, 6)) == [0, 2, 2]
    assert list(oracle.allocate(w, 8)) == [2, 2, 4]
    assert list(oracle.allocate(w, 48)) == [16, 16, 16]
    assert list(oracle.allocate(w, 0)) == [0, 0, 0]
    assert list(oracle.allocate([0.0, 3.0], 32)) == [0, 16]


def test_widths_grow_with_the_budget_and_ignore_scale():
    rng = np.random.default_rng(7)
    w = rng.lognormal(0, 2, 300).astype(np.float32)
    prev = None
    for budget in range(0, 16 * 300 + 1, 97):
        b = oracle.allocate(w, budget)
        assert b.astype(int).sum() <= budget
        if prev is not None:
            assert np.all(b >= prev)
        prev = b
        # a power-of-two scale of every weight scales every breakpoint exactly
        assert np.array_equal(oracle.allocate(w * np.float32(8), budget), b)


def test_allocation_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.multiplier([1.0, -1.0], 4)
    with pytest.raises(ValueError):
        oracle.multiplier([1.0, np.nan], 4)
    with pytest.raises(ValueError):
        oracle.multiplier([1.0], -1)


def test_pipeline_meets_both_budgets():
    rng = np.random.default_rng(8)
    B, Hkv, G, T, d = 2, 2, 2, 48, 32
    q = rng.standard_normal((B, Hkv * G, T, d)).astype(np.float16)
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    vb, kb = oracle.rdkv_widths(q, k, d ** -0.5, 3.0, 5.0)
    for b in range(B):
        assert vb[b].astype(int).sum() <= 3.0 * Hkv * T
        assert kb[b].astype(int).sum() <= 5.0 * Hkv * d
    assert set(np.unique(vb)) <= set(WIDTHS) and set(np.unique(kb)) <= set(WIDTHS)
    # the most attended token of a sequence never gets fewer bits than the
    # least attended one
    wt = oracle.token_weights(q, k, d ** -0.5)
    for b in range(B):
        i, j = np.argmax(wt[b]), np.argmin(wt[b])
        assert vb[b].ravel()[i] >= vb[b].ravel()[j]
