"""Oracle: RDKV bit allocation -- distortion weights and the Lagrangian
width assignment that produce the zoned cache's width maps.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the page defines ([P3 sec 2.1, theoretical formulation] and [P3 sec
2.2, bit-allocation pipeline]):

* value-cache unit = token, weight w_t = sum over query positions tau of the
  attention a_{tau,t} the token receives;
* key-cache unit = channel, weight w_c = ||Q_{:,c}||_2 ||K_{:,c}||_2 / sqrt(d);
* widths b_u in {0, 2, 4, 8, 16} minimize sum_u w_u sigma_u 2^(-b_u) subject
  to sum_u b_u <= B, by Lagrangian relaxation (reverse water-filling); the
  weights are computed once after prefill from the full cache; phase 2
  assigns token widths, phase 3 channel widths over the tokens phase 2 kept.

Readings fixed here:

* a_{tau,t} is the causal prefill attention (t <= tau) with logits scaled by
  sm_scale; with grouped heads a KV token's weight sums over the G query
  heads that read it.  Q_{:,c} is the channel over every query position of
  those G heads; K_{:,c} runs over the kept tokens only.
* sigma_u = 1 (the page does not define it).
* for a multiplier lam >= 0 every unit takes the width that minimizes
  w 2^(-b) + lam b, the smaller width on a tie; lam is the smallest value at
  which the total width fits the budget.  Between consecutive widths b < b'
  the unit prefers b' exactly while lam < w (2^-b - 2^-b') / (b' - b); the
  four factors 3/8, 3/32, 15/1024, 255/524288 decrease, so the minimizing
  width is 2[lam < 3w/8] + 2[lam < 3w/32] + 4[lam < 15w/1024]
  + 8[lam < 255w/524288].  The products w * factor are formed in float64:
  exact for float32 weights (the tests' hand-made and GPU-produced weights),
  one rounding for float64 weights.
* a budget covers one row of units; the pipeline below uses one row per
  sequence, over all its KV heads (the objective sums over every unit of the
  cache under one B), with B = floor(average width x number of units).

Parity: pinned by tests/test_oracle_rdkv.py (harmonic closed form of uniform
attention, the two-token sigmoid form, GQA grouping, hand-worked channel
norms with evicted tokens, the width rule against an exact rational argmin,
Lagrangian optimality by brute force on tiny instances, minimality of the
multiplier, a hand-worked allocation, monotonicity in the budget).
"""

import numpy as np

WIDTHS = (0, 2, 4, 8, 16)
# (factor, width increment) per breakpoint, largest factor first
BREAKPOINTS = ((3.0 / 8, 2), (3.0 / 32, 2), (15.0 / 1024, 4), (255.0 / 524288, 8))


def token_weights(q16, k16, sm_scale):
    """w [B, Hkv, T] (fp64): causal attention received by every key token,
    summed over query positions and over the G query heads of a KV head.

    q16 fp16 [B, Hq, T, d] (every prefill query position), k16 fp16
    [B, Hkv, T, d] (keys as attention reads them)."""
    q = np.asarray(q16, np.float16).astype(np.float64)
    k = np.asarray(k16, np.float16).astype(np.float64)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    w = np.zeros((B, Hkv, T))
    causal = np.tril(np.ones((T, T), bool))          # [tau, t]: t <= tau
    for b in range(B):
        for h in range(Hq):
            s = sm_scale * (q[b, h] @ k[b, h // G].T)     # [tau, t]
            s = np.where(causal, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            w[b, h // G] += p.sum(axis=0)
    return w


def token_weight_rows(q16, k16, sm_scale, rows):
    """Contribution of the query positions ``rows`` only: [B, Hkv, T].  When
    rows holds every position from t0 to T-1, the entries t >= t0 are the
    full weights (the last tokens of a long sequence can be checked without
    forming its whole attention matrix)."""
    q = np.asarray(q16, np.float16).astype(np.float64)
    k = np.asarray(k16, np.float16).astype(np.float64)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    rows = np.asarray(rows)
    w = np.zeros((B, Hkv, T))
    causal = np.arange(T)[None, :] <= rows[:, None]
    for b in range(B):
        for h in range(Hq):
            s = sm_scale * (q[b, h, rows] @ k[b, h // G].T)
            s = np.where(causal, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            w[b, h // G] += p.sum(axis=0)
    return w


def channel_weights(q16, k16, keep):
    """w [B, Hkv, d] (fp64): ||Q_{:,c}|| ||K_{kept,c}|| / sqrt(d); keep
    [B, Hkv, T] marks the tokens phase 2 kept (nonzero = kept)."""
    q = np.asarray(q16, np.float16).astype(np.float64)
    k = np.asarray(k16, np.float16).astype(np.float64)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    w = np.zeros((B, Hkv, d))
    for b in range(B):
        for h in range(Hkv):
            qn = np.sqrt((q[b, h * G:(h + 1) * G] ** 2).sum(axis=(0, 1)))
            kept = np.asarray(keep[b, h]) != 0
            kn = np.sqrt((k[b, h][kept] ** 2).sum(axis=0))
            w[b, h] = qn * kn / np.sqrt(d)
    return w


def widths_at(w, lam):
    """Width of every unit at the multiplier lam (ties to the smaller
    width)."""
    w = np.asarray(w, np.float64)
    b = np.zeros(w.shape, np.int64)
    for f, inc in BREAKPOINTS:
        b += inc * (lam < w * f)
    return b.astype(np.int8)


def multiplier(w, budget):
    """Smallest lam >= 0 at which widths_at(w, lam) totals <= budget.  The
    total only changes at a breakpoint w_u * f and never rises with lam, so
    lam is 0 or a breakpoint; the totals of all candidates are counted from
    the sorted breakpoints."""
    w = np.asarray(w, np.float64).ravel()
    if np.any(~np.isfinite(w)) or np.any(w < 0):
        raise ValueError("weights must be finite and non-negative")
    if budget < 0:
        raise ValueError("budget must be non-negative")
    bps = [np.sort(w * f) for f, _ in BREAKPOINTS]
    cands = np.unique(np.concatenate([[0.0]] + bps))
    total = np.zeros(cands.shape, np.int64)
    for (f, inc), bp in zip(BREAKPOINTS, bps):
        # units whose breakpoint lies strictly above the candidate
        total += inc * (len(bp) - np.searchsorted(bp, cands, side="right"))
    return cands[np.flatnonzero(total <= budget)[0]]


def allocate(w, budget):
    """Widths int8 [..., n] for weights w [..., n]: one Lagrangian problem
    per row (last axis) with the same total budget (bits) for every row."""
    w = np.asarray(w, np.float64)
    rows = w.reshape(-1, w.shape[-1])
    out = np.empty(rows.shape, np.int8)
    for i, wr in enumerate(rows):
        out[i] = widths_at(wr, multiplier(wr, budget))
    return out.reshape(w.shape)


def budget_bits(avg_width, n_units):
    """Total budget of a row of n_units units at an average width."""
    return int(np.floor(avg_width * n_units))


def rdkv_widths(q16, k16, sm_scale, v_avg_width, k_avg_width):
    """Phases 1-3: (v_bits [B, Hkv, T], k_bits [B, Hkv, d]) int8.  One row per
    sequence over all its KV heads; the value budget counts tokens, the key
    budget channels.  The allocation runs on the weights exactly as their
    definitions give them (float64), as [P3 sec 2.1] and [P3 sec 2.2,
    bit-allocation pipeline] define the objective on w_u itself."""
    B, Hq, T, d = np.shape(q16)
    Hkv = np.shape(k16)[1]
    wt = token_weights(q16, k16, sm_scale)
    vb = allocate(wt.reshape(B, Hkv * T), budget_bits(v_avg_width, Hkv * T))
    vb = vb.reshape(B, Hkv, T)
    wc = channel_weights(q16, k16, vb)
    kb = allocate(wc.reshape(B, Hkv * d), budget_bits(k_avg_width, Hkv * d))
    return vb, kb.reshape(B, Hkv, d)
