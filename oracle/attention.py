"""Oracle: decode attention over a dequantized KIVI-layout cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where it is defined:

* [P1 para 2] / [P3 sec 1]: at each decode step the new query attends over
  every cached key/value; the whole cache is read.
* [P1 para 6]: the attention output is the softmax-weighted sum of the
  value vectors; quality is judged on this output.
* [P1 para 7]: keys are quantized *before* RoPE and the rotation is applied
  after dequantization (KVQuant ordering).  RoPE rotates pairs of channels
  by an angle proportional to the token position.
* [P1 para 8]: up to 128 most recent tokens stay in full precision (the
  residual buffer); they are attended together with the quantized tokens.

Readings (the pages give no formulas): softmax scale passed by the caller
(1/sqrt(d) in every workload); query head h reads KV head h // (Hq/Hkv);
RoPE pairs are interleaved channels (2i, 2i+1) with frequency
theta^(-2i/d), angle = position * frequency, and (a, b) -> (a cos - b sin,
a sin + b cos); quantized tokens sit at positions 0..T_q-1 and recent tokens
at T_q..T_q+R-1; the query arrives already rotated.
"""

import numpy as np

from .quant import GROUP, unpack_codes, unpack_v_codes, dequantize_k, dequantize_v


def rope_frequencies(d, theta):
    """omega_i = theta^(-2i/d), i = 0..d/2-1, in fp64 ([P1 para 7], reading
    of the rotary frequency schedule)."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / d)


def rope_rotate(x, positions, theta):
    """Rotate interleaved channel pairs of x [T, d] (fp64) by position.

    For pair i of token t: phi = positions[t] * omega_i,
    (a, b) -> (a cos phi - b sin phi, a sin phi + b cos phi).
    """
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    w = rope_frequencies(d, theta)
    phi = np.asarray(positions, dtype=np.float64)[:, None] * w[None, :]
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = a * c - b * s
    out[:, 1::2] = a * s + b * c
    return out


def attention_fp64(q, k, v, sm_scale):
    """Single-query softmax attention in fp64.

    q : [G, d] (G query heads sharing one KV head), k, v : [T, d].
    Returns [G, d] = softmax(sm_scale * q k^T) v, softmax with the maximum
    subtracted ([P1 para 6]: weighted sum of values by softmax scores).
    T == 0 returns zeros (no key to attend).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]))
    logits = sm_scale * (q @ k.T)                       # [G, T]
    logits = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def _dequant_unit(cache, b, h):
    """Dequantized keys (pre-RoPE) and values of one (batch, KV head) unit,
    quantized tokens first, then recent tokens, in fp64."""
    bits, d, T_q = cache["bits"], cache["d"], cache["T_q"]
    parts_k, parts_v = [], []
    if T_q > 0:
        kc = unpack_codes(cache["k_codes"][b, h], bits, d)[None, None]
        vc = unpack_v_codes(cache["v_codes"][b, h], bits, d)[None, None]
        parts_k.append(dequantize_k(kc, cache["k_scale"][b, h][None, None],
                                    cache["k_zero"][b, h][None, None])[0, 0])
        parts_v.append(dequantize_v(vc, cache["v_scale"][b, h][None, None],
                                    cache["v_zero"][b, h][None, None])[0, 0])
    if cache["R"] > 0:
        parts_k.append(cache["k_recent"][b, h].astype(np.float64))
        parts_v.append(cache["v_recent"][b, h].astype(np.float64))
    if not parts_k:
        return np.zeros((0, d)), np.zeros((0, d))
    return np.concatenate(parts_k), np.concatenate(parts_v)


def kivi_decode_attention(q16, cache, sm_scale, rows=None):
    """Decode attention over a KIVI-layout cache, read back from its packed
    buffers.

    q16   : float16 [B, Hq, d] (already rotated when RoPE is on)
    cache : dict with keys B, Hq, Hkv, d, bits, T_q, R, rope_theta (<= 0: no
            RoPE), k_codes (packed uint32 words [B, Hkv, T_q, d*bits/32],
            token-major), v_codes (uint32 [B, Hkv, T_q/32, d*bits], 32-token
            blocks stored channel-major), k_scale/k_zero (fp16 [B, Hkv,
            T_q/32, d]),
            v_scale/v_zero (fp16 [B, Hkv, T_q, d/32]), k_recent/v_recent
            (fp16 [B, Hkv, R, d], keys before RoPE).
    rows  : optional iterable of (b, hq) pairs; only those output rows are
            computed (the others stay NaN).
    Returns fp64 [B, Hq, d].
    """
    B, Hq, Hkv, d = cache["B"], cache["Hq"], cache["Hkv"], cache["d"]
    G = Hq // Hkv
    out = np.full((B, Hq, d), np.nan)
    if rows is None:
        rows = [(b, h) for b in range(B) for h in range(Hq)]
    by_unit = {}
    for b, hq in rows:
        by_unit.setdefault((b, hq // G), []).append(hq)
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    for (b, h), heads in sorted(by_unit.items()):
        k, v = _dequant_unit(cache, b, h)
        if cache["rope_theta"] > 0 and k.shape[0] > 0:
            k = rope_rotate(k, np.arange(k.shape[0]), cache["rope_theta"])
        o = attention_fp64(q[b, heads], k, v, sm_scale)
        out[b, heads] = o
    return out
