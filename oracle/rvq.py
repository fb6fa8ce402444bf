"""Oracle: residual vector quantization of cache vectors, and decode attention
over the reconstructed cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where it is defined ([P2 sec 2, key components]):

* RSimVQ, residual VQ: a cache vector is mapped to the nearest entry of a
  codebook; the residual (vector minus the chosen entry) is quantized by the
  next codebook; this repeats for N codebooks, so a vector is represented by
  N integer indices whose codewords add up to the reconstruction.
* at prefill only the indices are kept; during decoding the key/value
  vectors are rebuilt on demand inside the attention computation.

Readings: "nearest" is squared Euclidean distance; an exact distance tie
goes to the lowest index; the residual is kept in fp32 and updated with one
IEEE fp32 subtraction per element; distances are evaluated in fp64
(sum over channels of (r_i - c_i)^2), which is exact up to one rounding of
the final sum; the codeword dimension is the whole head vector; one set of
N codebooks for keys and one for values, shared across batch and heads.
"""

import numpy as np

from .attention import attention_fp64

_CHUNK = 32


def rvq_stage_distances(r32, cb16):
    """Squared Euclidean distances in fp64.

    r32  : float32 [m, d] residuals
    cb16 : float16 [Kc, d] one codebook
    Returns fp64 [m, Kc], entry (i, j) = sum_c (r[i, c] - cb[j, c])^2.
    """
    r = np.asarray(r32, np.float32).astype(np.float64)
    c = np.asarray(cb16, np.float16).astype(np.float64)
    out = np.empty((r.shape[0], c.shape[0]))
    for i0 in range(0, r.shape[0], _CHUNK):
        diff = r[i0:i0 + _CHUNK, None, :] - c[None, :, :]
        out[i0:i0 + _CHUNK] = np.sum(diff * diff, axis=2)
    return out


def rvq_encode(x16, codebooks16, prefix=None):
    """Greedy residual VQ encode ([P2 sec 2, RSimVQ steps 1-4]).

    x16         : float16 [n, d] vectors
    codebooks16 : float16 [N, Kc, d]
    prefix      : optional int array [n, p]: the first p stages use these
                  indices instead of searching (used to continue from
                  another encoder's choices after a documented tie).
    Returns (idx int16 [n, N], residual float32 [n, d] after the last stage).
    """
    x16 = np.asarray(x16, np.float16)
    cbs = np.asarray(codebooks16, np.float16)
    N = cbs.shape[0]
    n = x16.shape[0]
    r = x16.astype(np.float32)                      # exact widening
    idx = np.empty((n, N), np.int64)
    p = 0 if prefix is None else np.asarray(prefix).shape[1]
    for s in range(N):
        if s < p:
            idx[:, s] = np.asarray(prefix)[:, s]
        else:
            dist = rvq_stage_distances(r, cbs[s])
            idx[:, s] = np.argmin(dist, axis=1)     # first minimum = lowest index
        r = r - cbs[s][idx[:, s]].astype(np.float32)   # fp32 subtraction
    return idx.astype(np.int16), r


def rvq_reconstruct(idx, codebooks16):
    """Reconstruction = sum over stages of the indexed codewords, fp64
    ([P2 sec 2, RSimVQ step 4]).  idx int [..., N] -> fp64 [..., d]."""
    cbs = np.asarray(codebooks16, np.float16).astype(np.float64)
    idx = np.asarray(idx).astype(np.int64)
    out = np.zeros(idx.shape[:-1] + (cbs.shape[2],))
    for s in range(cbs.shape[0]):
        out += cbs[s][idx[..., s]]
    return out


def rvq_decode_attention(q16, k_idx, v_idx, k_cb16, v_cb16, sm_scale, rows=None):
    """Decode attention with keys and values rebuilt from their indices
    ([P2 sec 2, decoding phase]), fp64.

    q16 [B, Hq, d]; k_idx, v_idx int [B, Hkv, T, N]; k_cb16, v_cb16 fp16
    [N, Kc, d].  Query head h reads KV head h // (Hq/Hkv).
    """
    B, Hq, d = q16.shape
    Hkv = k_idx.shape[1]
    G = Hq // Hkv
    out = np.full((B, Hq, d), np.nan)
    if rows is None:
        rows = [(b, h) for b in range(B) for h in range(Hq)]
    by_unit = {}
    for b, hq in rows:
        by_unit.setdefault((b, hq // G), []).append(hq)
    q = np.asarray(q16, np.float16).astype(np.float64)
    for (b, h), heads in sorted(by_unit.items()):
        k = rvq_reconstruct(k_idx[b, h], k_cb16)
        v = rvq_reconstruct(v_idx[b, h], v_cb16)
        out[b, heads] = attention_fp64(q[b, heads], k, v, sm_scale)
    return out
