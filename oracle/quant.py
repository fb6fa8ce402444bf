"""Oracle: asymmetric uniform integer quantization of the KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where it is defined:

* [P1 para 3, uniform integer quantization]: the value range of a group is
  divided into the levels the format can represent (2 bits -> 4 levels).
* [P1 para 1]: every group carries its own scale factor and zero point;
  groups hold 32 elements.
* [P1 para 4] keys are grouped per channel (a group = one channel over 32
  tokens); [P1 para 5] values are grouped per token (a group = one token
  over 32 channels).

Readings fixed here (the pages give no formula):

* scale  s = (max - min) / (2^b - 1), computed in fp32 and stored as fp16
  (round to nearest even); zero  z = min, stored as fp16 (exact, since the
  minimum is itself an fp16 value).
* codes are formed against the *stored* fp16 scale and zero:
  ``q = clamp(rint((x - z) / s), 0, 2^b - 1)`` with IEEE fp32 subtraction
  and division, rint = round half to even.  A group whose stored scale is 0
  (constant group) gets all-zero codes.
* dequantized value  x_hat = q * s + z.
* packing: a sequence of codes forms one little-endian bit stream; element
  f occupies bits [f*b, f*b + b), i.e. word f*b // 32, bit (f*b) % 32.  32 is
  a multiple of every supported width so no code straddles a word.  Keys
  are packed in row-major [token][channel] order.  Values are packed in
  blocks of 32 tokens, channel-major inside a block: block k holds, for
  channel 0, 1, ..., d-1 in turn, the codes of tokens 32k..32k+31.
"""

import numpy as np

GROUP = 32


def quantize_groups(x16, bits):
    """Quantize the last axis of ``x16`` as independent groups.

    Parameters
    ----------
    x16 : float16 array, shape [..., n] (n = 32 everywhere except the
          partially filled last group of a mixed-width segment)
    bits : int in {2, 4, 8}

    Returns
    -------
    codes : uint8 array [..., n]
    scale : float16 array [...]
    zero  : float16 array [...]

    Follows [P1 para 3] (range split into 2^b levels) and [P1 para 1]
    (scale factor and zero point per group).  Parity: pinned by
    tests/test_oracle_quant.py (four levels at 2 bits, constant-group round
    trip, |x - x_hat| <= s/2, nearest-level brute force, hand fixtures).
    """
    x16 = np.asarray(x16, dtype=np.float16)
    assert x16.shape[-1] >= 1
    levels = np.float32(2 ** bits - 1)
    x = x16.astype(np.float32)                       # exact widening
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    s32 = (mx - mn) / levels                         # fp32 sub, fp32 div
    scale = s32.astype(np.float16)                   # RNE to fp16
    zero = mn.astype(np.float16)                     # exact
    sf = scale.astype(np.float32)[..., None]
    zf = zero.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (x - zf) / sf                            # fp32 sub, fp32 div
    q = np.clip(np.rint(t), np.float32(0), levels)
    q = np.where(sf == 0, np.float32(0), q)
    return q.astype(np.uint8), scale, zero


def quantize_k(k16, bits):
    """Per-channel key quantization [P1 para 4]: each (channel, 32-token block)
    is a group.

    k16 : float16 [B, H, T, d], T a multiple of 32 (keys before RoPE, [P1 para 7]).
    Returns codes uint8 [B, H, T, d], scale/zero float16 [B, H, T/32, d].
    """
    k16 = np.asarray(k16, dtype=np.float16)
    B, H, T, d = k16.shape
    assert T % GROUP == 0
    g = k16.reshape(B, H, T // GROUP, GROUP, d).transpose(0, 1, 2, 4, 3)
    codes, scale, zero = quantize_groups(g, bits)     # [B,H,T/32,d,32]
    codes = codes.transpose(0, 1, 2, 4, 3).reshape(B, H, T, d)
    return codes, scale, zero


def quantize_v(v16, bits):
    """Per-token value quantization [P1 para 5]: each (token, 32-channel block)
    is a group.

    v16 : float16 [B, H, T, d], d a multiple of 32.
    Returns codes uint8 [B, H, T, d], scale/zero float16 [B, H, T, d/32].
    """
    v16 = np.asarray(v16, dtype=np.float16)
    B, H, T, d = v16.shape
    assert d % GROUP == 0
    g = v16.reshape(B, H, T, d // GROUP, GROUP)
    codes, scale, zero = quantize_groups(g, bits)     # [B,H,T,d/32,32]
    return codes.reshape(B, H, T, d), scale, zero


def dequantize_k(codes, scale, zero):
    """x_hat = q * s + z in fp64 (exact for fp16 s, z and q < 256), with the
    per-channel (32-token block) parameters of :func:`quantize_k`."""
    B, H, T, d = codes.shape
    s = np.repeat(scale.astype(np.float64), GROUP, axis=2)
    z = np.repeat(zero.astype(np.float64), GROUP, axis=2)
    return codes.astype(np.float64) * s + z


def dequantize_v(codes, scale, zero):
    """x_hat = q * s + z in fp64 with the per-token (32-channel block)
    parameters of :func:`quantize_v`."""
    s = np.repeat(scale.astype(np.float64), GROUP, axis=-1)
    z = np.repeat(zero.astype(np.float64), GROUP, axis=-1)
    return codes.astype(np.float64) * s + z


def pack_codes(codes, bits):
    """Pack codes (any shape, row-major order) into a little-endian uint32
    bit stream, element f at bits [f*bits, f*bits + bits).

    Returns uint32 array of shape codes.shape[:-1] + (codes.shape[-1]*bits//32,).
    """
    codes = np.asarray(codes)
    per_word = 32 // bits
    assert codes.shape[-1] * bits % 32 == 0
    flat = codes.reshape(-1, per_word).astype(np.uint64)
    words = np.zeros(flat.shape[0], dtype=np.uint64)
    for j in range(per_word):
        words |= flat[:, j] << np.uint64(j * bits)
    out_shape = codes.shape[:-1] + (codes.shape[-1] * bits // 32,)
    return words.astype(np.uint32).reshape(out_shape)


def pack_v_codes(codes, bits):
    """Value codes [B, H, T, d] (T a multiple of 32) -> words [B, H, T/32,
    d*bits]: each 32-token block is stored channel-major (for each channel,
    its 32 tokens' codes in token order), as one bit stream."""
    codes = np.asarray(codes)
    B, H, T, d = codes.shape
    assert T % GROUP == 0
    blocks = codes.reshape(B, H, T // GROUP, GROUP, d).transpose(0, 1, 2, 4, 3)
    return pack_codes(blocks.reshape(B, H, T // GROUP, d * GROUP), bits)


def unpack_v_codes(words, bits, d):
    """Inverse of :func:`pack_v_codes`: words [..., T/32, d*bits] -> codes
    [..., T, d]."""
    words = np.asarray(words, dtype=np.uint32)
    lead = words.shape[:-2]
    nb = words.shape[-2]
    c = unpack_codes(words, bits, d * GROUP).reshape(lead + (nb, d, GROUP))
    return np.swapaxes(c, -1, -2).reshape(lead + (nb * GROUP, d))


def unpack_codes(words, bits, last_dim):
    """Inverse of :func:`pack_codes`: words [..., last_dim*bits/32] -> uint8
    codes [..., last_dim]."""
    words = np.asarray(words, dtype=np.uint32)
    per_word = 32 // bits
    mask = np.uint32(2 ** bits - 1)
    flat = words.reshape(-1)
    out = np.empty((flat.shape[0], per_word), dtype=np.uint8)
    for j in range(per_word):
        out[:, j] = ((flat >> np.uint32(j * bits)) & mask).astype(np.uint8)
    return out.reshape(words.shape[:-1] + (last_dim,))
