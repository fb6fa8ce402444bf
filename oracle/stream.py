"""Oracle: streaming append to a uniform-layout (KIVI) cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[P1 para 8, residual buffer]: per-channel key statistics depend on tokens
that have not been generated yet, so the newest tokens are kept in full
precision (a window of up to 128 of them) and quantized in groups once
enough of them have been collected.

Reading fixed here (the page gives no algorithm): new tokens join the
full-precision window after the tokens already in it; then, while the
window holds more than R_max tokens and at least one whole group (32), its
oldest 32 tokens are quantized as one key group per channel and one value
group per token and 32 channels -- exactly as ``quantize_k`` /
``quantize_v`` quantize those 32 tokens -- and appended after the tokens
already quantized.  The window keeps the rest in order.

Parity: pinned by tests/test_oracle_stream.py (streaming equals batch
quantization of the same tokens, window bounds and token accounting, a
hand-counted flush sequence, attention unchanged by the chunking).
"""

import numpy as np

from .quant import GROUP, quantize_k, quantize_v


def empty_stream(B, H, d):
    """A cache with no tokens: unpacked codes uint8 and fp16 scale/zero, as
    ``quantize_k`` / ``quantize_v`` return them, plus the fp16 window."""
    z8 = np.zeros((B, H, 0, d), np.uint8)
    return dict(k_codes=z8, k_scale=np.zeros((B, H, 0, d), np.float16),
                k_zero=np.zeros((B, H, 0, d), np.float16),
                v_codes=z8.copy(), v_scale=np.zeros((B, H, 0, d // GROUP), np.float16),
                v_zero=np.zeros((B, H, 0, d // GROUP), np.float16),
                k_recent=np.zeros((B, H, 0, d), np.float16),
                v_recent=np.zeros((B, H, 0, d), np.float16))


def flush_count(rows, R_max):
    """Groups quantized when ``rows`` tokens sit in the window."""
    f = 0
    while rows > R_max and rows >= GROUP:
        rows -= GROUP
        f += 1
    return f


def kivi_append(state, k_new, v_new, bits, R_max):
    """Append fp16 tokens [B, H, n, d] (keys before RoPE) to ``state`` (a dict
    from :func:`empty_stream` or an earlier call) and flush whole groups as
    the reading above says.  Returns the new state; the input is not
    modified."""
    k_all = np.concatenate([state["k_recent"], np.asarray(k_new, np.float16)], axis=2)
    v_all = np.concatenate([state["v_recent"], np.asarray(v_new, np.float16)], axis=2)
    f = flush_count(k_all.shape[2], R_max)
    out = dict(state)
    if f > 0:
        n = f * GROUP
        kc, ks, kz = quantize_k(k_all[:, :, :n], bits)
        vc, vs, vz = quantize_v(v_all[:, :, :n], bits)
        out["k_codes"] = np.concatenate([state["k_codes"], kc], axis=2)
        out["k_scale"] = np.concatenate([state["k_scale"], ks], axis=2)
        out["k_zero"] = np.concatenate([state["k_zero"], kz], axis=2)
        out["v_codes"] = np.concatenate([state["v_codes"], vc], axis=2)
        out["v_scale"] = np.concatenate([state["v_scale"], vs], axis=2)
        out["v_zero"] = np.concatenate([state["v_zero"], vz], axis=2)
    out["k_recent"] = k_all[:, :, f * GROUP:].copy()
    out["v_recent"] = v_all[:, :, f * GROUP:].copy()
    return out
