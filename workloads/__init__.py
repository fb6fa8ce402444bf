"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and casts them; it holds none of the
quantization or attention arithmetic.  Every array is produced by
``numpy.random.default_rng(seed)``; draws are float32 normal samples (or
categorical choices) cast to fp16 with round-to-nearest-even, in a fixed
order: query, keys, values, outlier channels, outlier factors, width maps,
codebooks.

The five workloads stand in for the model caches the pages measure on
(Llama-2-13B, Llama-3.1-8B, Llama-3.2-3B shapes; no weights, no datasets).
The bit allocator reads the prefill of the mixed-width cache: queries of
every position and keys (``rdkv_inputs``, same draw order without values).
Outlier channels imitate the stable high-magnitude key channels described
in [P1 para 3] ([P1] = ihal.it/?p=61653, KV-cache quantization axes).
"""

import numpy as np

CONFIGS = {
    # tiny correctness case: one head, 256 quantized tokens, 2 fixed outlier
    # key channels scaled x50
    "tiny-kivi": dict(workload="tiny-kivi", seed=1, kind="kivi", B=1, Hq=1, Hkv=1, d=64,
               T_q=256, R=0, bits=(2,), rope_theta=0.0,
               outliers=("fixed", (5, 37), 50.0)),
    # Llama-2-13B-shaped layer: MHA, 4096 tokens, 4% outlier key channels
    "llama2-13b-decode-layer": dict(workload="llama2-13b-decode-layer", seed=2, kind="kivi", B=8, Hq=40,
               Hkv=40, d=128, T_q=4096, R=0, bits=(2,), rope_theta=0.0,
               outliers=("lognormal", 0.04, 3.0, 1.0)),
    # Llama-3.1-8B-shaped GQA decode: 32k quantized tokens + 128 fp16 recent
    # tokens, RoPE theta 5e5 applied to the dequantized pre-RoPE keys
    "llama3.1-8b-gqa-32k": dict(workload="llama3.1-8b-gqa-32k", seed=3, kind="kivi", B=4, Hq=32,
               Hkv=8, d=128, T_q=32768, R=128, bits=(2, 4),
               rope_theta=500000.0, outliers=("lognormal", 0.04, 3.0, 1.0)),
    # mixed-width zoned cache: 16384 old tokens + 64 new fp16 tokens
    "mixed-width-zoned-16k": dict(workload="mixed-width-zoned-16k", seed=4, kind="zoned", B=2, Hq=32,
               Hkv=8, d=128, T_old=16384, C=64,
               v_width_probs={0: 0.5, 2: 0.2, 4: 0.15, 8: 0.1, 16: 0.05},
               k_width_probs={2: 0.4, 4: 0.3, 8: 0.2, 16: 0.1},
               outliers=("lognormal", 0.04, 3.0, 1.0),
               # mean widths of the maps above (value bits per token, key bits
               # per channel): the budgets of the allocator on this cache
               rdkv_mean_widths=(2.6, 5.2),
               # sink window and key outlier side lists measured beside the
               # plain layout: 4 sink tokens, one entry per key group
               zoned_variant=dict(sink=4, k_out=1)),
    # residual-VQ cache, Llama-3.2-3B shape: 4 codebooks x 1024 entries
    "rvq-llama3.2-3b-8k": dict(workload="rvq-llama3.2-3b-8k", seed=5, kind="rvq", B=2, Hq=24, Hkv=8,
               d=128, T=8192, N=4, Kc=1024),
}


def _outlier_keys(rng, k32, spec):
    """Scale selected key channels in place (float32 [B, H, T, d])."""
    B, H, T, d = k32.shape
    if spec is None:
        return
    if spec[0] == "fixed":
        _, chans, factor = spec
        for c in chans:
            if c < d:
                k32[..., c] *= np.float32(factor)
        return
    _, frac, mu, sigma = spec
    n_out = max(1, int(round(frac * d)))
    chans = np.stack([rng.choice(d, size=n_out, replace=False) for _ in range(H)])
    factors = rng.lognormal(mean=mu, sigma=sigma, size=(H, n_out)).astype(np.float32)
    for h in range(H):
        for j in range(n_out):
            k32[:, h, :, chans[h, j]] *= factors[h, j]


def _normal16(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32).astype(np.float16)


def kivi_inputs(B, Hq, Hkv, d, T_q, R, seed, outliers=None):
    """Query [B, Hq, d] and keys/values [B, Hkv, T_q + R, d] (fp16); the last R
    tokens form the fp16 recent zone.  Keys are pre-RoPE."""
    rng = np.random.default_rng(seed)
    q = _normal16(rng, (B, Hq, d))
    k32 = rng.standard_normal(size=(B, Hkv, T_q + R, d), dtype=np.float32)
    v = _normal16(rng, (B, Hkv, T_q + R, d))
    _outlier_keys(rng, k32, outliers)
    k = k32.astype(np.float16)
    del k32
    return dict(q=q, k=k[:, :, :T_q].copy(), v=v[:, :, :T_q].copy(),
                k_recent=k[:, :, T_q:].copy(), v_recent=v[:, :, T_q:].copy())


def zoned_inputs(B, Hq, Hkv, d, T_old, C, seed, v_width_probs, k_width_probs,
                 outliers=None):
    """Query, old keys/values [B, Hkv, T_old, d], per-token value widths
    [B, Hkv, T_old], per-channel key widths [B, Hkv, d] and C new tokens."""
    rng = np.random.default_rng(seed)
    q = _normal16(rng, (B, Hq, d))
    k32 = rng.standard_normal(size=(B, Hkv, T_old + C, d), dtype=np.float32)
    v = _normal16(rng, (B, Hkv, T_old + C, d))
    _outlier_keys(rng, k32, outliers)
    k = k32.astype(np.float16)
    del k32
    vw = np.array(sorted(v_width_probs))
    kw = np.array(sorted(k_width_probs))
    v_bits = rng.choice(vw, size=(B, Hkv, T_old),
                        p=[v_width_probs[w] for w in vw]).astype(np.int8)
    k_bits = rng.choice(kw, size=(B, Hkv, d),
                        p=[k_width_probs[w] for w in kw]).astype(np.int8)
    return dict(q=q, k=k[:, :, :T_old].copy(), v=v[:, :, :T_old].copy(),
                k_new=k[:, :, T_old:].copy(), v_new=v[:, :, T_old:].copy(),
                v_bits=v_bits, k_bits=k_bits)


def rdkv_inputs(B, Hq, Hkv, d, T, seed, outliers=None):
    """Prefill queries [B, Hq, T, d] (every position) and keys [B, Hkv, T, d]
    (fp16), keys with the outlier channels of ``outliers``."""
    rng = np.random.default_rng(seed)
    q = _normal16(rng, (B, Hq, T, d))
    k32 = rng.standard_normal(size=(B, Hkv, T, d), dtype=np.float32)
    _outlier_keys(rng, k32, outliers)
    k = k32.astype(np.float16)
    del k32
    return dict(q=q, k=k)


def rvq_inputs(B, Hq, Hkv, d, T, N, Kc, seed):
    """Query, keys/values [B, Hkv, T, d] ~ N(0, 1) and two codebook sets
    (keys, values) [N, Kc, d] whose stage n is drawn N(0, 0.5^n) (variance)."""
    rng = np.random.default_rng(seed)
    q = _normal16(rng, (B, Hq, d))
    k = _normal16(rng, (B, Hkv, T, d))
    v = _normal16(rng, (B, Hkv, T, d))
    cbs = []
    for _ in range(2):
        stages = [(rng.standard_normal(size=(Kc, d), dtype=np.float32)
                   * np.float32(np.sqrt(0.5 ** n))).astype(np.float16)
                  for n in range(N)]
        cbs.append(np.stack(stages))
    return dict(q=q, k=k, v=v, k_cb=cbs[0], v_cb=cbs[1])


def config_inputs(name, seed=None):
    """Inputs of a named workload; the seed defaults to the workload's own."""
    cfg = CONFIGS[name]
    seed = cfg["seed"] if seed is None else seed
    if cfg["kind"] == "kivi":
        return kivi_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T_q"],
                           cfg["R"], seed, cfg["outliers"])
    if cfg["kind"] == "zoned":
        return zoned_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"],
                            cfg["T_old"], cfg["C"], seed, cfg["v_width_probs"],
                            cfg["k_width_probs"], cfg["outliers"])
    return rvq_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T"],
                      cfg["N"], cfg["Kc"], seed)
