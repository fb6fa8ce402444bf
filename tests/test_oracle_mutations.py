"""Planted mistakes in the oracle (on the CPU) must each fail at least one
pin.  This shows the pins are sharp enough to catch a dropped term, a wrong
sign, a wrong axis or index, or a wrong rounding rule.  CPU only."""
import numpy as np
import pytest

import oracle
import oracle.attention as oatt
import oracle.quant as oq
import oracle.rvq as orvq
import oracle.zoned as oz
import test_oracle_attention as TA
import test_oracle_quant as TQ
import test_oracle_rvq as TR
import test_oracle_zoned as TZ
import test_oracle_stream as TS
import oracle.stream as ost
import oracle.rdkv as orr

_orig_qg = oq.quantize_groups


def _qg_variant(levels_fn=None, round_fn=np.rint, zero_fn=None, fp32_scale=False):
    def qg(x16, bits):
        x16 = np.asarray(x16, np.float16)
        L = np.float32(levels_fn(bits) if levels_fn else 2 ** bits - 1)
        x = x16.astype(np.float32)
        mn, mx = x.min(-1), x.max(-1)
        s32 = (mx - mn) / L
        s = s32.astype(np.float16)
        z = (zero_fn(mn, mx) if zero_fn else mn).astype(np.float16)
        sf = (s32 if fp32_scale else s.astype(np.float32))[..., None]
        zf = z.astype(np.float32)[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            t = (x - zf) / sf
        q = np.clip(round_fn(t), 0, L)
        q = np.where(sf == 0, 0, q)
        return q.astype(np.uint8), s, z
    return qg


def _half_away(t):
    return np.sign(t) * np.floor(np.abs(t) + 0.5)


QUANT_MUTANTS = {
    "levels_2^b": _qg_variant(levels_fn=lambda b: 2 ** b),
    "floor": _qg_variant(round_fn=np.floor),
    "round_half_away": _qg_variant(round_fn=_half_away),
    "zero_is_mean": _qg_variant(zero_fn=lambda mn, mx: (mn + mx) / 2),
    "codes_vs_fp32_scale": _qg_variant(fp32_scale=True),
}


def _run_quant_pins():
    for case in TQ._read_quant_cases():
        TQ.test_hand_fixtures(case)
    for bits in (2, 4, 8):
        TQ.test_levels_are_exactly_two_to_the_b(bits)
        TQ.test_error_at_most_half_scale(bits)
        TQ.test_codes_hit_both_ends(bits)


@pytest.mark.parametrize("name", sorted(QUANT_MUTANTS))
def test_quantizer_mutants_are_caught(monkeypatch, name):
    _run_quant_pins()                                    # clean oracle passes
    monkeypatch.setattr(TQ, "quantize_groups", QUANT_MUTANTS[name])
    with pytest.raises(AssertionError):
        _run_quant_pins()


def test_key_axis_mutant_is_caught(monkeypatch):
    # keys grouped along channels instead of tokens
    monkeypatch.setattr(TQ, "quantize_k", oq.quantize_v)
    monkeypatch.setattr(oracle, "dequantize_k", oq.dequantize_v)
    with pytest.raises(AssertionError):
        TQ.test_axis_pins_keys_per_channel_values_per_token()


def test_pack_order_mutant_is_caught(monkeypatch):
    def pack_msb_first(codes, bits):
        codes = np.asarray(codes)
        per = 32 // bits
        flat = codes.reshape(-1, per).astype(np.uint64)
        w = np.zeros(flat.shape[0], np.uint64)
        for j in range(per):
            w |= flat[:, j] << np.uint64((per - 1 - j) * bits)
        return w.astype(np.uint32).reshape(codes.shape[:-1] + (codes.shape[-1] * bits // 32,))
    monkeypatch.setattr(TQ, "pack_codes", pack_msb_first)
    with pytest.raises(AssertionError):
        for case in TQ._read_pack_cases():
            TQ.test_pack_hand_fixtures(case)


def test_rope_mutants_are_caught(monkeypatch):
    orig = oatt.rope_rotate

    def sign_flipped(x, positions, theta):
        return orig(x, -np.asarray(positions, np.float64), theta)

    def half_split(x, positions, theta):
        x = np.asarray(x, np.float64)
        T, d = x.shape
        w = oatt.rope_frequencies(d, theta)
        phi = np.asarray(positions, np.float64)[:, None] * w[None]
        a, b = x[:, :d // 2], x[:, d // 2:]
        return np.concatenate([a * np.cos(phi) - b * np.sin(phi), a * np.sin(phi) + b * np.cos(phi)], 1)

    for mutant in (sign_flipped, half_split):
        monkeypatch.setattr(TA, "rope_rotate", mutant)
        with pytest.raises(AssertionError):
            TA.test_rope_properties()


def test_attention_mutants_are_caught(monkeypatch):
    def no_scale(q, k, v, sm_scale):
        return oatt.attention_fp64.__wrapped__(q, k, v, 1.0) if hasattr(oatt.attention_fp64, "__wrapped__") else _attn(q, k, v, 1.0)

    def _attn(q, k, v, s):
        lg = s * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
        p = np.exp(lg - lg.max(1, keepdims=True))
        return (p / p.sum(1, keepdims=True)) @ np.asarray(v, np.float64)

    def transposed_weights(q, k, v, s):
        lg = s * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
        p = np.exp(lg - lg.max(1, keepdims=True))
        p = p / p.sum(1, keepdims=True)
        return p[:, ::-1] @ np.asarray(v, np.float64)

    for mutant in (no_scale, transposed_weights):
        monkeypatch.setattr(TA, "attention_fp64", mutant)
        with pytest.raises(AssertionError):
            TA.test_matches_library_sdpa()


def test_gqa_mapping_mutant_is_caught(monkeypatch):
    orig = oatt.kivi_decode_attention

    def modulo_mapping(q16, cache, sm_scale, rows=None):
        c = dict(cache)
        # query head h reads KV head h % Hkv instead of h // G
        B, Hq, Hkv = c["B"], c["Hq"], c["Hkv"]
        out = np.empty((B, Hq, c["d"]))
        for h in range(Hq):
            sub = dict(c, Hq=Hkv)
            qq = np.asarray(q16)[:, [h] * Hkv]
            out[:, h] = orig(qq, sub, sm_scale)[:, h % Hkv]
        return out

    monkeypatch.setattr(TA, "kivi_decode_attention", modulo_mapping)
    with pytest.raises(AssertionError):
        TA.test_gqa_head_mapping()


def test_rvq_mutants_are_caught(monkeypatch):
    orig_dist = orvq.rvq_stage_distances

    def plus_residual(x16, cbs, prefix=None):
        cbs = np.asarray(cbs, np.float16)
        r = np.asarray(x16, np.float16).astype(np.float32)
        idx = np.empty((r.shape[0], cbs.shape[0]), np.int64)
        for s in range(cbs.shape[0]):
            idx[:, s] = orig_dist(r, cbs[s]).argmin(1)
            r = r + cbs[s][idx[:, s]].astype(np.float32)      # wrong sign
        return idx.astype(np.int16), r

    def last_tie(x16, cbs, prefix=None):
        cbs = np.asarray(cbs, np.float16)
        r = np.asarray(x16, np.float16).astype(np.float32)
        idx = np.empty((r.shape[0], cbs.shape[0]), np.int64)
        for s in range(cbs.shape[0]):
            dd = orig_dist(r, cbs[s])
            idx[:, s] = dd.shape[1] - 1 - dd[:, ::-1].argmin(1)  # highest index on ties
            r = r - cbs[s][idx[:, s]].astype(np.float32)
        return idx.astype(np.int16), r

    monkeypatch.setattr(TR, "rvq_encode", plus_residual)
    with pytest.raises(AssertionError):
        TR.test_brute_force_nearest_tiny_codebooks()
    monkeypatch.setattr(TR, "rvq_encode", last_tie)
    with pytest.raises(AssertionError):
        TR.test_ties_go_to_lowest_index_small_integers()


def test_zoned_eviction_mutant_is_caught(monkeypatch):
    orig_layout = oz._unit_layout

    def keep_evicted(vb, kb, d, C, sink=0, k_out=0):
        vb = np.where(np.asarray(vb) == 0, 2, vb)         # width 0 kept at 2 bits
        return orig_layout(vb, kb, d, C, sink, k_out)

    monkeypatch.setattr(oz, "_unit_layout", keep_evicted)
    with pytest.raises(AssertionError):
        TZ.test_width_zero_is_eviction()


def test_stream_mutants_are_caught(monkeypatch):
    orig_append = ost.kivi_append

    def newest_first(state, k_new, v_new, bits, R_max):
        # quantizes the newest 32 tokens of the window instead of the oldest
        k_all = np.concatenate([state["k_recent"], np.asarray(k_new, np.float16)], axis=2)
        v_all = np.concatenate([state["v_recent"], np.asarray(v_new, np.float16)], axis=2)
        f = ost.flush_count(k_all.shape[2], R_max)
        n, R = f * 32, k_all.shape[2] - f * 32
        out = dict(state)
        if f:
            kc, ks, kz = oq.quantize_k(k_all[:, :, R:], bits)
            vc, vs, vz = oq.quantize_v(v_all[:, :, R:], bits)
            for name, x in [("k_codes", kc), ("k_scale", ks), ("k_zero", kz), ("v_codes", vc),
                            ("v_scale", vs), ("v_zero", vz)]:
                out[name] = np.concatenate([state[name], x], axis=2)
        out["k_recent"], out["v_recent"] = k_all[:, :, :R].copy(), v_all[:, :, :R].copy()
        return out

    def flush_at_bound(rows, R_max):
        f = 0
        while rows >= R_max and rows >= 32:         # flushes when the window is merely full
            rows -= 32
            f += 1
        return f

    monkeypatch.setattr(TS, "kivi_append", newest_first)
    with pytest.raises(AssertionError):
        TS.test_streaming_equals_batch_quantization(2, 128, 1)
    monkeypatch.setattr(TS, "kivi_append", orig_append)
    monkeypatch.setattr(ost, "flush_count", flush_at_bound)
    with pytest.raises(AssertionError):
        TS.test_hand_counted_flushes_one_token_at_a_time()


def _run_rdkv_pins():
    import test_oracle_rdkv as TK
    for name in dir(TK):
        if name.startswith("test_"):
            getattr(TK, name)()


def _token_weights_variant(axis=0, upper=False, modulo=False):
    def tw(q16, k16, sm_scale):
        q = np.asarray(q16, np.float16).astype(np.float64)
        k = np.asarray(k16, np.float16).astype(np.float64)
        B, Hq, T, d = q.shape
        Hkv = k.shape[1]
        G = Hq // Hkv
        w = np.zeros((B, Hkv, T))
        mask = np.tril(np.ones((T, T), bool))
        if upper:
            mask = mask.T
        for b in range(B):
            for h in range(Hq):
                kv = h % Hkv if modulo else h // G
                s = sm_scale * (q[b, h] @ k[b, kv].T)
                s = np.where(mask, s, -np.inf)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                w[b, kv] += p.sum(axis=axis)
        return w
    return tw


def _channel_weights_variant(per_head=False, no_keep=False, no_sqrt_d=False):
    def cw(q16, k16, keep):
        q = np.asarray(q16, np.float16).astype(np.float64)
        k = np.asarray(k16, np.float16).astype(np.float64)
        B, Hq, T, d = q.shape
        Hkv = k.shape[1]
        G = Hq // Hkv
        w = np.zeros((B, Hkv, d))
        for b in range(B):
            for h in range(Hkv):
                heads = slice(h * G, h * G + 1) if per_head else slice(h * G, (h + 1) * G)
                qn = np.sqrt((q[b, heads] ** 2).sum(axis=(0, 1)))
                kept = np.ones(T, bool) if no_keep else np.asarray(keep[b, h]) != 0
                kn = np.sqrt((k[b, h][kept] ** 2).sum(axis=0))
                w[b, h] = qn * kn / (1.0 if no_sqrt_d else np.sqrt(d))
        return w
    return cw


def _widths_at_ties_up(w, lam):
    w = np.asarray(w, np.float64)
    b = np.zeros(w.shape, np.int64)
    for f, inc in orr.BREAKPOINTS:
        b += inc * (lam <= w * f)
    return b.astype(np.int8)


def _multiplier_variant(pick):
    def mult(w, budget):
        w = np.asarray(w, np.float64).ravel()
        if np.any(~np.isfinite(w)) or np.any(w < 0) or budget < 0:
            raise ValueError("bad input")
        cands = np.unique(np.concatenate([[0.0]] + [w * f for f, _ in orr.BREAKPOINTS]))
        tot = np.array([orr.widths_at(w, c).astype(int).sum() for c in cands])
        return cands[pick(np.flatnonzero(tot <= budget))]
    return mult


RDKV_MUTANTS = {
    "row_sums": ("token_weights", _token_weights_variant(axis=1)),
    "anti_causal": ("token_weights", _token_weights_variant(upper=True)),
    "modulo_heads": ("token_weights", _token_weights_variant(modulo=True)),
    "one_head_query_norm": ("channel_weights", _channel_weights_variant(per_head=True)),
    "evicted_keys_counted": ("channel_weights", _channel_weights_variant(no_keep=True)),
    "no_sqrt_d": ("channel_weights", _channel_weights_variant(no_sqrt_d=True)),
    "ties_to_larger": ("widths_at", _widths_at_ties_up),
    "largest_fitting_multiplier": ("multiplier", _multiplier_variant(lambda ok: ok[-1])),
    "multiplier_one_step_low": ("multiplier", _multiplier_variant(lambda ok: max(ok[0] - 1, 0))),
}


@pytest.mark.parametrize("name", sorted(RDKV_MUTANTS))
def test_rdkv_mutants_are_caught(monkeypatch, name):
    _run_rdkv_pins()
    attr, fn = RDKV_MUTANTS[name]
    monkeypatch.setattr(orr, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    with pytest.raises(AssertionError):
        _run_rdkv_pins()


def _iso_variant(tie_low=False, stale_mean=False):
    def iso(x16, k_out):
        x = np.asarray(x16, np.float16).astype(np.float32)
        rem = list(range(len(x)))
        out = []
        for _ in range(k_out):
            if len(rem) <= 2:
                break
            xs = x[rem]
            if xs.min() == xs.max():
                break
            src = x if stale_mean else xs
            total = np.float32(0.0)
            for v in src:
                total = np.float32(total + v)
            mean = np.float32(total / np.float32(len(src)))
            hi = rem[int(np.argmax(xs))]
            lo = rem[int(np.argmin(xs))]
            d_hi, d_lo = abs(np.float32(x[hi] - mean)), abs(np.float32(x[lo] - mean))
            pick = (hi if d_hi > d_lo else lo) if tie_low else (hi if d_hi >= d_lo else lo)
            out.append(pick)
            rem.remove(pick)
        return sorted(out)
    return iso


def test_zoned_sink_and_outlier_mutants_are_caught(monkeypatch):
    for name, fn in (("ties_to_smallest", _iso_variant(tie_low=True)),
                     ("stale_mean", _iso_variant(stale_mean=True))):
        monkeypatch.setattr(oz, "isolate_outliers", fn)
        with pytest.raises(AssertionError):
            TZ.test_outlier_rule_hand_worked()
    monkeypatch.undo()
    orig_deq = oz._dequant_unit

    def no_replacement(k16u, v16u, vb, kb, lay):
        orig = oz._quantize_unit_keys

        def strip(k, l):
            return {w: [g[:5] + ([],) for g in gs] for w, gs in orig(k, l).items()}
        oz._quantize_unit_keys = strip
        try:
            return orig_deq(k16u, v16u, vb, kb, lay)
        finally:
            oz._quantize_unit_keys = orig

    monkeypatch.setattr(oz, "_dequant_unit", no_replacement)
    with pytest.raises(AssertionError):
        TZ.test_outlier_attention_and_layout()
    monkeypatch.undo()
    orig_layout = oz._unit_layout

    def sink_ignored(vb, kb, d, C, sink=0, k_out=0):
        return orig_layout(vb, kb, d, C, 0, k_out)          # sink tokens stay in the segments

    monkeypatch.setattr(oz, "_unit_layout", sink_ignored)
    with pytest.raises(AssertionError):
        TZ.test_sink_tokens_are_new_tokens_at_the_front()
