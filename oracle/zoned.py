"""Oracle: mixed-bitwidth ("TriZone") cache layout and decode attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages define ([P3 sec 2.2, bit-allocation pipeline] and [P3 sec 2.2,
TriZone packed decoding]):

* bit widths come from the set {0, 2, 4, 8, 16}; width 0 means the unit is
  evicted.  Values get a width per token; keys get a width per channel, for
  the tokens that were kept, independently of the token's value width
  ([P3 sec 2.1]: a key channel's weight is the logit deviation caused by
  zeroing that channel, so an evicted key channel is a zeroed one).
* zone A holds the packed old cache -- key rows and the kept value rows at 2,
  4 or 8 bits -- grouped by width so that each group dequantizes uniformly;
  zone B holds the fp16 value rows of 16-bit tokens; zone C holds fp16 keys
  and values of newly generated tokens.
* the attention kernel combines the three zones with dequantization fused
  into the products.

Readings (the pages give neither formulas nor byte layouts); all of them are
listed here:

* a token whose value width is 0 is dropped together with its key.
* a key channel whose width is 0 is not stored: the kept old tokens' keys
  read 0 in that channel.  The new tokens of zone C keep every channel
  (the widths are assigned to the cache present after prefill).
* kept tokens are partitioned by value width into four segments, in the
  order 2, 4, 8, 16, keeping token order inside a segment; each segment is
  cut into groups of 32 slots, the last group padded with masked slots.
* key channels are partitioned by key width into classes in the order
  2, 4, 8, 16 (channel order kept inside a class); each (group, quantized
  channel) is one quantization group over the group's valid slots, at the
  channel's width, with the scale/zero rule of ``quant.quantize_groups``;
  16-bit key channels are stored as raw fp16.
* value rows at width 2/4/8 are quantized per token in 32-channel groups
  (as in the uniform layout); 16-bit value rows go to zone B as raw fp16.
* sink window ([P1 para 11]: high-precision windows for the attention sinks
  as well as the recent tokens): the first S old tokens are kept whole --
  fp16 keys and values over every channel -- whatever their widths; they
  open zone C, before the new tokens.  S = 0 is the layout above.
* outlier side list ([P1 para 9]: a small share of outliers isolated from
  the quantized keys): in every key quantization group up to k_out entries
  are taken out, one at a time -- the group's smallest or largest remaining
  value, whichever lies farther from the float32 mean of the remaining
  values (summed in slot order; the largest on a tie, the lowest slot among
  equal values) -- stopping while only two values remain or all remaining
  values are equal.  The group is quantized over the remaining values; a
  removed entry keeps code 0 in the dense codes and its fp16 value in the
  side list, and dequantizes to that value exactly.  k_out = 0 is the layout
  above.

Byte layout of the blob (little endian), one region per (batch, KV head)
unit in batch-major order, each region starting at a multiple of 256 bytes:

* zone A: the groups of segment 2, then 4, then 8, then 16.  A group of
  segment w holds, each block starting at a multiple of 16 bytes:
  key codes [32 slots][W_K words]; key scales [n_kq] fp16; key zeros [n_kq]
  fp16; and for w < 16 also value codes [32][d*w/32 words], value scales
  [32][d/32] fp16 and value zeros [32][d/32] fp16.
  A key row is the concatenation of one block per key class: class w in
  {2, 4, 8} packs its channels' codes LSB first into ceil(m_w*w/32) words;
  class 16 stores its channels' fp16 bit patterns two per word
  (ceil(m_16/2) words).  n_kq = m_2 + m_4 + m_8 and the scale/zero arrays
  follow the class order.  Value codes use the flat LSB-first stream of
  ``quant.pack_codes``.  Masked slots hold zero bits everywhere.
  With k_out > 0 every group also holds, after the key zeros, its side
  list: slot offsets [33] uint16 (the entries of slot s are entries
  offs[s] .. offs[s+1]-1), then the entries' class-ordered channel positions
  [n_kq * k_out] uint16, then their fp16 values [n_kq * k_out], each block
  16-byte aligned; entries are sorted by slot, then channel position; unused
  entries are zero.
* zone B: [P_16 slots][d] fp16 value rows of the 16-bit segment (masked
  slots zero), where P_w is the segment's padded slot count.
* zone C: keys [S + C][d] fp16, then values [S + C][d] fp16: the S sink
  tokens, then the new tokens.
"""

import numpy as np

from .quant import GROUP, quantize_groups, quantize_v, dequantize_v, pack_codes

WIDTHS = (0, 2, 4, 8, 16)
SEGMENT_WIDTHS = (2, 4, 8, 16)
KEY_WIDTHS = (2, 4, 8, 16)
UNIT_ALIGN = 256
BLOCK_ALIGN = 16


def _pad(n, a):
    return (n + a - 1) // a * a


OUT_OFFS = GROUP + 1          # slot offsets of a side list


def _unit_layout(vb, kb, d, C, sink=0, k_out=0):
    """Sizes and offsets (bytes, relative to the unit start) of one unit."""
    vb = np.asarray(vb)
    past_sink = np.arange(len(vb)) >= sink
    seg_tokens = {w: np.flatnonzero((vb == w) & past_sink) for w in SEGMENT_WIDTHS}
    classes = {w: np.flatnonzero(kb == w) for w in KEY_WIDTHS}
    m = {w: len(classes[w]) for w in KEY_WIDTHS}
    kwords = {w: (m[w] * w + 31) // 32 for w in KEY_WIDTHS}
    W_K = sum(kwords.values())
    n_kq = m[2] + m[4] + m[8]
    k_codes_b = GROUP * W_K * 4
    k_sz_b = _pad(n_kq * 2, BLOCK_ALIGN)
    n_cap = n_kq * k_out
    out_b = (_pad(OUT_OFFS * 2, BLOCK_ALIGN) + 2 * _pad(n_cap * 2, BLOCK_ALIGN)) if k_out else 0
    group_bytes = {}
    for w in SEGMENT_WIDTHS:
        gb = k_codes_b + 2 * k_sz_b + out_b
        if w < 16:
            gb += GROUP * (d * w // 32) * 4 + 2 * _pad(GROUP * (d // 32) * 2, BLOCK_ALIGN)
        group_bytes[w] = gb
    off = 0
    seg = {}
    for w in SEGMENT_WIDTHS:
        n = len(seg_tokens[w])
        P = _pad(n, GROUP)
        seg[w] = dict(tokens=seg_tokens[w], n=n, P=P, groups=P // GROUP,
                      offset=off, group_bytes=group_bytes[w])
        off += (P // GROUP) * group_bytes[w]
    zone_b = off
    off += seg[16]["P"] * d * 2
    zone_c = off
    off += 2 * (sink + C) * d * 2
    return dict(seg=seg, classes=classes, m=m, kwords=kwords, W_K=W_K,
                n_kq=n_kq, k_codes_bytes=k_codes_b, k_sz_bytes=k_sz_b,
                k_out=k_out, n_out_cap=n_cap, out_bytes=out_b, sink=sink,
                zone_b=zone_b, zone_c=zone_c, size=_pad(off, UNIT_ALIGN))


def zoned_layout(v_bits, k_bits, d, C, sink=0, k_out=0):
    """Layout of every unit.

    v_bits : int array [B, Hkv, T_old] with values in {0, 2, 4, 8, 16}
    k_bits : int array [B, Hkv, d] with values in {0, 2, 4, 8, 16} (0: the
             channel is evicted and not stored)
    Returns (list of per-unit layout dicts with an added 'base' byte offset,
    total blob size in bytes).
    """
    v_bits = np.asarray(v_bits)
    k_bits = np.asarray(k_bits)
    B, H, _ = v_bits.shape
    units, base = [], 0
    for b in range(B):
        for h in range(H):
            lay = _unit_layout(v_bits[b, h], k_bits[b, h], d, C, sink, k_out)
            lay["base"] = base
            base += lay["size"]
            units.append(lay)
    return units, base


def isolate_outliers(x16, k_out):
    """Slots (ascending) taken out of one key quantization group: x16 fp16
    [n] holds the group's valid values in slot order.  See the module
    docstring for the rule."""
    x = np.asarray(x16, np.float16).astype(np.float32)
    rem = list(range(len(x)))
    out = []
    for _ in range(k_out):
        if len(rem) <= 2:
            break
        xs = x[rem]
        if xs.min() == xs.max():
            break
        total = np.float32(0.0)
        for v in xs:                                    # slot order, float32
            total = np.float32(total + v)
        mean = np.float32(total / np.float32(len(rem)))
        hi = rem[int(np.argmax(xs))]                    # first (lowest) slot
        lo = rem[int(np.argmin(xs))]
        d_hi = abs(np.float32(x[hi] - mean))
        d_lo = abs(np.float32(x[lo] - mean))
        pick = hi if d_hi >= d_lo else lo
        out.append(pick)
        rem.remove(pick)
    return sorted(out)


def _quantize_channel(x16, bits, k_out):
    """One key quantization group with its outliers taken out: (codes uint8
    [n], scale fp16, zero fp16, removed slots)."""
    out = isolate_outliers(x16, k_out) if k_out else []
    keep = np.setdiff1d(np.arange(len(x16)), out)
    cq, sc, z = quantize_groups(np.asarray(x16, np.float16)[keep][None], bits)
    codes = np.zeros(len(x16), np.uint8)
    codes[keep] = cq[0]
    return codes, sc[0], z[0], out


def _quantize_unit_keys(k16u, lay):
    """Per (segment, group, quantized channel) key quantization of one unit.

    Returns {w: list over groups of (codes uint8 [n_valid, n_kq] in class
    order, scale fp16 [n_kq], zero fp16 [n_kq], raw16 fp16 [n_valid, m_16],
    token indices [n_valid], outliers: list of (slot, class position, fp16
    value) sorted by slot then position)}.
    """
    raw_chan = lay["classes"][16]
    k_out = lay.get("k_out", 0)
    out = {}
    for w in SEGMENT_WIDTHS:
        toks = lay["seg"][w]["tokens"]
        groups = []
        for g in range(lay["seg"][w]["groups"]):
            t = toks[g * GROUP:(g + 1) * GROUP]
            x = k16u[t]                                     # [n_valid, d]
            cs, ss, zs, outl = [], [], [], []
            pc0 = 0
            for cw in (2, 4, 8):
                chans = lay["classes"][cw]
                if k_out == 0:
                    # one quantization group per channel of the class: the
                    # channel's values over the group's valid slots
                    cq, s, z = quantize_groups(x[:, chans].T, cw)
                    cs.append(cq.T)
                    ss.append(s)
                    zs.append(z)
                else:
                    cq = np.zeros((len(t), len(chans)), np.uint8)
                    s = np.zeros(len(chans), np.float16)
                    z = np.zeros(len(chans), np.float16)
                    for i, ch in enumerate(chans):
                        cq[:, i], s[i], z[i], rem = _quantize_channel(x[:, ch], cw, k_out)
                        outl += [(slot, pc0 + i, x[slot, ch]) for slot in rem]
                    cs.append(cq)
                    ss.append(s)
                    zs.append(z)
                pc0 += len(chans)
            codes = np.concatenate(cs, axis=1).astype(np.uint8)
            scale = np.concatenate(ss).astype(np.float16)
            zero = np.concatenate(zs).astype(np.float16)
            outl.sort(key=lambda e: (e[0], e[1]))
            groups.append((codes, scale, zero, x[:, raw_chan], t, outl))
        out[w] = groups
    return out


def _dequant_unit(k16u, v16u, vb, kb, lay):
    """Dequantized (fp64) keys and values of the kept old tokens of one unit
    (sink tokens excluded), segment by segment, in slot order."""
    d = k16u.shape[1]
    qchan = np.concatenate([lay["classes"][w] for w in (2, 4, 8)]).astype(np.int64)
    raw_chan = lay["classes"][16]
    kq = _quantize_unit_keys(k16u, lay)
    ks, vs = [], []
    for w in SEGMENT_WIDTHS:
        for codes, scale, zero, raw, t, outl in kq[w]:
            kh = np.zeros((len(t), d))                      # evicted key channels read 0
            kh[:, qchan] = codes * scale.astype(np.float64) + zero.astype(np.float64)
            kh[:, raw_chan] = raw.astype(np.float64)
            for slot, pc, val in outl:                      # side-list entries are exact
                kh[slot, qchan[pc]] = float(val)
            ks.append(kh)
            if w < 16:
                vc, vsc, vz = quantize_v(v16u[t][None, None], w)
                vs.append(dequantize_v(vc, vsc, vz)[0, 0])
            else:
                vs.append(v16u[t].astype(np.float64))
    if not ks:
        return np.zeros((0, d)), np.zeros((0, d))
    return np.concatenate(ks), np.concatenate(vs)


def zoned_decode_attention(q16, k16, v16, v_bits, k_bits, k_new, v_new,
                           sm_scale, rows=None, sink=0, k_out=0):
    """Decode attention over the mixed-width cache, fp64, computed from the
    dequantized values (independently of the byte layout).

    q16 [B, Hq, d]; k16, v16 [B, Hkv, T_old, d]; v_bits [B, Hkv, T_old];
    k_bits [B, Hkv, d]; k_new, v_new [B, Hkv, C, d] (zone C, fp16).
    Keys attended: the sink tokens (fp16), the kept old tokens
    (dequantized), then the C new tokens.
    """
    from .attention import attention_fp64
    B, Hq, d = q16.shape
    Hkv = k16.shape[1]
    C = k_new.shape[2]
    G = Hq // Hkv
    out = np.full((B, Hq, d), np.nan)
    if rows is None:
        rows = [(b, h) for b in range(B) for h in range(Hq)]
    by_unit = {}
    for b, hq in rows:
        by_unit.setdefault((b, hq // G), []).append(hq)
    q = np.asarray(q16, np.float16).astype(np.float64)
    for (b, h), heads in sorted(by_unit.items()):
        lay = _unit_layout(v_bits[b, h], k_bits[b, h], d, C, sink, k_out)
        k, v = _dequant_unit(k16[b, h], v16[b, h], v_bits[b, h], k_bits[b, h], lay)
        k = np.concatenate([np.asarray(k16[b, h][:sink], np.float64), k, k_new[b, h].astype(np.float64)])
        v = np.concatenate([np.asarray(v16[b, h][:sink], np.float64), v, v_new[b, h].astype(np.float64)])
        out[b, heads] = attention_fp64(q[b, heads], k, v, sm_scale)
    return out


def _pack_key_rows(codes, raw, lay):
    """Key rows [n_valid, W_K] uint32 from class-ordered codes and raw fp16."""
    n = codes.shape[0]
    rows = np.zeros((n, lay["W_K"]), np.uint32)
    col, cc = 0, 0
    for w in (2, 4, 8):
        mw, nw = lay["m"][w], lay["kwords"][w]
        if mw:
            pad = nw * 32 // w - mw
            c = np.concatenate([codes[:, cc:cc + mw], np.zeros((n, pad), np.uint8)], axis=1)
            rows[:, col:col + nw] = pack_codes(c, w)
        col += nw
        cc += mw
    m16, n16 = lay["m"][16], lay["kwords"][16]
    if m16:
        bitsu16 = raw.view(np.uint16).astype(np.uint32)
        if m16 % 2:
            bitsu16 = np.concatenate([bitsu16, np.zeros((n, 1), np.uint32)], axis=1)
        rows[:, col:col + n16] = bitsu16[:, 0::2] | (bitsu16[:, 1::2] << np.uint32(16))
    return rows


def zoned_pack(k16, v16, v_bits, k_bits, k_new, v_new, sink=0, k_out=0):
    """Byte image (uint8 array) of the packed mixed-width cache, following
    the layout in the module docstring."""
    k16 = np.asarray(k16, np.float16)
    v16 = np.asarray(v16, np.float16)
    B, H, T, d = k16.shape
    C = k_new.shape[2]
    units, total = zoned_layout(v_bits, k_bits, d, C, sink, k_out)
    blob = np.zeros(total, np.uint8)

    def put(off, arr):
        b = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        blob[off:off + b.size] = b

    for u, lay in enumerate(units):
        b, h = divmod(u, H)
        base = lay["base"]
        kq = _quantize_unit_keys(k16[b, h], lay)
        for w in SEGMENT_WIDTHS:
            sg = lay["seg"][w]
            for g, (codes, scale, zero, raw, t, outl) in enumerate(kq[w]):
                go = base + sg["offset"] + g * sg["group_bytes"]
                rows = np.zeros((GROUP, lay["W_K"]), np.uint32)
                rows[:len(t)] = _pack_key_rows(codes, raw, lay)
                put(go, rows)
                o = go + lay["k_codes_bytes"]
                put(o, scale)
                o += lay["k_sz_bytes"]
                put(o, zero)
                o += lay["k_sz_bytes"]
                if k_out:
                    cap = lay["n_out_cap"]
                    offs = np.zeros(OUT_OFFS, np.uint16)
                    for slot, _, _ in outl:
                        offs[slot + 1:] += 1
                    pcs = np.zeros(cap, np.uint16)
                    vals = np.zeros(cap, np.float16)
                    for i, (slot, pc, val) in enumerate(outl):
                        pcs[i] = pc
                        vals[i] = val
                    put(o, offs)
                    o += _pad(OUT_OFFS * 2, BLOCK_ALIGN)
                    put(o, pcs)
                    o += _pad(cap * 2, BLOCK_ALIGN)
                    put(o, vals)
                    o += _pad(cap * 2, BLOCK_ALIGN)
                if w < 16:
                    vc, vsc, vz = quantize_v(v16[b, h][t][None, None], w)
                    vrows = np.zeros((GROUP, d * w // 32), np.uint32)
                    vrows[:len(t)] = pack_codes(vc[0, 0], w)
                    put(o, vrows)
                    o += GROUP * (d * w // 32) * 4
                    vs_full = np.zeros((GROUP, d // 32), np.float16)
                    vz_full = np.zeros((GROUP, d // 32), np.float16)
                    vs_full[:len(t)] = vsc[0, 0]
                    vz_full[:len(t)] = vz[0, 0]
                    put(o, vs_full)
                    o += _pad(GROUP * (d // 32) * 2, BLOCK_ALIGN)
                    put(o, vz_full)
        zb = np.zeros((lay["seg"][16]["P"], d), np.float16)
        zb[:lay["seg"][16]["n"]] = v16[b, h][lay["seg"][16]["tokens"]]
        put(base + lay["zone_b"], zb)
        zck = np.concatenate([k16[b, h][:sink], np.asarray(k_new[b, h], np.float16)])
        zcv = np.concatenate([v16[b, h][:sink], np.asarray(v_new[b, h], np.float16)])
        put(base + lay["zone_c"], zck)
        put(base + lay["zone_c"] + (sink + C) * d * 2, zcv)
    return blob
