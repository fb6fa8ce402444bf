"""C-ABI library checks that need no GPU: every function declared in
include/dqattn.h is exported, and invalid arguments are rejected by host
validation (before any HIP call) with the documented status."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import dequant_decode_attention_amd as dqa
from dequant_decode_attention_amd import lib, KiviCacheStruct

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "dqattn.h")
FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: validation rejects first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["quantize_pack_k", "quantize_pack_v", "decode_attention_qkv", "rvq_encode",
              "rvq_decode_attention", "zoned_plan", "zoned_pack", "decode_attention_zoned",
              "dqa_status_string", "kivi_append", "rdkv_token_weights", "rdkv_channel_weights",
              "rdkv_allocate", "rdkv_widths"]:
        assert n in names


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", dqa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    for n in _declared():
        getattr(lib, n)


def test_status_strings():
    for s in range(9):
        assert lib.dqa_status_string(s).startswith(b"DQA_")
    assert lib.dqa_status_string(8).startswith(b"DQA_ERR_ALIGN")
    assert lib.dqa_status_string(99) == b"DQA_ERR_UNKNOWN"
    assert lib.dqa_abi_version() >= 1


@pytest.mark.parametrize("fn", ["quantize_pack_k", "quantize_pack_v"])
def test_quantize_validation(fn):
    f = getattr(lib, fn)
    assert f(FAKE, 1, 1, 32, 96, 2, FAKE, FAKE, FAKE, None) == 2          # d
    assert f(FAKE, 1, 1, 32, 128, 3, FAKE, FAKE, FAKE, None) == 3         # bits
    assert f(FAKE, 1, 1, 32, 128, 16, FAKE, FAKE, FAKE, None) == 3
    assert f(None, 1, 1, 32, 128, 2, FAKE, FAKE, FAKE, None) == 1         # null
    assert f(FAKE, 1, 1, 32, 128, 2, FAKE, None, FAKE, None) == 1
    assert f(FAKE, -1, 1, 32, 128, 2, FAKE, FAKE, FAKE, None) == 2
    assert f(None, 0, 4, 32, 128, 2, None, None, None, None) == 0         # empty: no work
    odd2, odd4 = ctypes.c_void_p(0x1002), ctypes.c_void_p(0x1004)
    assert f(odd2, 1, 1, 32, 128, 2, FAKE, FAKE, FAKE, None) == 8         # 16-byte alignment
    assert f(FAKE, 1, 1, 32, 128, 2, odd4, FAKE, FAKE, None) == 8
    if fn == "quantize_pack_k":
        assert f(FAKE, 1, 1, 33, 128, 2, FAKE, FAKE, FAKE, None) == 2     # T % 32


def _cache(**kw):
    base = dict(B=2, Hq=8, Hkv=2, d=128, bits=2, T_q=64, R=16, rope_theta=0.0,
                k_codes=0x1000, k_scale=0x1000, k_zero=0x1000, v_codes=0x1000,
                v_scale=0x1000, v_zero=0x1000, k_recent=0x1000, v_recent=0x1000, T_cap=0, R_cap=0,
                rope_table=None)
    base.update(kw)
    return KiviCacheStruct(*[base[n] for n, _ in KiviCacheStruct._fields_])


def test_decode_workspace_query_and_validation():
    ws = lib.decode_attention_workspace_bytes(ctypes.byref(_cache()))
    # merge counters first: one uint32 per (batch, KV head), at least 16384
    counters = 16384 * 4
    # 3 tiles per (batch, KV head): a single split, no partial states
    assert ws == counters
    # 128 + 1 tiles over 4 units: 33 splits of partial states [m, l, o[d]] per head
    big = lib.decode_attention_workspace_bytes(ctypes.byref(_cache(T_q=4096)))
    assert big == counters + 4 * 33 * 4 * (128 + 2) * 4
    # more than 16384 units: one counter each, rounded up to 256 bytes
    many = lib.decode_attention_workspace_bytes(ctypes.byref(_cache(B=5000, Hkv=4, Hq=16)))
    assert many == (5000 * 4 * 4 + 255) // 256 * 256
    for bad, code in [(dict(d=96), 2), (dict(bits=3), 3), (dict(T_q=40), 2), (dict(R=129), 2),
                      (dict(Hq=6, Hkv=4), 2), (dict(Hq=24, Hkv=2), 5), (dict(Hq=16, Hkv=2), 5),
                      (dict(k_codes=None), 1), (dict(k_recent=None), 1)]:
        c = _cache(**bad)
        st = lib.decode_attention_qkv(FAKE, ctypes.byref(c), 0.1, FAKE, 1 << 30, FAKE, None)
        assert st == code, (bad, st)
    c = _cache()
    assert lib.decode_attention_qkv(None, ctypes.byref(c), 0.1, FAKE, 1 << 30, FAKE, None) == 1
    assert lib.decode_attention_qkv(FAKE, ctypes.byref(c), 0.1, None, 1 << 30, FAKE, None) == 4
    assert lib.decode_attention_qkv(FAKE, ctypes.byref(c), 0.1, FAKE, ws - 1, FAKE, None) == 4
    # every device pointer must be 16-byte aligned (checked before any launch)
    odd = ctypes.c_void_p(0x1008)
    assert lib.decode_attention_qkv(odd, ctypes.byref(c), 0.1, FAKE, 1 << 30, FAKE, None) == 8
    assert lib.decode_attention_qkv(FAKE, ctypes.byref(c), 0.1, FAKE, 1 << 30, odd, None) == 8
    for name in ["k_codes", "v_scale", "v_recent", "rope_table"]:
        c2 = _cache(**{name: 0x1004}, rope_theta=1e4)
        assert lib.decode_attention_qkv(FAKE, ctypes.byref(c2), 0.1, FAKE, 1 << 30, FAKE, None) == 8
    # the recent-zone pointers are not used (nor checked) without recent tokens
    c3 = _cache(R=0, k_recent=0x1002, v_recent=None)
    assert lib.decode_attention_qkv(FAKE, ctypes.byref(c3), 0.1, None, 1 << 30, FAKE, None) == 4
    # buffer capacities: 0 means dense; else at least the tokens in use, and
    # the quantized capacity a multiple of 32
    for bad in [dict(T_cap=32), dict(T_cap=96 + 8), dict(T_cap=-32), dict(R_cap=8), dict(R_cap=-1)]:
        c4 = _cache(**bad)
        assert lib.decode_attention_qkv(FAKE, ctypes.byref(c4), 0.1, FAKE, 1 << 30, FAKE, None) == 2, bad
        assert lib.decode_attention_workspace_bytes(ctypes.byref(c4)) == 0, bad
    assert lib.decode_attention_workspace_bytes(ctypes.byref(_cache(T_cap=4096, R_cap=128))) == ws
    # the merge phase validates its own arguments
    assert lib.decode_attention_qkv_merge(ctypes.byref(c), FAKE, 1 << 30, None, None) == 1
    assert lib.decode_attention_qkv_merge(ctypes.byref(c), None, 1 << 30, FAKE, None) == 4
    assert lib.decode_attention_qkv_merge(ctypes.byref(c), FAKE, ws - 1, FAKE, None) == 4
    assert lib.decode_attention_qkv_merge(ctypes.byref(c), FAKE, 1 << 30, odd, None) == 8
    assert lib.decode_attention_qkv_merge(ctypes.byref(_cache(bits=3)), FAKE, 1 << 30, FAKE, None) == 3
    assert lib.decode_attention_qkv_partial(None, ctypes.byref(c), 0.1, FAKE, 1 << 30, FAKE, None) == 1
    assert lib.decode_attention_workspace_bytes(ctypes.byref(_cache(d=80))) == 0
    assert lib.decode_attention_workspace_bytes(None) == 0


def test_rope_table_validation():
    assert lib.kivi_rope_table_words(128) == 4 + 2 * 32 * 64 + 2 * 64
    assert lib.kivi_rope_table_words(64) == 4 + 2 * 32 * 32 + 2 * 32
    assert lib.kivi_rope_table_words(96) == 0
    f = lib.kivi_rope_table
    assert f(1e4, 128, 2, None, None) == 1
    assert f(0.0, 128, 2, FAKE, None) == 2          # no RoPE
    assert f(-1.0, 128, 2, FAKE, None) == 2
    assert f(1e4, 80, 2, FAKE, None) == 2
    assert f(1e4, 128, 8, FAKE, None) == 3          # the table serves the 2- and 4-bit kernel
    assert f(1e4, 128, 3, FAKE, None) == 3
    assert f(1e4, 128, 4, ctypes.c_void_p(0x1004), None) == 8


def test_noalloc_decode_validation():
    """The allocation-free decode rejects, before any HIP call, a shape whose
    partial states exceed the library's array, and validates like the
    workspace variant."""
    scratch = lib.decode_attention_noalloc_scratch_bytes()
    assert scratch == 2 << 20
    f = lib.decode_attention_qkv_noalloc
    assert f(FAKE, ctypes.byref(_cache(d=96)), 0.1, FAKE, None) == 2
    assert f(FAKE, ctypes.byref(_cache(bits=3)), 0.1, FAKE, None) == 3
    # grow the batch until the partial states no longer fit the array
    B = 1
    while lib.decode_attention_workspace_bytes(ctypes.byref(_cache(B=B, Hkv=8, Hq=32, T_q=256, R=0))) <= scratch:
        B += 1
        assert B < 4096
    assert f(FAKE, ctypes.byref(_cache(B=B, Hkv=8, Hq=32, T_q=256, R=0)), 0.1, FAKE, None) == 4
    assert f(None, ctypes.byref(_cache(B=0)), 0.1, None, None) == 0      # empty: nothing to do


def test_stream_copy_validation():
    assert lib.dqa_stream_copy(FAKE, None, 64, None) == 1
    assert lib.dqa_stream_copy(FAKE, FAKE, 20, None) == 2
    assert lib.dqa_stream_copy(ctypes.c_void_p(0x1008), FAKE, 64, None) == 2


def _plan(vb, kb, C, d, sink=0, k_out=0):
    vb = np.ascontiguousarray(vb, np.int8)
    kb = np.ascontiguousarray(kb, np.int8)
    B, H, T = vb.shape
    n = lib.zoned_plan_words(B, H, T, d)
    words = np.zeros(n, np.int32)
    blob = ctypes.c_size_t(0)
    st = lib.zoned_plan(ctypes.c_void_p(vb.ctypes.data), ctypes.c_void_p(kb.ctypes.data), B, H, T,
                        C, d, sink, k_out, ctypes.c_void_p(words.ctypes.data), n, ctypes.byref(blob))
    return st, words, blob.value


@pytest.mark.parametrize("seed,T,C,d,sink,k_out", [(0, 500, 64, 128, 0, 0), (1, 77, 0, 64, 0, 0),
                                                   (2, 1, 3, 128, 0, 0), (3, 0, 5, 64, 0, 0),
                                                   (4, 300, 16, 128, 4, 1), (5, 90, 0, 64, 90, 2),
                                                   (6, 200, 8, 128, 0, 4)])
def test_zoned_plan_matches_oracle_layout(seed, T, C, d, sink, k_out):
    """The host planner (C++) and the oracle's layout agree on the blob size
    (and hence on every segment/zone size) for random width maps."""
    import oracle
    rng = np.random.default_rng(seed)
    B, H = 2, 3
    vb = rng.choice([0, 2, 4, 8, 16], size=(B, H, T), p=[.5, .2, .15, .1, .05]).astype(np.int8)
    kb = rng.choice([2, 4, 8, 16], size=(B, H, d), p=[.4, .3, .2, .1]).astype(np.int8)
    st, words, blob = _plan(vb, kb, C, d, sink, k_out)
    assert st == 0
    _, total = oracle.zoned_layout(vb, kb, d, C, sink, k_out)
    assert blob == total
    ws = lib.decode_attention_zoned_workspace_bytes(ctypes.c_void_p(words.ctypes.data), 4 * H)
    assert ws > 0


def test_zoned_plan_validation():
    vb = np.full((1, 1, 64), 2, np.int8)
    kb = np.full((1, 1, 128), 4, np.int8)
    assert _plan(vb, kb, 0, 128)[0] == 0
    bad_v = vb.copy()
    bad_v[0, 0, 5] = 3
    assert _plan(bad_v, kb, 0, 128)[0] == 3
    bad_k = kb.copy()
    bad_k[0, 0, 1] = 3              # not a width of the set
    assert _plan(vb, bad_k, 0, 128)[0] == 3
    evict_k = kb.copy()
    evict_k[0, 0, 1] = 0            # width 0 evicts a key channel
    assert _plan(vb, evict_k, 0, 128)[0] == 0
    assert _plan(vb, kb, 300, 128)[0] == 2                  # C too large
    assert _plan(vb, kb, 200, 128, sink=60)[0] == 2         # sink + C too large
    assert _plan(vb, kb, 0, 128, sink=65)[0] == 2           # sink longer than the cache
    assert _plan(vb, kb, 0, 128, sink=-1)[0] == 2
    assert _plan(vb, kb, 0, 128, k_out=5)[0] == 2           # side list too long
    assert _plan(vb, kb, 0, 128, k_out=-1)[0] == 2
    assert _plan(vb, kb, 0, 128, sink=64, k_out=4)[0] == 0
    assert lib.zoned_plan_words(1, 1, 64, 96) == 0
    n = lib.zoned_plan_words(1, 1, 64, 128)
    words = np.zeros(n, np.int32)
    blob = ctypes.c_size_t(0)
    assert lib.zoned_plan(ctypes.c_void_p(vb.ctypes.data), ctypes.c_void_p(kb.ctypes.data), 1, 1,
                          64, 0, 128, 0, 0, ctypes.c_void_p(words.ctypes.data), n - 1,
                          ctypes.byref(blob)) == 4
    # a corrupted plan is refused by the device entry points before any launch
    st, words, blob = _plan(vb, kb, 0, 128)
    words[0] ^= 1
    assert lib.zoned_pack(ctypes.c_void_p(words.ctypes.data), FAKE, FAKE, FAKE, None, None, FAKE,
                          None) == 7
    assert lib.decode_attention_zoned(FAKE, 4, ctypes.c_void_p(words.ctypes.data), FAKE, FAKE,
                                      0.1, FAKE, 1 << 20, FAKE, None) == 7
    st, words, blob = _plan(vb, kb, 0, 128)
    assert lib.decode_attention_zoned(FAKE, 3, ctypes.c_void_p(words.ctypes.data), FAKE, FAKE,
                                      0.1, FAKE, 1 << 20, FAKE, None) == 5   # ratio 3 not built
    assert lib.decode_attention_zoned(FAKE, 4, ctypes.c_void_p(words.ctypes.data), FAKE, FAKE,
                                      0.1, FAKE, 16, FAKE, None) == 4
    odd = ctypes.c_void_p(0x1008)
    for blob_p, ws_p, out_p in ((odd, FAKE, FAKE), (FAKE, odd, FAKE), (FAKE, FAKE, odd)):
        assert lib.decode_attention_zoned(FAKE, 4, ctypes.c_void_p(words.ctypes.data), FAKE, blob_p,
                                          0.1, ws_p, 1 << 20, out_p, None) == 8


# plan word indices (header and unit record), as zoned.hip lays them out
H_BLOB_LO, H_MAX_GROUPS, H_UNIT_OFF, H_PERM_OFF, H_TOK_OFF = 8, 10, 11, 12, 13
U_N, U_M, U_SEG_OFF, U_SIZE, U_TOK_PREFIX = 0, 4, 20, 32, 34
UNIT_WORDS = 40


def _corruptions(words, units, d, T):
    """(name, corrupted copy, token-map-only) for a valid plan."""
    u1 = 16 + UNIT_WORDS          # record of unit 1
    perm0, tok0 = words[H_PERM_OFF], words[H_TOK_OFF]
    out = []

    def mod(name, fn, tok_only=False):
        w = words.copy()
        fn(w)
        out.append((name, w, tok_only))

    mod("truncated (last unit's record and tables zeroed)",
        lambda w: w.__setitem__(slice(16 + (units - 1) * UNIT_WORDS, None), 0))
    mod("unit record offset", lambda w: w.__setitem__(H_UNIT_OFF, 17))
    mod("permutation offset", lambda w: w.__setitem__(H_PERM_OFF, perm0 + 1))
    mod("token map offset", lambda w: w.__setitem__(H_TOK_OFF, tok0 - 1))
    mod("max groups", lambda w: w.__setitem__(H_MAX_GROUPS, w[H_MAX_GROUPS] + 1))
    mod("blob size", lambda w: w.__setitem__(H_BLOB_LO, w[H_BLOB_LO] + 256))
    mod("unit size", lambda w: w.__setitem__(u1 + U_SIZE, w[u1 + U_SIZE] + 256))
    mod("segment offset", lambda w: w.__setitem__(u1 + U_SEG_OFF + 1, w[u1 + U_SEG_OFF + 1] + 16))
    mod("kept tokens beyond T_old", lambda w: w.__setitem__(u1 + U_N, T + 1))
    mod("negative channel count", lambda w: w.__setitem__(u1 + U_M, -1))
    mod("channels beyond d", lambda w: w.__setitem__(u1 + U_M + 3, d + 1))
    mod("token-map prefix", lambda w: w.__setitem__(u1 + U_TOK_PREFIX + 1, w[u1 + U_TOK_PREFIX + 1] + 1))
    mod("unused record word", lambda w: w.__setitem__(u1 + 39, 5))
    mod("channel listed twice", lambda w: w.__setitem__(perm0 + d + 1, w[perm0 + d]))
    mod("channel out of range", lambda w: w.__setitem__(perm0 + 2, d))
    return out


@pytest.mark.parametrize("sink,k_out", [(0, 0), (3, 2)])
def test_zoned_plan_corruption_refused(sink, k_out):
    """A plan zoned_plan could not have written is refused (DQA_ERR_PLAN)
    by every entry point that reads it, before any launch: truncated plans,
    shifted offsets, records that disagree with their own counts, a wrong
    blob size, a broken channel permutation.  (The token map is not read on
    the host; the packer clamps its entries into range.)"""
    rng = np.random.default_rng(9)
    B, H, T, d = 2, 3, 100, 128
    vb = rng.choice([0, 2, 4, 8, 16], size=(B, H, T), p=[.3, .3, .2, .1, .1]).astype(np.int8)
    kb = rng.choice([2, 4, 8, 16], size=(B, H, d), p=[.4, .3, .2, .1]).astype(np.int8)
    st, words, blob = _plan(vb, kb, 8, d, sink, k_out)
    assert st == 0
    ptr = lambda w: ctypes.c_void_p(w.ctypes.data)
    assert lib.decode_attention_zoned_workspace_bytes(ptr(words), 4 * H) > 0
    for name, w, tok_only in _corruptions(words, B * H, d, T):
        assert lib.zoned_pack(ptr(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 7, name
        if tok_only:
            continue
        assert lib.decode_attention_zoned_workspace_bytes(ptr(w), 4 * H) == 0, name
        assert lib.decode_attention_zoned(FAKE, 4 * H, ptr(w), FAKE, FAKE, 0.1, FAKE, 1 << 30, FAKE,
                                          None) == 7, name


def test_rvq_validation_and_workspace():
    assert lib.rvq_encode_workspace_bytes(4, 1024) == 4 * 1024 * 4
    assert lib.rvq_encode_workspace_bytes(9, 1024) == 0
    assert lib.rvq_encode_workspace_bytes(4, 1000) == 0          # Kc % 64
    ws = 1 << 20
    assert lib.rvq_encode(FAKE, 10, 64, FAKE, 4, 1024, FAKE, FAKE, ws, None) == 2   # d
    assert lib.rvq_encode(FAKE, 10, 128, FAKE, 0, 1024, FAKE, FAKE, ws, None) == 2  # N
    assert lib.rvq_encode(FAKE, 10, 128, FAKE, 4, 32, FAKE, FAKE, ws, None) == 2    # Kc
    assert lib.rvq_encode(None, 10, 128, FAKE, 4, 1024, FAKE, FAKE, ws, None) == 1
    assert lib.rvq_encode(FAKE, 10, 128, FAKE, 4, 1024, FAKE, FAKE, 100, None) == 4
    assert lib.rvq_encode(None, 0, 128, None, 4, 1024, None, None, 0, None) == 0    # empty
    odd = ctypes.c_void_p(0x1004)
    assert lib.rvq_encode(odd, 10, 128, FAKE, 4, 1024, FAKE, FAKE, ws, None) == 8     # alignment
    assert lib.rvq_encode(FAKE, 10, 128, odd, 4, 1024, FAKE, FAKE, ws, None) == 8
    assert lib.rvq_encode(FAKE, 10, 128, FAKE, 4, 1024, FAKE, odd, ws, None) == 8
    w = lib.rvq_decode_attention_workspace_bytes(2, 24, 8, 8192, 128)
    assert w > 16 * 65536                     # room for a 64 KB key-logit table per unit
    assert lib.rvq_decode_attention_workspace_bytes(2, 24, 8, 8192, 64) == 0
    assert lib.rvq_decode_attention_workspace_bytes(2, 40, 8, 8192, 128) == 5 - 5   # ratio 5
    args = lambda **k: [k.get(n, v) for n, v in [
        ("q", FAKE), ("B", 2), ("Hq", 24), ("Hkv", 8), ("T", 100), ("d", 128), ("ki", FAKE),
        ("vi", FAKE), ("kc", FAKE), ("vc", FAKE), ("N", 4), ("Kc", 1024), ("sc", 0.1),
        ("ws", FAKE), ("wsb", w), ("out", FAKE), ("st", None)]]
    assert lib.rvq_decode_attention(*args(Hq=40)) == 5
    assert lib.rvq_decode_attention(*args(N=9)) == 2
    assert lib.rvq_decode_attention(*args(ki=None)) == 1
    assert lib.rvq_decode_attention(*args(wsb=16)) == 4
    assert lib.rvq_decode_attention(*args(q=ctypes.c_void_p(0x1002))) == 8
    assert lib.rvq_decode_attention(*args(vc=ctypes.c_void_p(0x1008))) == 8


def test_kivi_append_validation():
    """Argument checks of the streaming append (all fail before any launch)."""
    assert lib.dqa_abi_version() == 14
    c = _cache(T_cap=128, R_cap=128)
    # staging holds the recent and the new rows of K and V
    assert lib.kivi_append_workspace_bytes(ctypes.byref(c), 20) == 2 * 2 * 2 * (16 + 20) * 128 * 2
    assert lib.kivi_append_workspace_bytes(ctypes.byref(_cache(d=96)), 1) == 0
    assert lib.kivi_append_workspace_bytes(ctypes.byref(c), -1) == 0
    ws = 1 << 30

    def call(cache, n_new=20, R_max=16, k=FAKE, v=FAKE, w=FAKE, wb=ws):
        before = (cache.T_q, cache.R)
        st = lib.kivi_append(ctypes.byref(cache), k, v, n_new, R_max, w, wb, None)
        assert (cache.T_q, cache.R) == before or st == 0
        return st

    assert call(_cache(T_cap=128, R_cap=128), R_max=129) == 2
    assert call(_cache(T_cap=128, R_cap=128), R_max=-1) == 2
    assert call(_cache(bits=3, T_cap=128, R_cap=128)) == 3
    # 16 + 20 rows over R_max = 16: one group of 32 goes to quantized position 64
    assert call(_cache(T_cap=64, R_cap=128)) == 2              # no room for the group
    assert call(_cache(T_cap=0, R_cap=128)) == 2               # dense buffers have no room
    assert call(_cache(T_cap=128, R_cap=2), R_max=0) == 2       # 4 rows stay, recent buffer holds 2
    assert call(_cache(T_cap=128, R_cap=128), k=None) == 1
    assert call(_cache(T_cap=128, R_cap=128, k_recent=None)) == 1
    assert call(_cache(T_cap=128, R_cap=128, v_codes=None)) == 1
    assert call(_cache(T_cap=128, R_cap=128), w=None) == 4
    assert call(_cache(T_cap=128, R_cap=128), wb=100) == 4
    assert call(_cache(T_cap=128, R_cap=128), k=ctypes.c_void_p(0x1008)) == 8
    assert call(_cache(T_cap=128, R_cap=128, k_zero=0x1002)) == 8
    # nothing to do: counts unchanged, no launch
    c0 = _cache(R=0, T_cap=128, R_cap=128)
    assert lib.kivi_append(ctypes.byref(c0), None, None, 0, 16, None, 0, None) == 0
    assert (c0.T_q, c0.R) == (64, 0)
    c1 = _cache(B=0, T_cap=128, R_cap=128)
    assert lib.kivi_append(ctypes.byref(c1), FAKE, FAKE, 40, 16, None, 0, None) == 0
    assert (c1.T_q, c1.R) == (64 + 32, 16 + 40 - 32)
    # a capacity of 0 means the current count; the call writes back the
    # capacity it used, so the recent rows keep their stride when R shrinks
    c2 = _cache(B=0, T_q=64, R=40, T_cap=96, R_cap=0)
    assert lib.kivi_append(ctypes.byref(c2), None, None, 0, 8, None, 0, None) == 0
    assert (c2.T_q, c2.R, c2.T_cap, c2.R_cap) == (96, 8, 96, 40)
    c3 = _cache(B=0, T_q=64, R=16, T_cap=0, R_cap=0)
    assert lib.kivi_append(ctypes.byref(c3), None, None, 0, 16, None, 0, None) == 0
    assert (c3.T_q, c3.R, c3.T_cap, c3.R_cap) == (64, 16, 64, 16)
    # a failed call leaves the capacities as they were
    c4 = _cache(B=0, T_q=64, R=40, T_cap=0, R_cap=0)
    assert lib.kivi_append(ctypes.byref(c4), None, None, 0, 8, None, 0, None) == 2
    assert (c4.T_q, c4.R, c4.T_cap, c4.R_cap) == (64, 40, 0, 0)


def test_rdkv_validation():
    """Argument checks of the RDKV allocation entry points (all fail before
    any launch)."""
    assert lib.rdkv_token_weights_workspace_bytes(2, 32, 1000) == 256 * ((2 * 32 * 1000 * 4 + 255) // 256)
    tw = lambda **k: lib.rdkv_token_weights(*[k.get(n, v) for n, v in [
        ("q", FAKE), ("k", FAKE), ("B", 2), ("Hq", 8), ("Hkv", 2), ("T", 100), ("d", 128),
        ("sc", 0.1), ("w", FAKE), ("ws", FAKE), ("wsb", 1 << 20), ("st", None)]])
    assert tw(d=96) == 5
    assert tw(Hq=6, Hkv=4) == 2
    assert tw(sc=0.0) == 2
    assert tw(sc=-1.0) == 2
    assert tw(sc=float("nan")) == 2
    assert tw(q=None) == 1
    assert tw(w=None) == 1
    assert tw(k=ctypes.c_void_p(0x1008)) == 8
    assert tw(wsb=100) == 4
    assert tw(ws=None) == 4
    assert tw(T=0, q=None, k=None, w=None) == 0            # empty: no work
    assert tw(B=0, q=None, k=None, w=None) == 0
    assert tw(B=40000, Hkv=2) == 2                          # B * Hkv above a grid dimension
    cw = lambda **k: lib.rdkv_channel_weights(*[k.get(n, v) for n, v in [
        ("q", FAKE), ("k", FAKE), ("keep", FAKE), ("B", 2), ("Hq", 8), ("Hkv", 2), ("T", 100),
        ("d", 64), ("w", FAKE), ("ws", FAKE), ("wsb", 1 << 20), ("st", None)]])
    assert lib.rdkv_channel_weights_workspace_bytes(2, 2, 100, 64) == 256 * ((1 * 2 * 2 * 2 * 64 * 4 + 255) // 256)
    assert lib.rdkv_channel_weights_workspace_bytes(2, 2, 100, 96) == 0
    assert cw(keep=None) == 1
    assert cw(d=32) == 5
    assert cw(wsb=16) == 4
    assert cw(k=ctypes.c_void_p(0x1004)) == 8
    al = lambda **k: lib.rdkv_allocate(*[k.get(n, v) for n, v in [
        ("w", FAKE), ("rows", 2), ("n", 5000), ("bud", 100), ("out", FAKE), ("ws", FAKE),
        ("wsb", 1 << 20), ("st", None)]])
    # per row state (32 bytes) then 2048-bin histograms per 4096-weight chunk
    assert lib.rdkv_allocate_workspace_bytes(2, 5000) == 256 + 2 * 2 * 2048 * 4
    assert al(bud=-1) == 2
    assert al(rows=70000) == 2
    assert al(n=-1) == 2
    assert al(w=None) == 1
    assert al(out=None) == 1
    assert al(wsb=256) == 4
    assert al(rows=0, w=None, out=None, ws=None) == 0
    assert al(n=0, w=None, out=None, ws=None) == 0
    wd = lambda **k: lib.rdkv_widths(*[k.get(n, v) for n, v in [
        ("q", FAKE), ("k", FAKE), ("B", 2), ("Hq", 8), ("Hkv", 2), ("T", 100), ("d", 128),
        ("sc", 0.1), ("vb", 300), ("kb", 300), ("v", FAKE), ("kbits", FAKE), ("ws", FAKE),
        ("wsb", 1 << 30), ("st", None)]])
    need = lib.rdkv_widths_workspace_bytes(2, 8, 2, 100, 128)
    assert need > lib.rdkv_token_weights_workspace_bytes(2, 8, 100)
    assert lib.rdkv_widths_workspace_bytes(2, 8, 2, 100, 80) == 0
    assert wd(vb=-1) == 2
    assert wd(kb=-1) == 2
    assert wd(v=None) == 1
    assert wd(kbits=None) == 1
    assert wd(wsb=need - 1) == 4
    assert wd(d=80) == 5
    assert wd(B=0, q=None, k=None, v=None, kbits=None, ws=None) == 0


def test_rvq_table_polls_hook():
    """The table-poll bound is a process setting: a negative value is
    refused and changes nothing; each call returns the previous value."""
    prev = lib.rvq_decode_set_table_polls(5)
    assert prev >= 0
    assert lib.rvq_decode_set_table_polls(-1) == -1
    assert lib.rvq_decode_set_table_polls(prev) == 5
