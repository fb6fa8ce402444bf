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
              "dqa_status_string"]:
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
    for s in range(8):
        assert lib.dqa_status_string(s).startswith(b"DQA_")
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
    if fn == "quantize_pack_k":
        assert f(FAKE, 1, 1, 33, 128, 2, FAKE, FAKE, FAKE, None) == 2     # T % 32


def _cache(**kw):
    base = dict(B=2, Hq=8, Hkv=2, d=128, bits=2, T_q=64, R=16, rope_theta=0.0,
                k_codes=0x1000, k_scale=0x1000, k_zero=0x1000, v_codes=0x1000,
                v_scale=0x1000, v_zero=0x1000, k_recent=0x1000, v_recent=0x1000)
    base.update(kw)
    return KiviCacheStruct(*[base[n] for n, _ in KiviCacheStruct._fields_])


def test_decode_workspace_query_and_validation():
    ws = lib.decode_attention_workspace_bytes(ctypes.byref(_cache()))
    assert ws > 0
    # counters (one per unit, 256-byte region) + partial states
    assert ws >= 256 + 2 * 2 * 4 * 130 * 4
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
    assert lib.decode_attention_workspace_bytes(ctypes.byref(_cache(d=80))) == 0
    assert lib.decode_attention_workspace_bytes(None) == 0


def test_stream_copy_validation():
    assert lib.dqa_stream_copy(FAKE, None, 64, None) == 1
    assert lib.dqa_stream_copy(FAKE, FAKE, 20, None) == 2
    assert lib.dqa_stream_copy(ctypes.c_void_p(0x1008), FAKE, 64, None) == 2
