"""decode_attention_qkv_noalloc (the entry point for callers that cannot
allocate): called through the C ABI, it must give exactly what
decode_attention_qkv gives with a caller workspace -- the same kernels on the
same inputs -- on two calls in a row, the second on a smaller cache (the
library's array keeps the first call's contents), and stay within the
attention tolerance of the oracle."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import say, dev, host, check_attention, oracle_cache, gpu_cache
from workloads import kivi_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dqa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dequant_decode_attention_amd as m
    return m


def _noalloc(dqa, q, cache, scale):
    """The entry point through the C ABI; out is the caller's buffer."""
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    st = cache.struct()
    rc = dqa.lib.decode_attention_qkv_noalloc(dqa._ptr(q), ctypes.byref(st), ctypes.c_float(scale),
                                              dqa._ptr(out), dqa._stream(q.device))
    assert rc == 0, dqa.lib.dqa_status_string(rc)
    return out


CALLS = [
    # B, Hq, Hkv, d, T_q, R, bits, rope: the second call is smaller and has
    # fewer splits, so it reads only part of what the first one left
    ((2, 32, 8, 128, 8192, 77, 2, 500000.0), (1, 8, 2, 64, 640, 5, 4, 10000.0)),
]


@pytest.mark.parametrize("calls", CALLS, ids=lambda c: "then".join("x".join(map(str, x[:6])) for x in c))
def test_noalloc_equals_workspace_call(dqa, calls):
    scratch = dqa.lib.decode_attention_noalloc_scratch_bytes()
    for i, (B, Hq, Hkv, d, T_q, R, bits, rope) in enumerate(calls):
        inp = kivi_inputs(B, Hq, Hkv, d, T_q, R, seed=31 + i, outliers=("lognormal", 0.04, 3.0, 1.0))
        scale = 1.0 / math.sqrt(d)
        cache = gpu_cache(dqa, inp, bits, Hq, rope)
        need = dqa.lib.decode_attention_workspace_bytes(ctypes.byref(cache.struct()))
        assert 256 < need <= scratch          # several splits, within the array
        q = dev(inp["q"])
        say("decode_attention_qkv_noalloc call", i, (B, Hq, Hkv, d, T_q, R, bits))
        got = _noalloc(dqa, q, cache, scale)
        ref_ws = dqa.decode_attention_qkv(q, cache, scale)
        torch.cuda.synchronize()
        assert np.array_equal(host(got), host(ref_ws))
        ref = oracle.kivi_decode_attention(inp["q"], oracle_cache(inp, bits, Hq, rope), scale)
        check_attention(host(got), ref, 1e-3, f"noalloc call {i}")
