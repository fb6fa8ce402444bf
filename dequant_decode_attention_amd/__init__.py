"""Python binding of libdqattn (decode attention over a low-bit KV cache on
MI355X / gfx950).

Argument marshalling only: every step runs in the HIP kernels of
``libdqattn.so``.  PyTorch supplies device memory (outputs and workspaces
are allocated with torch) and the current stream.  Importing this package
raises if the library has not been built; there is no fallback path.

Function names and semantics mirror ``include/dqattn.h``.
"""

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DQA_LIBRARY names another build of the same library (the host-sanitizer
# build of build.py --host-sanitize, for CPU runs under AddressSanitizer)
LIB_PATH = os.environ.get("DQA_LIBRARY") or os.path.join(_HERE, "libdqattn.so")

DQA_OK = 0
_STATUS = {0: "DQA_OK", 1: "DQA_ERR_NULL", 2: "DQA_ERR_SHAPE", 3: "DQA_ERR_BITS",
           4: "DQA_ERR_WORKSPACE", 5: "DQA_ERR_UNSUPPORTED", 6: "DQA_ERR_HIP",
           7: "DQA_ERR_PLAN", 8: "DQA_ERR_ALIGN"}


class DqaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {lib.dqa_status_string(status).decode()}")


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python dequant_decode_attention_amd/build.py`")

lib = ctypes.CDLL(LIB_PATH)

_vp, _i, _sz, _f, _i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_int64


class KiviCacheStruct(ctypes.Structure):
    """Mirror of ``dqa_kivi_cache``."""
    _fields_ = [("B", _i), ("Hq", _i), ("Hkv", _i), ("d", _i), ("bits", _i),
                ("T_q", _i), ("R", _i), ("rope_theta", _f),
                ("k_codes", _vp), ("k_scale", _vp), ("k_zero", _vp),
                ("v_codes", _vp), ("v_scale", _vp), ("v_zero", _vp),
                ("k_recent", _vp), ("v_recent", _vp), ("T_cap", _i), ("R_cap", _i),
                ("rope_table", _vp)]


_SIGS = {
    "dqa_status_string": (ctypes.c_char_p, [_i]),
    "dqa_abi_version": (_i, []),
    "quantize_pack_k": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "quantize_pack_v": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "decode_attention_workspace_bytes": (_sz, [ctypes.POINTER(KiviCacheStruct)]),
    "decode_attention_qkv": (_i, [_vp, ctypes.POINTER(KiviCacheStruct), _f, _vp, _sz, _vp, _vp]),
    "decode_attention_qkv_noalloc": (_i, [_vp, ctypes.POINTER(KiviCacheStruct), _f, _vp, _vp]),
    "decode_attention_noalloc_scratch_bytes": (_sz, []),
    "decode_attention_qkv_partial": (_i, [_vp, ctypes.POINTER(KiviCacheStruct), _f, _vp, _sz, _vp, _vp]),
    "decode_attention_qkv_merge": (_i, [ctypes.POINTER(KiviCacheStruct), _vp, _sz, _vp, _vp]),
    "kivi_rope_table_words": (_sz, [_i]),
    "kivi_rope_table": (_i, [_f, _i, _i, _vp, _vp]),
    "kivi_append_workspace_bytes": (_sz, [ctypes.POINTER(KiviCacheStruct), _i]),
    "kivi_append": (_i, [ctypes.POINTER(KiviCacheStruct), _vp, _vp, _i, _i, _vp, _sz, _vp]),
    "zoned_plan_words": (_sz, [_i, _i, _i, _i]),
    "zoned_plan": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, ctypes.POINTER(_sz)]),
    "zoned_pack": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "decode_attention_zoned_workspace_bytes": (_sz, [_vp, _i]),
    "decode_attention_zoned": (_i, [_vp, _i, _vp, _vp, _vp, _f, _vp, _sz, _vp, _vp]),
    "rvq_encode_workspace_bytes": (_sz, [_i, _i]),
    "rvq_encode": (_i, [_vp, _i64, _i, _vp, _i, _i, _vp, _vp, _sz, _vp]),
    "rvq_decode_attention_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "rvq_decode_attention": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _i, _f,
                                  _vp, _sz, _vp, _vp]),
    "rvq_decode_set_table_polls": (_i, [_i]),
    "rdkv_token_weights_workspace_bytes": (_sz, [_i, _i, _i]),
    "rdkv_token_weights": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _vp, _sz, _vp]),
    "rdkv_channel_weights_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "rdkv_channel_weights": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "rdkv_allocate_workspace_bytes": (_sz, [_i, _i]),
    "rdkv_allocate": (_i, [_vp, _i, _i, ctypes.c_longlong, _vp, _vp, _sz, _vp]),
    "rdkv_widths_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "rdkv_widths": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _f, ctypes.c_longlong, ctypes.c_longlong,
                         _vp, _vp, _vp, _sz, _vp]),
    "dqa_stream_copy": (_i, [_vp, _vp, _sz, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def _check(fn, status):
    if status != DQA_OK:
        raise DqaError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev16(t, name):
    if t.dtype != torch.float16 or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA float16 tensor")
    return t.contiguous()


# ---------------------------------------------------------------- quantize

def _quant_out(out, shapes, device):
    """Output tensors of a quantizer: `out` (codes, scale, zero) checked
    against the expected shapes, or fresh ones."""
    dts = (torch.int32, torch.float16, torch.float16)
    if out is None:
        return tuple(torch.empty(sh, dtype=dt, device=device) for sh, dt in zip(shapes, dts))
    if len(out) != 3:
        raise ValueError("out must be (codes, scale, zero)")
    for t, sh, dt in zip(out, shapes, dts):
        if tuple(t.shape) != tuple(sh) or t.dtype != dt or t.device != device or not t.is_contiguous():
            raise ValueError(f"out tensor {tuple(t.shape)} {t.dtype}: expected contiguous {tuple(sh)} {dt}")
    return tuple(out)


def quantize_pack_k(k, bits, out=None):
    """k: fp16 [B, Hkv, T, d] -> (codes int32 [B, Hkv, T, d*bits/32] holding
    uint32 words, scale fp16 [B, Hkv, T/32, d], zero fp16 [B, Hkv, T/32, d]),
    written into `out` when given."""
    k = _dev16(k, "k")
    B, H, T, d = k.shape
    codes, scale, zero = _quant_out(out, ((B, H, T, d * bits // 32), (B, H, T // 32, d), (B, H, T // 32, d)),
                                    k.device)
    _check("quantize_pack_k", lib.quantize_pack_k(_ptr(k), B, H, T, d, bits, _ptr(codes),
                                                  _ptr(scale), _ptr(zero), _stream(k.device)))
    return codes, scale, zero


def quantize_pack_v(v, bits, out=None):
    """v: fp16 [B, Hkv, T, d] -> (codes int32 [B, Hkv, T, d*bits/32], scale fp16
    [B, Hkv, T, d/32], zero fp16 [B, Hkv, T, d/32]), written into `out` when
    given."""
    v = _dev16(v, "v")
    B, H, T, d = v.shape
    codes, scale, zero = _quant_out(out, ((B, H, T, d * bits // 32), (B, H, T, d // 32), (B, H, T, d // 32)),
                                    v.device)
    _check("quantize_pack_v", lib.quantize_pack_v(_ptr(v), B, H, T, d, bits, _ptr(codes),
                                                  _ptr(scale), _ptr(zero), _stream(v.device)))
    return codes, scale, zero


# ---------------------------------------------------------------- KIVI decode

def kivi_rope_table(rope_theta, d, bits, device):
    """The in-tile rotation table of a RoPE cache: int32 [kivi_rope_table_words(d)] on device."""
    n = lib.kivi_rope_table_words(d)
    if n == 0:
        raise DqaError("kivi_rope_table", 2)
    table = torch.empty(n, dtype=torch.int32, device=device)
    _check("kivi_rope_table", lib.kivi_rope_table(float(rope_theta), d, bits, _ptr(table), _stream(device)))
    return table


class KiviCache:
    """Device tensors of a uniform-layout cache plus its descriptor.

    k_codes/v_codes int32 [B, Hkv, T_cap, d*bits/32]; k_scale/k_zero fp16
    [B, Hkv, T_cap/32, d]; v_scale/v_zero fp16 [B, Hkv, T_cap, d/32];
    k_recent/v_recent fp16 [B, Hkv, R_cap, d] (keys before RoPE) or None.
    The capacities are the tensors' token dimensions; T_q (default T_cap)
    and R (default R_cap) are the tokens in use.  A 2- or 4-bit cache with
    RoPE builds its in-tile rotation table once (kivi_rope_table) unless
    rope_table=False.
    """

    def __init__(self, Hq, bits, k_codes, k_scale, k_zero, v_codes, v_scale, v_zero,
                 k_recent=None, v_recent=None, rope_theta=0.0, T_q=None, B=None, Hkv=None, d=None,
                 R=None, rope_table=True):
        ref = k_codes if k_codes is not None else k_recent
        self.B = ref.shape[0] if B is None else B
        self.Hkv = ref.shape[1] if Hkv is None else Hkv
        self.d = (k_scale.shape[3] if k_scale is not None else k_recent.shape[3]) if d is None else d
        self.T_cap = k_codes.shape[2] if k_codes is not None else 0
        self.R_cap = k_recent.shape[2] if k_recent is not None else 0
        self.T_q = self.T_cap if T_q is None else T_q
        self.R = self.R_cap if R is None else R
        self.Hq, self.bits, self.rope_theta = Hq, bits, float(rope_theta)
        self.tensors = dict(k_codes=k_codes, k_scale=k_scale, k_zero=k_zero, v_codes=v_codes,
                            v_scale=v_scale, v_zero=v_zero, k_recent=k_recent, v_recent=v_recent)
        self.tensors = {k: (None if v is None else v.contiguous()) for k, v in self.tensors.items()}
        self._ws = None
        self.rope_table = None
        if rope_table and self.rope_theta > 0 and bits in (2, 4):
            self.rope_table = kivi_rope_table(self.rope_theta, self.d, bits, ref.device)

    def struct(self):
        t = self.tensors
        return KiviCacheStruct(self.B, self.Hq, self.Hkv, self.d, self.bits, self.T_q, self.R,
                               self.rope_theta, *[(None if t[n] is None else t[n].data_ptr()) for n in
                                                  ("k_codes", "k_scale", "k_zero", "v_codes",
                                                   "v_scale", "v_zero", "k_recent", "v_recent")],
                               self.T_cap, self.R_cap,
                               None if self.rope_table is None else self.rope_table.data_ptr())

    def workspace_bytes(self):
        return lib.decode_attention_workspace_bytes(ctypes.byref(self.struct()))

    def workspace(self, device):
        """A zeroed workspace of the required size, cached on the cache
        object (every decode call leaves its merge counters zero)."""
        n = self.workspace_bytes()
        if self._ws is None or self._ws.numel() < n or self._ws.device != device:
            self._ws = torch.zeros(max(n, 256), dtype=torch.uint8, device=device)
        return self._ws


def decode_attention_workspace_bytes(cache):
    return cache.workspace_bytes()


def decode_attention_qkv(q, cache, sm_scale, out=None, workspace=None):
    """q: fp16 [B, Hq, d] (rotated when the cache uses RoPE) -> fp32 [B, Hq, d]."""
    q = _dev16(q, "q")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    ws = cache.workspace(q.device) if workspace is None else workspace
    st = cache.struct()
    _check("decode_attention_qkv",
           lib.decode_attention_qkv(_ptr(q), ctypes.byref(st), float(sm_scale), _ptr(ws),
                                    ws.numel(), _ptr(out), _stream(q.device)))
    return out


def decode_attention_qkv_noalloc(q, cache, sm_scale, out):
    """decode_attention_qkv with the library's per-GPU partial-state array
    instead of a workspace (the call allocates no device memory; calls that
    overlap on one GPU race).  out: fp32 [B, Hq, d], provided by the caller."""
    q = _dev16(q, "q")
    st = cache.struct()
    with torch.cuda.device(q.device):
        _check("decode_attention_qkv_noalloc",
               lib.decode_attention_qkv_noalloc(_ptr(q), ctypes.byref(st), float(sm_scale), _ptr(out),
                                                _stream(q.device)))
    return out


def decode_attention_qkv_partial(q, cache, sm_scale, out, workspace):
    """First phase of decode_attention_qkv (the split kernel); see the header."""
    q = _dev16(q, "q")
    st = cache.struct()
    _check("decode_attention_qkv_partial",
           lib.decode_attention_qkv_partial(_ptr(q), ctypes.byref(st), float(sm_scale),
                                            _ptr(workspace), workspace.numel(), _ptr(out),
                                            _stream(q.device)))
    return out


def decode_attention_qkv_merge(cache, out, workspace):
    """Second phase of decode_attention_qkv (merge of the splits)."""
    st = cache.struct()
    _check("decode_attention_qkv_merge",
           lib.decode_attention_qkv_merge(ctypes.byref(st), _ptr(workspace), workspace.numel(),
                                          _ptr(out), _stream(out.device)))
    return out


def kivi_append(cache, k_new, v_new, R_max=128, workspace=None):
    """Append fp16 tokens k_new, v_new [B, Hkv, n_new, d] (keys before RoPE)
    to the cache's recent zone, quantizing its oldest 32 tokens into the
    quantized buffers while it holds more than R_max (see the header).
    Updates cache.T_q and cache.R; returns the number of 32-token groups
    quantized."""
    n_new = 0
    if k_new is not None:
        k_new, v_new = _dev16(k_new, "k_new"), _dev16(v_new, "v_new")
        n_new = k_new.shape[2]
    dev = (k_new if k_new is not None else cache.tensors["k_recent"]).device
    st = cache.struct()
    n = lib.kivi_append_workspace_bytes(ctypes.byref(st), n_new)
    if n == 0:
        raise DqaError("kivi_append", 2)
    ws = torch.empty(n, dtype=torch.uint8, device=dev) if workspace is None else workspace
    T0 = cache.T_q
    _check("kivi_append", lib.kivi_append(ctypes.byref(st), _ptr(k_new), _ptr(v_new), n_new, int(R_max),
                                          _ptr(ws), ws.numel(), _stream(dev)))
    cache.T_q, cache.R = st.T_q, st.R
    return (cache.T_q - T0) // 32


# ---------------------------------------------------------------- zoned

class ZonedPlan:
    """Host plan words (numpy int32), their device copy and the blob size."""

    def __init__(self, words, blob_bytes, device):
        self.words = words
        self.blob_bytes = blob_bytes
        self.dev = torch.from_numpy(words).to(device)

    def host_ptr(self):
        return ctypes.c_void_p(self.words.ctypes.data)


def zoned_plan(v_bits, k_bits, C_new, d, device, sink=0, k_out=0):
    """v_bits int8 [B, Hkv, T_old] and k_bits int8 [B, Hkv, d] in
    {0,2,4,8,16} (host arrays); sink: old tokens kept whole; k_out: outlier
    side-list entries per key group -> ZonedPlan."""
    v_bits = np.ascontiguousarray(np.asarray(v_bits, dtype=np.int8))
    k_bits = np.ascontiguousarray(np.asarray(k_bits, dtype=np.int8))
    B, H, T = v_bits.shape
    n = lib.zoned_plan_words(B, H, T, d)
    if n == 0:
        raise DqaError("zoned_plan_words", 2)
    words = np.zeros(n, dtype=np.int32)
    blob = ctypes.c_size_t(0)
    _check("zoned_plan", lib.zoned_plan(ctypes.c_void_p(v_bits.ctypes.data),
                                        ctypes.c_void_p(k_bits.ctypes.data), B, H, T, C_new, d,
                                        int(sink), int(k_out), ctypes.c_void_p(words.ctypes.data), n,
                                        ctypes.byref(blob)))
    return ZonedPlan(words, blob.value, device)


def zoned_pack(plan, k, v, k_new=None, v_new=None, out=None):
    """Pack fp16 caches into a uint8 blob of plan.blob_bytes bytes (every
    byte written; `out`, if given, is a uint8 device tensor of that size)."""
    k, v = _dev16(k, "k"), _dev16(v, "v")
    k_new = None if k_new is None else _dev16(k_new, "k_new")
    v_new = None if v_new is None else _dev16(v_new, "v_new")
    if out is None:
        blob = torch.empty(plan.blob_bytes, dtype=torch.uint8, device=k.device)
    else:
        if out.dtype != torch.uint8 or out.numel() != plan.blob_bytes or not out.is_contiguous() \
                or out.device != k.device:
            raise ValueError(f"zoned_pack: out must be a contiguous uint8 tensor of {plan.blob_bytes} "
                             f"bytes on {k.device}")
        blob = out
    _check("zoned_pack", lib.zoned_pack(plan.host_ptr(), _ptr(plan.dev), _ptr(k), _ptr(v),
                                        _ptr(k_new), _ptr(v_new), _ptr(blob), _stream(k.device)))
    return blob


def decode_attention_zoned(q, plan, blob, sm_scale, out=None, workspace=None):
    q = _dev16(q, "q")
    Hq = q.shape[1]
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if workspace is None:
        n = lib.decode_attention_zoned_workspace_bytes(plan.host_ptr(), Hq)
        workspace = torch.zeros(max(n, 1), dtype=torch.uint8, device=q.device)
    _check("decode_attention_zoned",
           lib.decode_attention_zoned(_ptr(q), Hq, plan.host_ptr(), _ptr(plan.dev), _ptr(blob),
                                      float(sm_scale), _ptr(workspace), workspace.numel(),
                                      _ptr(out), _stream(q.device)))
    return out


# ---------------------------------------------------------------- RVQ

def rvq_encode(x, codebooks, workspace=None):
    """x fp16 [n, d]; codebooks fp16 [N, Kc, d] -> idx int16 [n, N]."""
    x, codebooks = _dev16(x, "x"), _dev16(codebooks, "codebooks")
    n, d = x.shape
    N, Kc, _ = codebooks.shape
    idx = torch.empty((n, N), dtype=torch.int16, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(lib.rvq_encode_workspace_bytes(N, Kc), 1), dtype=torch.uint8,
                                device=x.device)
    _check("rvq_encode", lib.rvq_encode(_ptr(x), n, d, _ptr(codebooks), N, Kc, _ptr(idx),
                                        _ptr(workspace), workspace.numel(), _stream(x.device)))
    return idx


def rvq_decode_attention(q, k_idx, v_idx, k_codebooks, v_codebooks, sm_scale, out=None,
                         workspace=None):
    """q fp16 [B, Hq, d]; k_idx/v_idx int16 [B, Hkv, T, N]; codebooks fp16
    [N, Kc, d] -> fp32 [B, Hq, d]."""
    q = _dev16(q, "q")
    B, Hq, d = q.shape
    _, Hkv, T, N = k_idx.shape
    Kc = k_codebooks.shape[1]
    if tuple(k_codebooks.shape) != (N, Kc, d) or tuple(v_codebooks.shape) != (N, Kc, d):
        raise ValueError(f"codebooks must both be [N={N}, Kc, d={d}], got {tuple(k_codebooks.shape)} "
                         f"and {tuple(v_codebooks.shape)}")
    if tuple(k_idx.shape) != (B, k_idx.shape[1], k_idx.shape[2], N) or tuple(v_idx.shape) != tuple(k_idx.shape):
        raise ValueError(f"k_idx and v_idx must both be [B, Hkv, T, N], got {tuple(k_idx.shape)} "
                         f"and {tuple(v_idx.shape)}")
    k_idx, v_idx = k_idx.contiguous(), v_idx.contiguous()
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if workspace is None:
        n = lib.rvq_decode_attention_workspace_bytes(B, Hq, Hkv, T, d)
        workspace = torch.zeros(max(n, 1), dtype=torch.uint8, device=q.device)
    _check("rvq_decode_attention",
           lib.rvq_decode_attention(_ptr(q), B, Hq, Hkv, T, d, _ptr(k_idx), _ptr(v_idx),
                                    _ptr(_dev16(k_codebooks, "k_codebooks")),
                                    _ptr(_dev16(v_codebooks, "v_codebooks")), N, Kc,
                                    float(sm_scale), _ptr(workspace), workspace.numel(),
                                    _ptr(out), _stream(q.device)))
    return out


def rvq_decode_set_table_polls(polls):
    """Polls of a unit's table flags before a workgroup builds the table
    alone (test hook; 0 forces that path).  Returns the previous value."""
    prev = lib.rvq_decode_set_table_polls(int(polls))
    if prev < 0:
        raise ValueError(f"polls must be >= 0, got {polls}")
    return prev


# ---------------------------------------------------------------- RDKV

def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def rdkv_token_weights(q, k, sm_scale, workspace=None):
    """q fp16 [B, Hq, T, d], k fp16 [B, Hkv, T, d] -> fp32 [B, Hkv, T]."""
    q, k = _dev16(q, "q"), _dev16(k, "k")
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    w = torch.empty((B, Hkv, T), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _ws(lib.rdkv_token_weights_workspace_bytes(B, Hq, T), q.device)
    _check("rdkv_token_weights",
           lib.rdkv_token_weights(_ptr(q), _ptr(k), B, Hq, Hkv, T, d, float(sm_scale), _ptr(w),
                                  _ptr(workspace), workspace.numel(), _stream(q.device)))
    return w


def rdkv_channel_weights(q, k, keep, workspace=None):
    """q, k as rdkv_token_weights; keep int8 [B, Hkv, T] -> fp32 [B, Hkv, d]."""
    q, k = _dev16(q, "q"), _dev16(k, "k")
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if keep.dtype != torch.int8 or not keep.is_cuda:
        raise TypeError("keep must be a CUDA int8 tensor")
    keep = keep.contiguous()
    w = torch.empty((B, Hkv, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _ws(lib.rdkv_channel_weights_workspace_bytes(B, Hkv, T, d), q.device)
    _check("rdkv_channel_weights",
           lib.rdkv_channel_weights(_ptr(q), _ptr(k), _ptr(keep), B, Hq, Hkv, T, d, _ptr(w),
                                    _ptr(workspace), workspace.numel(), _stream(q.device)))
    return w


def rdkv_allocate(w, budget, workspace=None):
    """w fp32 [..., n] -> int8 widths of the same shape; one allocation per
    row (last axis), each row's total <= budget bits."""
    if w.dtype != torch.float32 or not w.is_cuda:
        raise TypeError("w must be a CUDA float32 tensor")
    w = w.contiguous()
    n = w.shape[-1] if w.dim() else 1
    rows = w.numel() // n if n else 0
    out = torch.empty(w.shape, dtype=torch.int8, device=w.device)
    if workspace is None:
        workspace = _ws(lib.rdkv_allocate_workspace_bytes(rows, n), w.device)
    _check("rdkv_allocate", lib.rdkv_allocate(_ptr(w), rows, n, int(budget), _ptr(out), _ptr(workspace),
                                              workspace.numel(), _stream(w.device)))
    return out


def rdkv_widths(q, k, sm_scale, v_budget, k_budget, workspace=None):
    """All three phases: (v_bits int8 [B, Hkv, T], k_bits int8 [B, Hkv, d]),
    per-sequence budgets in bits."""
    q, k = _dev16(q, "q"), _dev16(k, "k")
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    v_bits = torch.empty((B, Hkv, T), dtype=torch.int8, device=q.device)
    k_bits = torch.empty((B, Hkv, d), dtype=torch.int8, device=q.device)
    if workspace is None:
        workspace = _ws(lib.rdkv_widths_workspace_bytes(B, Hq, Hkv, T, d), q.device)
    _check("rdkv_widths",
           lib.rdkv_widths(_ptr(q), _ptr(k), B, Hq, Hkv, T, d, float(sm_scale), int(v_budget),
                           int(k_budget), _ptr(v_bits), _ptr(k_bits), _ptr(workspace),
                           workspace.numel(), _stream(q.device)))
    return v_bits, k_bits


def stream_copy(src, dst):
    """Plain device copy of src.numel()*element_size bytes into dst."""
    nbytes = src.numel() * src.element_size()
    _check("dqa_stream_copy", lib.dqa_stream_copy(_ptr(src), _ptr(dst), nbytes,
                                                  _stream(src.device)))
