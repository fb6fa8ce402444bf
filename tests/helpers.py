"""Shared test helpers: tensor moves, error norms, and building the same
uniform-layout cache once with the oracle and once with the HIP library
(from the same seeded inputs; the two paths share nothing else)."""
import sys

import numpy as np
import torch

import oracle


def say(*a):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(x, device="cuda:0"):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def worst_row_rel(got, ref):
    g = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    r = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    num = np.linalg.norm(g - r, axis=1)
    den = np.maximum(np.linalg.norm(r, axis=1), 1e-30)
    return float((num / den).max())


def check_attention(got, ref, tol, label=""):
    """Attention parity: relative L2 over the whole output and the worst
    (batch, query head) row's relative L2, both within tol."""
    err, worst = rel_l2(got, ref), worst_row_rel(got, ref)
    print(f"{label} rel_l2={err:.3e} worst_row={worst:.3e}", flush=True)
    assert err <= tol, (label, err)
    assert worst <= tol, (label, worst)
    return err


def oracle_cache(inp, bits, Hq, rope_theta):
    """Oracle's own quantize + pack of the inputs, as the dict
    oracle.kivi_decode_attention reads."""
    B, Hkv, T_q, d = inp["k"].shape
    R = inp["k_recent"].shape[2]
    kc, ks, kz = oracle.quantize_k(inp["k"], bits)
    vc, vs, vz = oracle.quantize_v(inp["v"], bits)
    return dict(B=B, Hq=Hq, Hkv=Hkv, d=d, bits=bits, T_q=T_q, R=R, rope_theta=rope_theta,
                k_codes=oracle.pack_codes(kc, bits), v_codes=oracle.pack_v_codes(vc, bits),
                k_scale=ks, k_zero=kz, v_scale=vs, v_zero=vz,
                k_recent=inp["k_recent"], v_recent=inp["v_recent"])


def gpu_cache(dqa, inp, bits, Hq, rope_theta, device="cuda:0", rope_table=True):
    """The library's quantize + pack of the same inputs, as a KiviCache."""
    B, Hkv, T_q, d = inp["k"].shape
    R = inp["k_recent"].shape[2]
    if T_q > 0:
        kc, ks, kz = dqa.quantize_pack_k(dev(inp["k"], device), bits)
        vc, vs, vz = dqa.quantize_pack_v(dev(inp["v"], device), bits)
    else:
        kc = ks = kz = vc = vs = vz = None
    kr = dev(inp["k_recent"], device) if R > 0 else None
    vr = dev(inp["v_recent"], device) if R > 0 else None
    return dqa.KiviCache(Hq, bits, kc, ks, kz, vc, vs, vz, kr, vr, rope_theta=rope_theta,
                         T_q=T_q, B=B, Hkv=Hkv, d=d, rope_table=rope_table)
