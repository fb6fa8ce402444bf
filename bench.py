"""Benchmark: decode attention over a 2-bit uniform (KIVI-layout) KV cache on
one MI355X, Llama-3.1-8B-shaped GQA workload (batch 4, 32 query / 8 KV
heads, head dim 128, 32768 quantized tokens + 128 fp16 recent tokens, RoPE
theta 5e5).

One step = one decode step over the whole batch, i.e. one
decode_attention_qkv call: one kernel (kivi_feat_kernel: every quantized
token's packed codes and scales plus the fp16 recent zone are read from
HBM and attended with the rotation folded into the key product; the last
workgroup of each (batch, KV head) merges its splits).  The kernel's average
duration, for the roofline figure, is timed separately over launches through
the split-phase entry point, each between its own HIP events (the launches
then run one after the other, as in the profiler's kernel trace; back to
back, a launch's last workgroups overlap the next one's first, and that
rate is reported beside it).  Inputs are resident
in HBM before the timed region.  The compressed cache (~98 MiB) fits in the
256 MB Infinity Cache, so the timed steps rotate over several independent
replicas whose total exceeds it.

The line also carries "rows": the other steps of the path timed on their
own workloads with HIP events, each against its own roofline (quantize +
pack of the 32k cache; zoned pack and decode on the mixed-width 16k cache;
residual-VQ encode, MFMA-bound, and decode on the 8k Llama-3.2-3B-shaped
cache; the decode at the other bit width and on the Llama-2-13B-shaped layer),
and "cpu_baseline": the oracle timed on a sample of the same step, with BLAS
on every core of the affinity mask and on one thread.

Prints one JSON line.  Usage:
    python bench.py [--steps K] [--warmup W] [--bits 2|4] [--replicas R]
                    [--no-cpu-baseline] [--no-rows]
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
# Vector-ALU issue peak: 256 CUs x 4 SIMDs, one wave64 VALU instruction per
# SIMD every 4 cycles (16 lanes per cycle) at the 2.4 GHz peak clock.
VALU_PEAK_GINST = 256 * 4 * 2.4 / 4
KERNEL_SOURCES = [os.path.join(ROOT, "dequant_decode_attention_amd", "csrc", f)
                  for f in ("decode_feat.hip", "decode_common.h", "decode_kivi.hip", "merge.h", "common.h")]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "kivi_feat_kernel_llama8b_gqa_32k_traffic.md")


def measured_traffic(bits, key_fmt="traffic_bytes_per_launch_{bits}bit"):
    """HBM bytes per launch of the split kernel from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, scaled by the
    copy-kernel calibration), or None when the summary is missing, covers
    another bit width, or was taken on a different kernel source.  With
    key_fmt "valu_instructions_per_launch_{bits}bit": the kernel's VALU wave
    instructions per launch (SQ_INSTS_VALU) under the same conditions."""
    import hashlib
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    src = hashlib.sha256(b"".join(open(f, "rb").read() for f in KERNEL_SOURCES)).hexdigest()
    if fields.get("kernel_source_sha256") != src:
        return None
    key = key_fmt.format(bits=bits)
    return int(fields[key]) if key in fields else None


def algorithmic_bytes(cfg, bits):
    """Bytes one decode step must move: packed codes, fp16 scale/zero of K
    and V, the fp16 recent zone, the query and the fp32 output."""
    B, Hq, Hkv, d, T_q, R = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T_q"], cfg["R"]
    units = B * Hkv
    codes = 2 * units * T_q * d * bits // 8
    k_sz = units * (T_q // 32) * d * 2 * 2
    v_sz = units * T_q * (d // 32) * 2 * 2
    recent = 2 * units * R * d * 2
    return codes + k_sz + v_sz + recent + B * Hq * d * 2 + B * Hq * d * 4


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_step_rate(inp, cfg, bits, scale, budget_s):
    """The oracle's decode (dequantization from the packed buffers + fp64
    attention) on whole (batch, KV head) units until the budget is spent;
    returns (KV-tokens/s of the full step, units done, seconds)."""
    import oracle
    B, Hkv, G = cfg["B"], cfg["Hkv"], cfg["Hq"] // cfg["Hkv"]
    units = [(b, h) for b in range(B) for h in range(Hkv)]
    done, elapsed = 0, 0.0
    for b, h in units:
        sub = {k: v[b:b + 1, h:h + 1] for k, v in inp.items() if k != "q"}
        kc, ks, kz = oracle.quantize_k(sub["k"], bits)          # not timed: cache build
        vc, vs, vz = oracle.quantize_v(sub["v"], bits)
        cache = dict(B=1, Hq=G, Hkv=1, d=cfg["d"], bits=bits, T_q=cfg["T_q"], R=cfg["R"],
                     rope_theta=cfg["rope_theta"], k_codes=oracle.pack_codes(kc, bits),
                     v_codes=oracle.pack_v_codes(vc, bits), k_scale=ks, k_zero=kz,
                     v_scale=vs, v_zero=vz, k_recent=sub["k_recent"], v_recent=sub["v_recent"])
        q = inp["q"][b:b + 1, h * G:(h + 1) * G]
        t0 = time.perf_counter()
        oracle.kivi_decode_attention(q, cache, scale)
        elapsed += time.perf_counter() - t0
        done += 1
        if elapsed > budget_s:
            break
    step_s = elapsed / done * len(units)
    return B * (cfg["T_q"] + cfg["R"]) / step_s, done, len(units), elapsed


def cpu_baseline(inp, cfg, bits, scale, budget_s=10.0):
    """The oracle timed on this machine's host cores in two settings: BLAS
    threads = every core in the process's affinity mask, and one thread."""
    from threadpoolctl import threadpool_limits
    ncores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=ncores):
        v_all, done, n, el = _oracle_step_rate(inp, cfg, bits, scale, budget_s)
    with threadpool_limits(limits=1):
        v_one, done1, n1, el1 = _oracle_step_rate(inp, cfg, bits, scale, budget_s)
    return dict(value=v_all, unit="KV-tokens/s", cores=ncores, kind="oracle",
                sample=f"{done} of {n} (batch, KV head) units, {el:.1f} s, BLAS threads = {ncores} "
                       f"(every core in the affinity mask); numpy dequantization + fp64 attention, "
                       f"scaled to the full step",
                single_thread={"value": v_one, "cores": 1,
                               "sample": f"{done1} of {n1} units, {el1:.1f} s, BLAS threads = 1"},
                cpu_model=_cpu_model())


MFMA_FP16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak, published


WARM_S = 0.3   # seconds of untimed work before each timed region


def _warm(torch, fn, n, seconds=WARM_S):
    """n untimed calls of fn(i), then more until `seconds` of wall time have
    passed: the GPU's clocks ramp up over the first tens of milliseconds of
    sustained work (a decode step measured 64.8 us at first, 56.5 us in
    steady state), and a few calls are over before that."""
    t0 = time.perf_counter()
    i = 0
    while i < n or time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def _event_ms(torch, fn, iters, warmup=3):
    """Average duration of fn() over iters calls, HIP events on the current
    stream (fn enqueues work only), after the warm-up of _warm."""
    _warm(torch, fn, warmup)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(iters):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def _hbm_row(kernel, workload, ms, nbytes, note=""):
    gbps = nbytes / (ms * 1e-3) / 1e9
    r = {"kernel": kernel, "workload": workload, "us": ms * 1e3, "bound": "hbm",
         "algorithmic_bytes": nbytes, "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
         "frac": gbps / HBM_PEAK_GBPS}
    if note:
        r["note"] = note
    return r


def time_quantize(dqa, torch, k, v, bits, cfg):
    """Rows a1-a3: quantize + pack of the whole llama3.1-8b-gqa-32k cache (fp16 in, codes and
    fp16 scale/zero out)."""
    B, Hkv, T, d = k.shape
    n = B * Hkv * T * d
    nbytes = n * 2 + n * bits // 8 + 2 * 2 * (n // 32)
    out = {}
    for name, x, fn in (("quantize_k", k, dqa.quantize_pack_k), ("quantize_v", v, dqa.quantize_pack_v)):
        dst = fn(x, bits)      # output buffers, reused by every timed call
        ms = _event_ms(torch, lambda i: fn(x, bits, out=dst), 50)
        out[name] = _hbm_row(f"{name}_kernel", cfg["workload"], ms, nbytes)
    return out


def time_append(dqa, torch, dev, cfg, bits):
    """Streaming append on the llama3.1-8b-gqa-32k shape: one new token per (batch, KV head)
    into a full 128-token fp16 window over a cache holding 32736 quantized
    tokens, so every call quantizes one group of 32 per (batch, KV head)
    (the counts are reset between calls)."""
    B, Hkv, d, Hq = cfg["B"], cfg["Hkv"], cfg["d"], cfg["Hq"]
    T_cap, T_q0, R_cap = cfg["T_q"], cfg["T_q"] - 32, 128
    w = d * bits // 32
    z = lambda *sh, dt=torch.float16: torch.zeros(sh, dtype=dt, device=dev)
    cache = dqa.KiviCache(Hq, bits, z(B, Hkv, T_cap, w, dt=torch.int32), z(B, Hkv, T_cap // 32, d),
                          z(B, Hkv, T_cap // 32, d), z(B, Hkv, T_cap, w, dt=torch.int32), z(B, Hkv, T_cap, d // 32),
                          z(B, Hkv, T_cap, d // 32), torch.randn(B, Hkv, R_cap, d, device=dev).half(),
                          torch.randn(B, Hkv, R_cap, d, device=dev).half(), rope_theta=cfg["rope_theta"],
                          T_q=T_q0, R=R_cap)
    kn = torch.randn(B, Hkv, 1, d, device=dev).half()
    vn = torch.randn(B, Hkv, 1, d, device=dev).half()
    cache.T_q, cache.R = T_q0, R_cap
    st = cache.struct()
    ws = torch.empty(dqa.lib.kivi_append_workspace_bytes(ctypes.byref(st), 1), dtype=torch.uint8, device=dev)

    def call(i):
        cache.T_q, cache.R = T_q0, R_cap
        dqa.kivi_append(cache, kn, vn, 128, workspace=ws)

    ms = _event_ms(torch, call, 50)
    units = B * Hkv
    nbytes = units * (2 * d * 2                       # the new token, K and V
                      + 2 * (R_cap + 1) * d * 2       # the window read
                      + 2 * (R_cap + 1 - 32) * d * 2  # the kept rows written back
                      + 2 * 32 * w * 4                # the group's key and value codes
                      + 2 * d * 2 + 2 * 32 * (d // 32) * 2)   # key and value scales and zeros
    return {"kivi_append": _hbm_row("flush_window_kernel", cfg["workload"], ms,
                                    nbytes, "one token into a full window: one 32-token group per (batch, KV head) "
                                    "quantized straight from the window, then the window moved in place; "
                                    "one launch of 64 workgroups, latency-bound")}


def time_zoned(dqa, torch, dev):
    """Rows a8-a9 on the mixed-width-zoned-16k workload: packer (fp16 K/V of
    kept tokens read, blob written) and decode (blob read; blob replicas
    rotated past the Infinity Cache); then the same pair with that workload's sink
    window and key outlier side lists."""
    from workloads import CONFIGS, zoned_inputs
    import numpy as np
    cfg = CONFIGS["mixed-width-zoned-16k"]
    inp = zoned_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T_old"], cfg["C"], seed=4,
                       v_width_probs=cfg["v_width_probs"], k_width_probs=cfg["k_width_probs"],
                       outliers=cfg["outliers"])
    k, v = torch.from_numpy(inp["k"]).to(dev), torch.from_numpy(inp["v"]).to(dev)
    kn, vn = torch.from_numpy(inp["k_new"]).to(dev), torch.from_numpy(inp["v_new"]).to(dev)
    q = torch.from_numpy(inp["q"]).to(dev)
    d = cfg["d"]
    scale = 1.0 / math.sqrt(d)
    out = {}
    variants = (("", 0, 0), ("_sink_outliers", cfg["zoned_variant"]["sink"], cfg["zoned_variant"]["k_out"]))
    for suffix, sink, k_out in variants:
        plan = dqa.zoned_plan(inp["v_bits"], inp["k_bits"], cfg["C"], d, dev, sink=sink, k_out=k_out)
        kept = int((inp["v_bits"][:, :, sink:] > 0).sum())
        pack_bytes = 2 * kept * d * 2 + 2 * (kn.numel() + q.shape[0] * cfg["Hkv"] * sink * d) * 2 \
            + plan.blob_bytes
        note = "fp16 K/V of kept tokens and new tokens read, blob written"
        if sink or k_out:
            note += f"; {sink} sink tokens, {k_out} side-list entries per key group"
        ms = _event_ms(torch, lambda i: dqa.zoned_pack(plan, k, v, kn, vn), 10)
        out["zoned_pack" + suffix] = _hbm_row("zoned_pack_kernel", cfg["workload"], ms, pack_bytes, note)
        blob = dqa.zoned_pack(plan, k, v, kn, vn)
        reps = max(2, int(np.ceil(320e6 / max(plan.blob_bytes, 1))))
        blobs = [blob.clone() for _ in range(reps)]
        res = torch.empty(q.shape, dtype=torch.float32, device=dev)
        n = dqa.lib.decode_attention_zoned_workspace_bytes(plan.host_ptr(), cfg["Hq"])
        ws = torch.zeros(max(n, 1), dtype=torch.uint8, device=dev)
        ms = _event_ms(torch, lambda i: dqa.decode_attention_zoned(q, plan, blobs[i % reps], scale,
                                                                    out=res, workspace=ws), 50)
        nbytes = plan.blob_bytes + q.numel() * 2 + res.numel() * 4
        out["zoned_decode" + suffix] = _hbm_row("zoned_decode_kernel", cfg["workload"], ms, nbytes,
                                                f"blob {plan.blob_bytes} B, {reps} replicas rotated")
        del blobs, blob
    return out


def time_rdkv(dqa, torch, dev):
    """RDKV allocation on the mixed-width cache's shape (2 sequences, 32
    query heads over 8 KV heads, 16384 prefill positions, d = 128): token
    weights (two causal logit passes on the matrix cores, one exponential per
    causal pair and pass), channel weights (one read of q and k), and the
    two Lagrangian allocations; the budgets are the mean widths of that cache's random maps."""
    from workloads import CONFIGS, rdkv_inputs
    cfg = CONFIGS["mixed-width-zoned-16k"]
    B, Hq, Hkv, d, T = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T_old"]
    inp = rdkv_inputs(B, Hq, Hkv, d, T, seed=4, outliers=cfg["outliers"])
    q, k = torch.from_numpy(inp["q"]).to(dev), torch.from_numpy(inp["k"]).to(dev)
    del inp
    scale = 1.0 / math.sqrt(d)
    vm, km = cfg["rdkv_mean_widths"]
    vbud, kbud = int(math.floor(vm * Hkv * T)), int(math.floor(km * Hkv * d))
    wl = cfg["workload"] + "-prefill"
    ws = torch.empty(dqa.lib.rdkv_widths_workspace_bytes(B, Hq, Hkv, T, d), dtype=torch.uint8, device=dev)
    ms_all = _event_ms(torch, lambda i: dqa.rdkv_widths(q, k, scale, vbud, kbud, workspace=ws), 5, warmup=1)
    wst = torch.empty(max(dqa.lib.rdkv_token_weights_workspace_bytes(B, Hq, T), 1), dtype=torch.uint8,
                      device=dev)
    ms = _event_ms(torch, lambda i: dqa.rdkv_token_weights(q, k, scale, workspace=wst), 5, warmup=1)
    pairs = T * (T + 1) // 2
    flop = 2 * 2 * d * pairs * B * Hq
    tf = flop / (ms * 1e-3) / 1e12
    out = {"rdkv_token_weights": {
        "kernel": "rdkv_lse_kernel + rdkv_colsum_kernel", "workload": wl, "us": ms * 1e3, "bound": "mfma",
        "algorithmic_flop": flop, "achieved": tf, "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": tf / MFMA_FP16_PEAK_TFLOPS,
        "exp_per_s": 2 * pairs * B * Hq / (ms * 1e-3),
        "note": "two passes over the causal logits (2 d flop per pair and pass); the exponentials "
                "on the vector ALU, not the matrix cores, set the pace"}}
    wt = dqa.rdkv_token_weights(q, k, scale, workspace=wst)
    vb = dqa.rdkv_allocate(wt.reshape(B, -1), vbud).reshape(B, Hkv, T)
    ms = _event_ms(torch, lambda i: dqa.rdkv_channel_weights(q, k, vb), 10)
    nbytes = q.numel() * 2 + k.numel() * 2 + vb.numel()
    out["rdkv_channel_weights"] = _hbm_row("rdkv_chan_partial_kernel", wl, ms, nbytes)
    wsa = torch.empty(dqa.lib.rdkv_allocate_workspace_bytes(B, Hkv * T), dtype=torch.uint8, device=dev)
    wflat = wt.reshape(B, -1)
    ms = _event_ms(torch, lambda i: dqa.rdkv_allocate(wflat, vbud, workspace=wsa), 20)
    out["rdkv_allocate"] = _hbm_row("rdkv_hist_kernel + rdkv_select_kernel", wl, ms,
                                    wflat.numel() * (4 * 7 + 1),
                                    "value widths of 2 x 131072 tokens; 13 small launches: latency-bound")
    out["rdkv_widths"] = {"workload": wl, "us": ms_all * 1e3,
                          "note": "all three phases in one call (token weights, value widths, channel "
                                  "weights over kept tokens, key widths)"}
    return out


def time_rvq(dqa, torch, dev):
    """Rows a10-a11 on the residual-VQ workload (rvq-llama3.2-3b-8k): encoding of every key
    and value vector (MFMA-bound: 2 N Kc d flop per vector) and decode
    attention from the indices (a few MB per step: latency-bound)."""
    from workloads import CONFIGS, rvq_inputs
    cfg = CONFIGS["rvq-llama3.2-3b-8k"]
    inp = rvq_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T"], cfg["N"], cfg["Kc"], seed=5)
    d, N, Kc = cfg["d"], cfg["N"], cfg["Kc"]
    k = torch.from_numpy(inp["k"]).to(dev).reshape(-1, d)
    v = torch.from_numpy(inp["v"]).to(dev).reshape(-1, d)
    kcb, vcb = torch.from_numpy(inp["k_cb"]).to(dev), torch.from_numpy(inp["v_cb"]).to(dev)
    ws = torch.empty(max(dqa.lib.rvq_encode_workspace_bytes(N, Kc), 1), dtype=torch.uint8, device=dev)

    def encode(i):
        dqa.rvq_encode(k, kcb, workspace=ws)
        dqa.rvq_encode(v, vcb, workspace=ws)
    ms = _event_ms(torch, encode, 10)
    flop = 2 * 2 * k.shape[0] * N * Kc * d
    tf = flop / (ms * 1e-3) / 1e12
    out = {"rvq_encode": {"kernel": "rvq_encode_kernel", "workload": cfg["workload"], "us": ms * 1e3,
                          "bound": "mfma", "algorithmic_flop": flop, "achieved": tf,
                          "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": tf / MFMA_FP16_PEAK_TFLOPS,
                          "note": "keys and values, N stages x Kc codewords each; distances only"}}
    kidx = dqa.rvq_encode(k, kcb, workspace=ws).reshape(cfg["B"], cfg["Hkv"], cfg["T"], N)
    vidx = dqa.rvq_encode(v, vcb, workspace=ws).reshape(cfg["B"], cfg["Hkv"], cfg["T"], N)
    q = torch.from_numpy(inp["q"]).to(dev)
    res = torch.empty(q.shape, dtype=torch.float32, device=dev)
    n = dqa.lib.rvq_decode_attention_workspace_bytes(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], d)
    wsd = torch.zeros(max(n, 1), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(d)
    ms = _event_ms(torch, lambda i: dqa.rvq_decode_attention(q, kidx, vidx, kcb, vcb, scale, out=res,
                                                              workspace=wsd), 50)
    nbytes = 2 * kidx.numel() * 2 + 2 * kcb.numel() * 2 + q.numel() * 2 + res.numel() * 4
    out["rvq_decode"] = _hbm_row("rvq_decode_kernel", cfg["workload"], ms, nbytes,
                                 "indices + codebooks (4 MB per step): latency-bound, not HBM")
    return out


def time_decode(dqa, torch, dev, cfg, bits, replicas, steps, warmup, inp=None):
    """One decode step = one decode_attention_qkv call (one kernel, which
    also merges the splits), over `replicas` independent copies of the
    quantized cache (rotated so that the working set exceeds the 256 MB
    Infinity Cache).  Returns the step time from HIP events around `steps`
    steps; the kernel's mean duration over `steps` launches through
    decode_attention_qkv_partial, each between its own pair of events; and
    the rate of the same launches back to back."""
    from workloads import kivi_inputs
    if inp is None:
        inp = kivi_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T_q"], cfg["R"], seed=cfg["seed"],
                          outliers=cfg["outliers"])
    scale = 1.0 / math.sqrt(cfg["d"])
    k = torch.from_numpy(inp["k"]).to(dev)
    v = torch.from_numpy(inp["v"]).to(dev)
    kc, ks, kz = dqa.quantize_pack_k(k, bits)
    vc, vs, vz = dqa.quantize_pack_v(v, bits)
    del k, v
    kr = torch.from_numpy(inp["k_recent"]).to(dev)
    vr = torch.from_numpy(inp["v_recent"]).to(dev)
    q = torch.from_numpy(inp["q"]).to(dev)
    caches = []
    for _ in range(replicas):
        t = [x.clone() for x in (kc, ks, kz, vc, vs, vz)]
        t += [x.clone() if x.shape[2] > 0 else None for x in (kr, vr)]
        caches.append(dqa.KiviCache(cfg["Hq"], bits, *t, rope_theta=cfg["rope_theta"], T_q=cfg["T_q"],
                                    B=cfg["B"], Hkv=cfg["Hkv"], d=cfg["d"]))
    del kc, ks, kz, vc, vs, vz
    out = torch.empty((cfg["B"], cfg["Hq"], cfg["d"]), dtype=torch.float32, device=dev)
    ws = [c.workspace(dev) for c in caches]
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    def step(i):
        dqa.decode_attention_qkv(q, caches[i % len(caches)], scale, out=out, workspace=ws[i % len(ws)])

    def split_only(i):
        dqa.decode_attention_qkv_partial(q, caches[i % len(caches)], scale, out, ws[i % len(ws)])

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fn in (("step_ms", step), ("kernel_ms_back_to_back", split_only)):
        _warm(torch, fn, warmup)
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    # the kernel's own duration: every launch between its own pair of
    # events, which order the launches one after the other as the profiler's
    # kernel trace does (back to back, a launch's last workgroups overlap the
    # next launch's first ones)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    _warm(torch, split_only, warmup)
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        split_only(i)
        b.record(stream)
    torch.cuda.synchronize()
    res["kernel_ms"] = sum(a.elapsed_time(b) for a, b in evs) / steps
    nbytes = algorithmic_bytes(cfg, bits)
    res["algorithmic_bytes"] = nbytes
    res["kv_tokens"] = cfg["B"] * (cfg["T_q"] + cfg["R"])
    res["replica_bytes"] = nbytes
    del caches, ws
    return res


def decode_kernel_name(cfg):
    """The split kernel the library picks: the rotated-feature product for
    2/4-bit caches with RoPE, the dequantize-then-rotate kernel otherwise."""
    return "kivi_feat_kernel" if cfg["rope_theta"] > 0 else "kivi_decode_kernel"


def _decode_row(cfg, bits, r):
    gbps = r["algorithmic_bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
    return {"kernel": decode_kernel_name(cfg), "workload": cfg["workload"], "bits": bits,
            "us_per_step": r["step_ms"] * 1e3, "kv_tokens_per_s": r["kv_tokens"] / (r["step_ms"] * 1e-3),
            "kernel_us": r["kernel_ms"] * 1e3, "bound": "hbm", "algorithmic_bytes": r["algorithmic_bytes"],
            "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
            "kernel_us_back_to_back": r["kernel_ms_back_to_back"] * 1e3,
            "note": "kernel_us: mean duration of launches of the split-phase entry point, each between its "
                    "own events; us_per_step: decode_attention_qkv calls back to back"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--bits", type=int, default=2, choices=[2, 4])
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip timing the other hot-path rows (quantize, zoned, RVQ, other decode shapes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the decode path shards "
              f"by (batch, KV head) with no communication", file=sys.stderr)
        return 2

    import torch
    import dequant_decode_attention_amd as dqa
    from workloads import CONFIGS, kivi_inputs

    cfg = CONFIGS["llama3.1-8b-gqa-32k"]
    bits = args.bits
    dev = torch.device("cuda:0")
    inp = kivi_inputs(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T_q"], cfg["R"], seed=cfg["seed"],
                      outliers=cfg["outliers"])
    scale = 1.0 / math.sqrt(cfg["d"])
    rows = {}
    if not args.no_rows:
        k = torch.from_numpy(inp["k"]).to(dev)
        v = torch.from_numpy(inp["v"]).to(dev)
        rows.update(time_quantize(dqa, torch, k, v, bits, cfg))
        del k, v
    r = time_decode(dqa, torch, dev, cfg, bits, args.replicas, args.steps, args.warmup, inp)
    ms, kernel_ms, nbytes = r["step_ms"], r["kernel_ms"], r["algorithmic_bytes"]
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    traffic = measured_traffic(bits)
    line = {
        "metric": "decode attention KV-tokens/s over a 2-bit cache (+ achieved HBM GB/s, % of peak)"
                  if bits == 2 else "decode attention KV-tokens/s over a 4-bit cache",
        "value": r["kv_tokens"] / (ms * 1e-3),
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 matrix-core operands (keys and query split hi+lo, fp16 p*scale for values), "
                 "fp32 accumulation and softmax",
        "data": "synthetic",
        "config": {"workload": cfg["workload"], "batch": cfg["B"], "q_heads": cfg["Hq"],
                   "kv_heads": cfg["Hkv"], "head_dim": cfg["d"], "quantized_tokens": cfg["T_q"],
                   "recent_tokens": cfg["R"], "bits": bits, "group": 32,
                   "rope_theta": cfg["rope_theta"], "replicas": args.replicas},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes": nbytes, "kernel": decode_kernel_name(cfg),
                     "kernel_ms": kernel_ms,
                     "kernel_ms_from": "mean over launches of the split-phase entry point, each between "
                                       "its own HIP events (launches one after the other, as in the "
                                       "kernel trace)",
                     "kernel_ms_back_to_back": r["kernel_ms_back_to_back"]},
    }
    # the vector-ALU issue rate the same kernel sustains (its instruction
    # count per launch from the committed counter summary)
    valu = measured_traffic(bits, "valu_instructions_per_launch_{bits}bit")
    if valu is not None:
        rate = valu / (kernel_ms * 1e-3) / 1e9
        line["roofline"]["valu"] = {"instructions": valu, "achieved": rate, "peak": VALU_PEAK_GINST,
                                    "unit": "G wave-instructions/s", "frac": rate / VALU_PEAK_GINST}

    # achievable streaming rate on a buffer of the same size, same run
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    src = torch.empty(nbytes // 16 * 16 * 4, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dqa.stream_copy(src, dst)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(10):
        dqa.stream_copy(src, dst)
    e1.record(stream)
    torch.cuda.synchronize()
    line["stream_copy_gbps"] = 2 * src.numel() * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst

    if not args.no_rows:
        # the other decode shapes: the same workload at the other width, and
        # the Llama-2-13B-shaped MHA layer (no RoPE)
        other = 4 if bits == 2 else 2
        rows[f"decode_{other}bit"] = _decode_row(cfg, other, time_decode(dqa, torch, dev, cfg, other,
                                                                        args.replicas, args.steps,
                                                                        args.warmup, inp))
        c2 = CONFIGS["llama2-13b-decode-layer"]
        rows["decode_llama2_13b"] = _decode_row(c2, 2, time_decode(dqa, torch, dev, c2, 2, args.replicas,
                                                                   args.steps, args.warmup))
        rows.update(time_append(dqa, torch, dev, cfg, bits))
        rows.update(time_zoned(dqa, torch, dev))
        rows.update(time_rvq(dqa, torch, dev))
        rows.update(time_rdkv(dqa, torch, dev))
        line["rows"] = rows
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, cfg, bits, scale)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
