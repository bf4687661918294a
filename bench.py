#!/usr/bin/env python3
"""Benchmark of the GQA layer forward on one MI355X.

One step = one ``gqa_layer_forward`` call (fused QKV projection with QK-norm
and RoPE, causal grouped attention, o_proj) over one batch of synthetic
input already resident in HBM.  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                  [--no-extra] [--no-decode] [--no-train] [--no-peaks]

The default workload is the largest prefill that the metric is quoted on:
batch 2 x 16384 tokens, hidden 5120, 64 query / 8 KV heads, head_dim 128
(8192-wide attention, wider than the residual).  ``value`` is its prefill
TFLOP/s (algorithmic FLOPs: QKV GEMM + unmasked causal QK^T and PV +
o_proj).  The same line carries:
- ``prefill``: the 8 x 2048 (hidden 1024) and 4 x 8192 (hidden 4096,
  head_dim from the quotient) prefills, each with its own roofline;
- ``decode``: KV GB/s of 64 sequences x 1 token against 32768-token caches
  (GQA and MQA, bf16 and FP8 caches), each with its own roofline;
- ``training``: forward-with-saved-activations and backward at 8 x 2048;
- ``measured_peaks``: the box's bf16 MFMA and streaming-read rates from the
  library's own microkernels (``libgqa_peaks.so``);
- ``roofline`` for the dominant kernel of the headline workload;
- ``cpu_baseline``: the CPU oracle (float32 numpy) timed on a bounded
  sample of the headline workload, extrapolated, and ``cpu_baselines`` for
  the other workloads.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GQA layer prefill TFLOP/s (bf16, % MFMA peak); decode KV GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

DEFAULT_WORKLOAD = "wide_h5120"
EXTRA_PREFILL = ("prefill_h1024", "quotient_h4096")
# MQA first: measured after the GQA workload's 8 GiB of caches were
# allocated and freed, its 1 GiB cache streamed about 4% slower.  (The
# decode records run before the prefills for the same reason.)
DECODE_WORKLOADS = ("decode_h2560_mqa", "decode_h2560_gqa", "decode_h2560_gqa_fp8",
                    "decode_h2560_mqa_fp8")
TRAIN_WORKLOAD = "prefill_h1024"


def flops_of(w):
    """Algorithmic FLOPs of one layer step: 2*T*H*N_qkv + 4*B*Hq*d*(causal
    pairs) + 2*T*Hq*d*H.  Causal pairs of a prefill without cache:
    L(L+1)/2 per sequence and head; with a cache of n tokens: sum over the
    new tokens of (n + i + 1)."""
    d = w.d
    T = w.batch * w.seq
    n_qkv = (w.hq + 2 * w.hkv) * d
    qkv = 2.0 * T * w.hidden * n_qkv
    if w.causal:
        pairs = sum(w.cache_len + i + 1 for i in range(w.seq))
    else:
        pairs = w.seq * (w.cache_len + w.seq)
    attn = 4.0 * w.batch * w.hq * d * pairs
    oproj = 2.0 * T * w.hq * d * w.hidden
    return {"qkv": qkv, "attn": attn, "oproj": oproj, "total": qkv + attn + oproj}


def bwd_flops_of(w):
    """Algorithmic FLOPs of the layer backward: each projection's input and
    weight gradients (two products the size of its forward), and the
    attention's five products over the visible pairs (scores recomputed,
    dP, dV, dQ, dK) where the forward has two."""
    f = flops_of(w)
    qkv, oproj, attn = 2.0 * f["qkv"], 2.0 * f["oproj"], 2.5 * f["attn"]
    return {"qkv": qkv, "attn": attn, "oproj": oproj, "total": qkv + attn + oproj}


def kv_bytes_of(w):
    """Bytes of K and V a decode step must read: every valid row of the
    cache including the appended one, for every sequence and KV head."""
    el = 1 if w.kv_fp8 else 2 if w.dtype == "bf16" else 4
    return 2.0 * w.batch * w.hkv * (w.cache_len + w.seq) * w.d * el


KERNEL_OF_PART = {"qkv": "qkv_gemm", "attn": "attn_prefill", "oproj": "oproj_gemm",
                  "attn_decode": "attn_decode"}


def kernel_of_part(w, part: str) -> str:
    """Kernel that runs a layer part for a workload, by the library's path
    rules: the fused QKV epilogue needs bf16, head_dim 128 and a rotary width
    of 64 or 128 (else projection GEMM + separate norm/RoPE pass); matrix-core
    attention needs bf16 and head_dim 64, 128 or 256 (else the vector-unit
    attention)."""
    rot = w.rotary_dim or w.d
    if part == "qkv" and not (w.dtype == "bf16" and w.d == 128 and rot in (64, 128)):
        return "qkv_gemm_normrope"
    if part in ("attn", "attn_decode") and not (w.dtype == "bf16" and w.d in (64, 128, 256)):
        return "attn_vec"
    return KERNEL_OF_PART[part]


SOURCES_OF_KERNEL = {"qkv_gemm": ("gemm_bf16.hip",), "oproj_gemm": ("gemm_bf16.hip",),
                     "attn_prefill": ("attn_bf16.hip", "attn_tiles.h"),
                     "attn_decode": ("attn_bf16.hip", "attn_tiles.h"),
                     "qkv_gemm_normrope": ("gemm_bf16.hip", "normrope_rows.hip"),
                     "attn_vec": ("f32_kernels.hip",)}
# MI355X fp32 vector peak as published (it counts packed-fp32 issue; plain
# FMAs, which these kernels use, reach half of it)
PEAK_F32_VALU_TFLOPS = 157.3


def kernel_source_sha(kernel: str) -> str:
    """Hash of the sources a kernel is built from (its file plus the shared
    headers), to tell whether stored counter readings still describe it."""
    import hashlib
    csrc = os.path.join(ROOT, "transformer_attention_layer_amd", "csrc")
    h = hashlib.sha256()
    for f in ("common.h", "kernels.h", *SOURCES_OF_KERNEL[kernel]):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) from the
    committed counter summary, or None when it is missing or was taken on a
    different version of the kernel's source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != kernel_source_sha(kernel):
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def _time_loop(fn, iters, torch):
    """Average ms per call over `iters` calls, timed with HIP events on the
    current stream (the stream the library launches on).  One untimed call
    goes to the stream just before the start event: it keeps the GPU busy
    while the host issues the timed calls, so a short step's timing does not
    include the host's latency to issue the first of them."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    fn()
    start.record()
    for _ in range(iters):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters  # ms


def layer_cfg(T, w, **kw):
    return T.GQAConfig(hidden_size=w.hidden, num_heads=w.hq, num_kv_heads=w.hkv,
                       head_dim=w.head_dim, rope_theta=w.rope_theta, rms_eps=w.rms_eps,
                       qk_norm=w.qk_norm, causal=w.causal, dtype=w.dtype, out_f32=True,
                       o_split=w.o_split, o_fp16=w.o_fp16, rotary_dim=w.rotary_dim, **kw)


def bench_prefill(w, steps, warmup, torch, T, GI):
    """Layer step time, and the time of each entry point (the QKV one is one
    kernel plus its small RoPE table build; attention and o_proj one kernel
    each) on the same stream and inputs.  The layer's own o_proj reads the
    attention output in its carrier format (fp16, or a bf16 hi + lo pair);
    the standalone o_proj reads one bf16 value per element, so the layer's
    o_proj time (with its W_o conversion, for fp16) is reported as the layer
    step minus the QKV and attention entry points."""
    cfg = layer_cfg(T, w)
    h = GI.device_layer_inputs(w)
    d = w.d
    dt = GI.torch_dtype(w)
    kc = torch.zeros((w.batch, w.hkv, w.seq, d), dtype=dt, device="cuda")
    vc = torch.zeros_like(kc)
    out = torch.empty((w.batch, w.seq, w.hidden), dtype=torch.float32, device="cuda")
    ws = T.LayerWorkspace(cfg, w.batch, w.seq, w.seq)

    def step():
        T.gqa_layer_forward(cfg, h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"], h["w_o"],
                            k_cache=kc, v_cache=vc, out=out, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms = _time_loop(step, steps, torch)

    q = torch.empty((w.batch, w.hq, w.seq, d), dtype=dt, device="cuda")
    o = torch.empty((w.batch, w.seq, w.hq * d), dtype=dt, device="cuda")
    parts = {
        "qkv": lambda: T.qkv_proj_normrope(cfg, h["x"], h["w_qkv"], h["q_norm_w"],
                                           h["k_norm_w"], k_cache=kc, v_cache=vc, q=q),
        "attn": lambda: T.gqa_attn_core(cfg, q, kc, vc, o=o),
        "oproj": lambda: T.gqa_o_proj(cfg, o, h["w_o"], out=out),
    }
    part_ms = {}
    for k, fn in parts.items():
        for _ in range(2):
            fn()
        part_ms[k] = _time_loop(fn, steps, torch)
    del ws, q, o, kc, vc, out, h
    torch.cuda.empty_cache()
    return ms, part_ms


def prefill_record(w, steps, warmup, torch, T, GI):
    """TFLOP/s of the layer step and the roofline of its dominant kernel."""
    ms, part_ms = bench_prefill(w, steps, warmup, torch, T, GI)
    fl = flops_of(w)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    value = fl["total"] / (ms * 1e-3) / 1e12
    layer_oproj_ms = ms - part_ms["qkv"] - part_ms["attn"]
    dom = max(part_ms, key=part_ms.get)
    kern = kernel_of_part(w, dom)
    ach = fl[dom] / (part_ms[dom] * 1e-3) / 1e12
    bound, kpeak = "mfma", peak
    if kern == "attn_vec":  # fp32 FMAs on the vector units
        bound, kpeak = "alu", PEAK_F32_VALU_TFLOPS
    rec = {"value": round(value, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 4),
           "frac_of_peak": round(value / peak, 4),
           "kernels_ms": {k: round(v, 4) for k, v in part_ms.items()},
           "layer_oproj_ms": round(layer_oproj_ms, 4),
           "kernels_tflops": {k: round(fl[k] / (v * 1e-3) / 1e12, 1) for k, v in part_ms.items()},
           "roofline": {"bound": bound, "kernel": kern, "achieved": round(ach, 2), "peak": kpeak,
                        "unit": "TFLOP/s", "frac": round(ach / kpeak, 4),
                        "traffic": stored_traffic(w.name, kern), "algorithmic_flop": fl[dom],
                        "avg_launch_ms": round(part_ms[dom], 5)}}
    return rec


def bench_train(w, steps, warmup, torch, T, GI):
    """The training pair on a prefill workload: gqa_layer_forward_train
    (which also keeps q, k, v, o, the fp32 projection and the row
    log-sum-exps) and gqa_layer_backward, each timed over `steps` calls."""
    cfg = layer_cfg(T, w)
    h = GI.device_layer_inputs(w)
    dout = GI.device_upstream_grad(w)
    out = torch.empty((w.batch, w.seq, w.hidden), dtype=torch.float32, device="cuda")
    saved = T.TrainSaved(cfg, w.batch, w.seq)
    ws = T.BackwardWorkspace(cfg, w.batch, w.seq)
    args5 = (cfg, h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"], h["w_o"])

    def fwd():
        T.gqa_layer_forward_train(*args5, saved=saved, out=out)

    fwd()
    grads = T.gqa_layer_backward(*args5, saved, dout, workspace=ws)

    def bwd():
        T.gqa_layer_backward(*args5, saved, dout, grads=grads, workspace=ws)

    for _ in range(warmup):
        fwd()
        bwd()
    fwd_ms = _time_loop(fwd, steps, torch)
    bwd_ms = _time_loop(bwd, steps, torch)
    del saved, ws, grads
    torch.cuda.empty_cache()
    return fwd_ms, bwd_ms


def bench_decode(w, steps, warmup, torch, T, GI):
    cfg = layer_cfg(T, w, kv_fp8=w.kv_fp8)
    h = GI.device_layer_inputs(w)
    c = GI.device_cache(w)
    cl = torch.full((w.batch,), w.cache_len, dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.seq, w.hidden), dtype=torch.float32, device="cuda")
    ws = T.LayerWorkspace(cfg, w.batch, w.seq, w.kv_capacity)

    def step():
        # the append rewrites the same row every step: the cache does not grow
        T.gqa_layer_forward(cfg, h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"], h["w_o"],
                            k_cache=c["k_cache"], v_cache=c["v_cache"], cache_len=cl, out=out,
                            workspace=ws)

    for _ in range(warmup):
        step()
    ms = _time_loop(step, steps, torch)
    q = torch.empty((w.batch, w.hq, w.seq, w.d), dtype=GI.torch_dtype(w), device="cuda")
    kvl = cl + w.seq
    o = torch.empty((w.batch, w.seq, w.hq * w.d), dtype=GI.torch_dtype(w), device="cuda")
    T.qkv_proj_normrope(cfg, h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"], start_pos=cl,
                        k_cache=c["k_cache"], v_cache=c["v_cache"], q=q)

    def attn():
        T.gqa_attn_core(cfg, q, c["k_cache"], c["v_cache"], kv_len=kvl, o=o)

    for _ in range(2):
        attn()
    attn_ms = _time_loop(attn, steps, torch)
    del c
    torch.cuda.empty_cache()
    return ms, attn_ms


def decode_record(w, steps, warmup, torch, T, GI):
    ms, attn_ms = bench_decode(w, steps, warmup, torch, T, GI)
    kvb = kv_bytes_of(w)
    gbs = kvb / (attn_ms * 1e-3) / 1e9
    return {"kv_gb_per_s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "attn_ms": round(attn_ms, 4), "layer_ms": round(ms, 4), "kv_bytes": kvb,
            "roofline": {"bound": "hbm", "kernel": "attn_decode", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": stored_traffic(w.name, "attn_decode"),
                         "algorithmic_bytes": kvb, "avg_launch_ms": round(attn_ms, 5)}}


def measured_peaks(torch):
    """What this machine delivers to the library's own microkernels
    (libgqa_peaks.so): a bf16 MFMA-only loop (4 waves per workgroup, 1024
    workgroups, 8 independent 32x32x16 MFMAs per trip) and a streaming read
    of 4 GiB (16-byte nontemporal loads, each byte once, 8192 workgroups).  Each is the best of 5 timed
    calls after 2 untimed ones, timed with HIP events on the launch stream."""
    from transformer_attention_layer_amd import peaks as P

    def best_ms(fn, n=5):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b))
        return min(times)
    wg, iters = 1024, 4000
    sink = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    flop = 4.0 * wg * iters * P.MFMA_FLOP_PER_WAVE_ITER
    mfma_ms = best_ms(lambda: P.mfma_bf16(wg, iters, sink))
    buf = torch.empty(1 << 32, dtype=torch.uint8, device="cuda")
    rwg = 8192  # the fastest of 1024 .. 16384 workgroups on an MI355X
    rsink = torch.empty(rwg * 256, dtype=torch.int32, device="cuda")
    read_ms = best_ms(lambda: P.stream_read(buf, rwg, rsink))
    del buf, sink, rsink
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(flop / (mfma_ms * 1e-3) / 1e12, 1),
            "mfma": f"gqa_peak_mfma_bf16: {wg} workgroups x 4 waves x {iters} trips of 8 "
                    "independent v_mfma_f32_32x32x16_bf16, best of 5",
            "hbm_read_gbs": round((1 << 32) / (read_ms * 1e-3) / 1e9, 1),
            "read": f"gqa_peak_stream_read: 4 GiB, {rwg} workgroups, 16-byte loads, best of 5"}


# ---------------------------------------------------------------------------
# CPU oracle baselines (test infrastructure: only this leg of the bench may
# call the oracle; it runs after every GPU measurement)
# ---------------------------------------------------------------------------

def _cores_and_blas():
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]["name"]
    except Exception:  # pragma: no cover
        blas = "unknown"
    return int(cores), blas


ROWS_PER_SEQUENCE = 2048  # oracle rows per sequence in the row-sampled CPU baseline


def sampled_rows(L: int, n: int = 256, head: int = 64):
    """The first `head` positions, the last, and an even stride between."""
    import numpy as np
    if L <= n:
        return list(range(L))
    rest = np.linspace(head, L - 1, n - head).round().astype(int)
    return sorted(set(range(head)) | set(int(t) for t in rest))


def cpu_prefill(w, budget_s):
    """The oracle, as it stands, in float32 (the precision the tutorial's
    attention step names) on a bounded sample of the workload.

    Sequences of up to 2048 tokens: whole sequences through
    ``layer_forward``, as many as fit the budget (at least one).  Longer
    ones: ``layer_forward_rows`` on 2048 rows per sequence (its first 64
    tokens, its last, an even stride between), which projects K and V for
    the whole sequence and runs Q, attention and o_proj for the sampled
    rows.  The rate is the algorithmic FLOPs of what the sample computed
    over its time; the whole workload's time at that rate is given as
    ``extrapolated_full_s``."""
    import numpy as np
    import gqa_inputs as GI
    from oracle import gqa_oracle as O
    cores, blas = _cores_and_blas()
    res = O.resolve_config(w.hidden, w.hq, w.hkv, w.head_dim)
    one = w.with_(batch=1)
    full = w.seq <= 2048
    done, elapsed, fl, nrows = 0, 0.0, 0.0, 0
    wall0 = time.perf_counter()  # the budget bounds wall time, input generation included
    while done < w.batch and (done == 0 or time.perf_counter() - wall0 < budget_s):
        h = GI.host_layer_inputs(one, seed=w.seed + 100 + done)
        if full:
            t0 = time.perf_counter()
            O.layer_forward(res, h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"], h["w_o"],
                            rope_theta=w.rope_theta, rms_eps=w.rms_eps, qk_norm=w.qk_norm,
                            causal=w.causal, dtype=np.float32)
            elapsed += time.perf_counter() - t0
            fl += flops_of(one)["total"]
        else:
            ts = sampled_rows(w.seq, n=ROWS_PER_SEQUENCE)
            rows = [(0, t) for t in ts]
            t0 = time.perf_counter()
            O.layer_forward_rows(res, h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"],
                                 h["w_o"], rows, rope_theta=w.rope_theta, rms_eps=w.rms_eps,
                                 qk_norm=w.qk_norm, rotary_dim=w.rotary_dim, dtype=np.float32)
            elapsed += time.perf_counter() - t0
            n = len(ts)
            kv = 2.0 * w.seq * w.hidden * 2 * w.hkv * w.d
            qp = 2.0 * n * w.hidden * w.hq * w.d
            att = 4.0 * w.hq * w.d * sum(t + 1 for t in ts)
            op = 2.0 * n * w.hq * w.d * w.hidden
            fl += kv + qp + att + op
            nrows += n
        done += 1
    rate = fl / elapsed
    rec = {"value": rate / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "host_cpus": os.cpu_count(), "blas": blas, "precision": "float32",
           "extrapolated_full_s": round(flops_of(w)["total"] / rate, 2)}
    if full:
        rec["sample"] = (f"{done} of {w.batch} whole sequences ({w.seq} tokens each), "
                         f"float32 numpy, {elapsed:.1f} s")
    else:
        rec["sample"] = (f"{nrows} rows of {done} of {w.batch} sequences "
                         f"({ROWS_PER_SEQUENCE} per sequence: "
                         f"t=0..63, t={w.seq - 1} and a stride; K/V projected for all {w.seq} "
                         f"tokens), float32 numpy, {elapsed:.1f} s; rate extrapolated to the "
                         "whole workload")
    return rec


def cpu_decode(w, budget_s):
    """The oracle's decode step (float32) on a few of the 64 sequences, each
    with its own host cache of the workload's length; the KV GB/s counts the
    cache bytes of the sampled sequences (the workload's element size) and
    the whole step's time is extrapolated by the sequence count."""
    import numpy as np
    import gqa_inputs as GI
    from oracle import gqa_oracle as O
    cores, blas = _cores_and_blas()
    res = O.resolve_config(w.hidden, w.hq, w.hkv, w.head_dim)
    one = w.with_(batch=1, kv_fp8=False)
    done, elapsed = 0, 0.0
    wall0 = time.perf_counter()  # the budget bounds wall time, input generation included
    while done < w.batch and (done == 0 or time.perf_counter() - wall0 < budget_s):
        h = GI.host_layer_inputs(one, seed=w.seed + 100 + done)
        c = GI.host_cache(one, seed=w.seed + 100 + done, fill_unused=0.0)
        kw = {}
        kc, vc = c["k_cache"], c["v_cache"]
        if w.kv_fp8:
            kc, vc = O.quantize_e4m3(kc), O.quantize_e4m3(vc)
            kw = {"kv_fp8": True}
        t0 = time.perf_counter()
        O.layer_forward(res, h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"], h["w_o"],
                        rope_theta=w.rope_theta, rms_eps=w.rms_eps, qk_norm=w.qk_norm,
                        k_cache=kc, v_cache=vc, cache_len=np.array([w.cache_len]),
                        dtype=np.float32, **kw)
        elapsed += time.perf_counter() - t0
        done += 1
    gbs = kv_bytes_of(one) * done / elapsed / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "host_cpus": os.cpu_count(), "blas": blas, "precision": "float32",
            "extrapolated_full_s": round(elapsed / done * w.batch, 2),
            "sample": f"{done} of {w.batch} sequences (cache {w.cache_len} tokens), float32 "
                      f"numpy, {elapsed:.1f} s; KV bytes counted at the workload's element size"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other prefill workloads")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the training forward + backward timing")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured MFMA / read microkernels")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer's multi-GPU sharding is a design, not a built path)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gqa_inputs as GI
    import transformer_attention_layer_amd as T
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    T.lib()

    w = GI.WORKLOADS[args.workload]
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": w.dtype, "data": "synthetic (seeded N(0,1) activations, N(0,0.02) "
              "weights, random init; no trained checkpoint)"}
    cfgd = {"workload": w.name, "batch": w.batch, "seq_len": w.seq, "hidden": w.hidden,
            "num_heads": w.hq, "num_kv_heads": w.hkv, "head_dim": w.d,
            "head_dim_explicit": w.head_dim is not None, "qk_norm": w.qk_norm,
            "rope_theta": w.rope_theta, "causal": w.causal, "cache_len": w.cache_len,
            "out_dtype": "f32", "o_split": w.o_split, "o_fp16": w.o_fp16,
            "kv_cache": "fp8_e4m3" if w.kv_fp8 else w.dtype}
    # The decode records run first, on allocations made before the prefills'
    # several GiB come and go, as a serving process allocates its KV cache
    # at start-up: caches allocated after large frees streamed about 4%
    # slower.
    dec = {}
    if not args.no_decode:
        for name in DECODE_WORKLOADS:
            if name == w.name:
                continue
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            dec[name] = decode_record(GI.WORKLOADS[name], args.steps, args.warmup, torch, T, GI)

    print(f"[bench] {w.name}", file=sys.stderr, flush=True)
    if w.cache_len == 0:
        rec = prefill_record(w, args.steps, args.warmup, torch, T, GI)
    else:
        rec = decode_record(w, args.steps, args.warmup, torch, T, GI)
        rec = {"value": rec["kv_gb_per_s"], "unit": "GB/s", "ms_per_step": rec["layer_ms"],
               "attn_ms": rec["attn_ms"], "roofline": rec["roofline"]}
    roof = rec.pop("roofline")
    result.update(rec)
    result["config"] = cfgd
    result["roofline"] = roof

    if not args.no_extra:
        pre = {}
        for name in EXTRA_PREFILL:
            if name == w.name:
                continue
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            pre[name] = prefill_record(GI.WORKLOADS[name], args.steps, args.warmup, torch, T, GI)
        result["prefill"] = pre

    tw = GI.WORKLOADS[TRAIN_WORKLOAD]
    if not args.no_train:
        print(f"[bench] training {tw.name}", file=sys.stderr, flush=True)
        fwd_ms, bwd_ms = bench_train(tw, args.steps, args.warmup, torch, T, GI)
        fb = bwd_flops_of(tw)
        ff = flops_of(tw)
        bt = fb["total"] / (bwd_ms * 1e-3) / 1e12
        result["training"] = {
            "workload": tw.name,
            "forward_train_ms": round(fwd_ms, 4), "backward_ms": round(bwd_ms, 4),
            "backward_tflops": round(bt, 2), "backward_frac_of_peak": round(bt / PEAK_BF16_TFLOPS, 4),
            "step_tflops": round((ff["total"] + fb["total"]) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 2),
            "backward_algorithmic_flop": fb["total"]}

    if not args.no_decode:
        result["decode"] = dec

    if not args.no_peaks:
        print("[bench] measured peaks", file=sys.stderr, flush=True)
        mp = measured_peaks(torch)
        result["measured_peaks"] = mp

        def rel(rl):
            ref = mp["mfma_bf16_tflops"] if rl["bound"] == "mfma" else \
                mp["hbm_read_gbs"] if rl["bound"] == "hbm" else None
            if ref:
                rl["frac_of_measured"] = round(rl["achieved"] / ref, 4)
        rel(result["roofline"])
        for r in result.get("prefill", {}).values():
            rel(r["roofline"])
        for r in result.get("decode", {}).values():
            rel(r["roofline"])

    if args.copy_probe_mb:
        # a plain device-to-device copy of known size, outside the timed
        # region, so that HBM byte counters can be calibrated against it
        n = args.copy_probe_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = n

    if not args.no_cpu_baseline:
        print("[bench] cpu baselines", file=sys.stderr, flush=True)
        if w.cache_len == 0:
            result["cpu_baseline"] = cpu_prefill(w, budget_s=20.0)
        else:
            result["cpu_baseline"] = cpu_decode(w, budget_s=10.0)
        extra = {}
        if not args.no_extra:
            for name in EXTRA_PREFILL:
                if name != w.name:
                    extra[name] = cpu_prefill(GI.WORKLOADS[name], budget_s=8.0)
        if not args.no_decode:
            for name in ("decode_h2560_gqa", "decode_h2560_mqa"):
                if name != w.name:
                    extra[name] = cpu_decode(GI.WORKLOADS[name], budget_s=8.0)
        result["cpu_baselines"] = extra
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
