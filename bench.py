#!/usr/bin/env python3
"""Benchmark of the GQA layer forward on one MI355X.

One step = one ``gqa_layer_forward`` call (fused QKV projection with QK-norm
and RoPE, causal grouped attention, o_proj) over one batch of synthetic
input already resident in HBM.  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                  [--no-decode]

The default workload is the bf16 prefill of a Qwen3-0.6B-shaped layer
(batch 8 x 2048 tokens, hidden 1024, 16 query / 8 KV heads, head_dim 128).
``value`` is its prefill TFLOP/s (algorithmic FLOPs: QKV GEMM + unmasked
causal QK^T and PV + o_proj).  The same line carries the decode workloads'
KV GB/s under ``decode`` (64 sequences x 1 token against a 32768-token
cache, GQA and MQA), a ``roofline`` object for the dominant kernel and a
``cpu_baseline`` (the CPU oracle timed on a bounded sample).
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
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(iters):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters  # ms


def bench_prefill(w, steps, warmup, torch, T, GI):
    cfg = T.GQAConfig(hidden_size=w.hidden, num_heads=w.hq, num_kv_heads=w.hkv,
                      head_dim=w.head_dim, rope_theta=w.rope_theta, rms_eps=w.rms_eps,
                      qk_norm=w.qk_norm, causal=w.causal, dtype=w.dtype, out_f32=True,
                      o_split=w.o_split)
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

    # per-entry-point timing (each is one kernel, the QKV one plus its small
    # RoPE table build), same stream, same inputs
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
    return ms, part_ms


def bench_train(w, steps, warmup, torch, T, GI):
    """The training pair on a prefill workload: gqa_layer_forward_train
    (which also keeps q, k, v, o, the fp32 projection and the row
    log-sum-exps) and gqa_layer_backward, each timed over `steps` calls."""
    cfg = T.GQAConfig(hidden_size=w.hidden, num_heads=w.hq, num_kv_heads=w.hkv,
                      head_dim=w.head_dim, rope_theta=w.rope_theta, rms_eps=w.rms_eps,
                      qk_norm=w.qk_norm, causal=w.causal, dtype=w.dtype, out_f32=True,
                      rotary_dim=w.rotary_dim)
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
    cfg = T.GQAConfig(hidden_size=w.hidden, num_heads=w.hq, num_kv_heads=w.hkv,
                      head_dim=w.head_dim, rope_theta=w.rope_theta, rms_eps=w.rms_eps,
                      qk_norm=w.qk_norm, causal=w.causal, dtype=w.dtype, out_f32=True,
                      o_split=w.o_split, kv_fp8=w.kv_fp8)
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


def measured_peaks(torch):
    """What this machine delivers to a library GEMM and to a library streaming
    read, as references beside the vendor peaks: a bf16 8192^3 torch.matmul
    with both operands K-contiguous (the layer's layout; hipBLASLt) and a
    row-sum over 2 GiB of fp32 (8192-wide rows).  Each is the best of 10
    timed calls after 3 untimed ones."""
    def best_ms(fn, n=10):
        for _ in range(3):
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
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    bt = torch.randn(n, n, device="cuda").to(torch.bfloat16)  # [N, K]
    gemm_ms = best_ms(lambda: torch.matmul(a, bt.t()))
    del a, bt
    x = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    read_ms = best_ms(lambda: x.view(-1, 8192).sum(1))
    del x
    torch.cuda.empty_cache()
    return {"gemm_bf16_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "gemm": "torch.matmul bf16 8192^3, A [M,K] x B[N,K]^T (hipBLASLt), best of 10",
            "hbm_read_gbs": round((1 << 31) / (read_ms * 1e-3) / 1e9, 1),
            "read": "torch row-sum over 2 GiB fp32, best of 10"}


def cpu_baseline(w, budget_s=12.0):
    """The oracle, as it is, on a bounded sample: whole sequences of the
    same workload (float64), as many as fit the time budget (at least one).
    Returns TFLOP/s over the sample's algorithmic FLOPs."""
    import numpy as np
    import gqa_inputs as GI
    from oracle import gqa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    one = w.with_(batch=1)
    res = O.resolve_config(w.hidden, w.hq, w.hkv, w.head_dim)
    done = 0
    elapsed = 0.0
    while done < w.batch and (done == 0 or elapsed < budget_s):
        h = GI.host_layer_inputs(one, seed=w.seed + 100 + done)
        t0 = time.perf_counter()
        O.layer_forward(res, h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"], h["w_o"],
                        rope_theta=w.rope_theta, rms_eps=w.rms_eps, qk_norm=w.qk_norm,
                        causal=w.causal)
        elapsed += time.perf_counter() - t0
        done += 1
    fl = flops_of(one)["total"] * done
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]["name"]
    except Exception:  # pragma: no cover
        blas = "unknown"
    return {"value": fl / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "host_cpus": os.cpu_count(), "blas": blas,
            "sample": f"{done} of {w.batch} sequences ({one.seq} tokens each), float64 numpy, "
                      f"{elapsed:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_h1024")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the training forward + backward timing")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured GEMM / read references")
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
            "out_dtype": "f32", "o_split": w.o_split,
            "kv_cache": "fp8_e4m3" if w.kv_fp8 else w.dtype}
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    if w.cache_len == 0:
        ms, part_ms = bench_prefill(w, args.steps, args.warmup, torch, T, GI)
        fl = flops_of(w)
        value = fl["total"] / (ms * 1e-3) / 1e12
        dom = max(part_ms, key=part_ms.get)
        ach = fl[dom] / (part_ms[dom] * 1e-3) / 1e12
        result.update({"value": round(value, 2), "unit": "TFLOP/s",
                       "ms_per_step": round(ms, 4), "frac_of_peak": round(value / peak, 4)})
        result["config"] = cfgd
        result["kernels_ms"] = {k: round(v, 4) for k, v in part_ms.items()}
        kern = kernel_of_part(w, dom)
        bound, kpeak = "mfma", peak
        if kern == "attn_vec":  # fp32 FMAs on the vector units
            bound, kpeak = "alu", PEAK_F32_VALU_TFLOPS
        result["roofline"] = {"bound": bound, "kernel": kern, "achieved": round(ach, 2),
                              "peak": kpeak, "unit": "TFLOP/s", "frac": round(ach / kpeak, 4),
                              "traffic": stored_traffic(w.name, kern),
                              "algorithmic_flop": fl[dom], "avg_launch_ms": round(part_ms[dom], 5)}
    else:
        ms, attn_ms = bench_decode(w, args.steps, args.warmup, torch, T, GI)
        kvb = kv_bytes_of(w)
        gbs = kvb / (attn_ms * 1e-3) / 1e9
        result.update({"value": round(gbs, 1), "unit": "GB/s", "ms_per_step": round(ms, 4)})
        result["config"] = cfgd
        result["roofline"] = {"bound": "hbm", "kernel": "attn_decode", "achieved": round(gbs, 1),
                              "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": round(gbs / PEAK_HBM_GBS, 4),
                              "traffic": stored_traffic(w.name, "attn_decode"),
                              "algorithmic_bytes": kvb, "avg_launch_ms": round(attn_ms, 5)}

    if w.cache_len == 0 and not args.no_train and w.dtype == "bf16" and w.d in (64, 128) \
            and not w.o_split:
        fwd_ms, bwd_ms = bench_train(w, args.steps, args.warmup, torch, T, GI)
        fb = bwd_flops_of(w)
        ff = flops_of(w)
        bt = fb["total"] / (bwd_ms * 1e-3) / 1e12
        result["training"] = {
            "forward_train_ms": round(fwd_ms, 4), "backward_ms": round(bwd_ms, 4),
            "backward_tflops": round(bt, 2), "backward_frac_of_peak": round(bt / peak, 4),
            "step_tflops": round((ff["total"] + fb["total"]) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 2),
            "backward_algorithmic_flop": fb["total"]}

    if w.cache_len == 0 and not args.no_decode:
        dec = {}
        for name in ("decode_h2560_gqa", "decode_h2560_mqa", "decode_h2560_gqa_fp8",
                     "decode_h2560_mqa_fp8"):
            wd = GI.WORKLOADS[name]
            dms, attn_ms = bench_decode(wd, args.steps, args.warmup, torch, T, GI)
            gbs = kv_bytes_of(wd) / (attn_ms * 1e-3) / 1e9
            dec[name] = {"kv_gb_per_s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                         "attn_ms": round(attn_ms, 4), "layer_ms": round(dms, 4),
                         "kv_bytes": kv_bytes_of(wd)}
        result["decode"] = dec

    if not args.no_peaks:
        mp = measured_peaks(torch)
        result["measured_peaks"] = mp
        rl = result["roofline"]
        ref = mp["gemm_bf16_tflops"] if rl["bound"] == "mfma" else mp["hbm_read_gbs"]
        rl["frac_of_measured"] = round(rl["achieved"] / ref, 4)
        for d in result.get("decode", {}).values():
            d["frac_of_measured_read"] = round(d["kv_gb_per_s"] / mp["hbm_read_gbs"], 4)

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
        result["cpu_baseline"] = cpu_baseline(w) if w.cache_len == 0 else None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
