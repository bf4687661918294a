"""Shared helpers of the GPU parity tests: run the HIP path through the
binding and the oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import sys

import numpy as np

import gqa_inputs as GI
from oracle import gqa_oracle as O

# Tolerances of the workload statement: bf16 storage with fp32 accumulation
# against the exact result, and fp32 configs.
TOL = {"bf16": (2e-2, 5e-3), "f32": (1e-4, 1e-4)}


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    denom = float(np.abs(ref).sum())
    mean_rel = float(diff.sum() / denom) if denom > 0 else float(diff.sum())
    return max_abs, mean_rel


def assert_close(got, ref, dtype: str, what: str):
    max_abs, mean_rel = errors(got, ref)
    tol_abs, tol_rel = TOL[dtype]
    print(f"  {what}: max_abs={max_abs:.3e} mean_rel={mean_rel:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_abs <= tol_abs and mean_rel <= tol_rel, \
        f"{what}: max_abs {max_abs:.3e} (tol {tol_abs}) mean_rel {mean_rel:.3e} (tol {tol_rel})"
    return max_abs, mean_rel


def announce(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def cfg_of(w: GI.Workload, out_f32: bool = True, o_split=None, o_fp16=None):
    """The binding's config for a workload, with the workload's own launch
    options.  Parity runs take the o_proj output in fp32 (the accumulator):
    a bf16 output is that value rounded once more, checked bit-exactly in
    its own test."""
    import transformer_attention_layer_amd as T
    return T.GQAConfig(hidden_size=w.hidden, num_heads=w.hq, num_kv_heads=w.hkv,
                       head_dim=w.head_dim, rope_theta=w.rope_theta, rms_eps=w.rms_eps,
                       qk_norm=w.qk_norm, causal=w.causal, dtype=w.dtype, out_f32=out_f32,
                       o_split=w.o_split if o_split is None else o_split,
                       o_fp16=w.o_fp16 if o_fp16 is None else o_fp16,
                       rotary_dim=w.rotary_dim)


def resolved(w: GI.Workload):
    return O.resolve_config(w.hidden, w.hq, w.hkv, w.head_dim)


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def oracle_layer(w: GI.Workload, h: dict, cache=None, cache_len=None, dtype=np.float64):
    return O.layer_forward(resolved(w), h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"],
                           h["w_o"], rope_theta=w.rope_theta, rms_eps=w.rms_eps,
                           qk_norm=w.qk_norm, causal=w.causal,
                           k_cache=None if cache is None else cache["k_cache"],
                           v_cache=None if cache is None else cache["v_cache"],
                           cache_len=cache_len, rotary_dim=w.rotary_dim, dtype=dtype)
