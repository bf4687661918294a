"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds workload shapes and random-number recipes only: none of
the layer's arithmetic.  Both the HIP path and the CPU oracle are fed from
here, so they see identical values.

Recipe (the pages fix the shapes; the distributions are the workload
statement's): x ~ N(0, 1); projection weights ~ N(0, 0.02); QK-norm weights
~ 1 + N(0, 0.1); decode K/V cache rows ~ N(0, 1).  bf16 workloads round every
input once to bf16 (round to nearest even) so both sides consume the same
values.  Host draws use numpy's PCG64 ``default_rng(seed)`` in the fixed
order x, w_qkv, q_norm_w, k_norm_w, w_o (then k_cache, v_cache).  Device
draws (large bench inputs) use a seeded torch CUDA generator with the same
distributions.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq: int                 # new tokens per sequence
    hidden: int
    hq: int
    hkv: int
    head_dim: Optional[int]  # None: derive hidden // hq
    qk_norm: bool
    rope_theta: float
    rms_eps: float
    dtype: str               # "f32" or "bf16"
    seed: int
    causal: bool = True
    cache_len: int = 0       # decode: tokens already in the cache
    # Launch options of the layer for this workload: how the attention output
    # reaches o_proj.  For the layers whose o_proj reduces over Hq*d >= 4096
    # values, where the bf16 rounding of the attention output alone moves
    # outputs by ~1e-2, it is carried either as fp16 (prefill: one fp16
    # o_proj pass over W_o converted to fp16) or as a bf16 hi + lo pair
    # (decode: a few tokens, where reading W_o twice costs less than
    # converting it).
    o_split: bool = False
    rotary_dim: Optional[int] = None  # partial rotary width; None = head_dim
    kv_fp8: bool = False      # K/V caches hold FP8 (E4M3) codes, scales 1
    o_fp16: bool = False

    @property
    def d(self) -> int:
        return self.head_dim if self.head_dim is not None else self.hidden // self.hq

    @property
    def kv_capacity(self) -> int:
        return self.cache_len + self.seq

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The workloads the layer is measured and checked on.  Shapes follow the
# models the pages discuss (Qwen3-0.6B-like, Qwen3-8B/32B-like quotient path,
# a wide 64-head layer, Qwen3-4B-like decode).
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 64, 256, 4, 2, 128, True, 1e6, 1e-6,
                         "f32", 0),
    "prefill_h1024": Workload("prefill_h1024", 8, 2048, 1024, 16, 8, 128, True,
                              1e6, 1e-6, "bf16", 1),
    "quotient_h4096": Workload("quotient_h4096", 4, 8192, 4096, 32, 8, None,
                               False, 5e5, 1e-6, "bf16", 2, o_fp16=True),
    "wide_h5120": Workload("wide_h5120", 2, 16384, 5120, 64, 8, 128, True, 1e6,
                           1e-6, "bf16", 3, o_fp16=True),
    "decode_h2560_gqa": Workload("decode_h2560_gqa", 64, 1, 2560, 32, 8, 128,
                                 True, 1e6, 1e-6, "bf16", 4, cache_len=32768,
                                 o_fp16=True),
    "decode_h2560_mqa": Workload("decode_h2560_mqa", 64, 1, 2560, 32, 1, 128,
                                 True, 1e6, 1e-6, "bf16", 4, cache_len=32768,
                                 o_fp16=True),
    # The decode workloads with FP8 (E4M3) K/V caches: half the cache bytes.
    "decode_h2560_gqa_fp8": Workload("decode_h2560_gqa_fp8", 64, 1, 2560, 32, 8, 128, True,
                                     1e6, 1e-6, "bf16", 4, cache_len=32768, o_fp16=True,
                                     kv_fp8=True),
    "decode_h2560_mqa_fp8": Workload("decode_h2560_mqa_fp8", 64, 1, 2560, 32, 1, 128, True,
                                     1e6, 1e-6, "bf16", 4, cache_len=32768, o_fp16=True,
                                     kv_fp8=True),
    # The explicit head_dim the pages cite for Gemma 3 (hidden 640, four
    # query heads, head_dim 256 rather than 160); one KV head.  Runs the
    # matrix-core attention, with the projection GEMM followed by a separate
    # norm/RoPE pass.
    "gemma_h640_d256": Workload("gemma_h640_d256", 4, 2048, 640, 4, 1, 256, True,
                                1e6, 1e-6, "bf16", 5),
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 holding exactly representable bf16 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # bits + 0x7FFF + (lowest kept bit), truncated: in 32-bit lanes, in place
    r = u >> 16
    r &= 1
    r += 0x7FFF
    r += u
    r &= 0xFFFF0000
    return r.view(np.float32).reshape(a.shape)


def _finish(a: np.ndarray, dtype: str) -> np.ndarray:
    a = a.astype(np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def host_layer_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """x [B, L, hidden], w_qkv [(Hq+2Hkv)d, hidden] (rows Q | K | V),
    q_norm_w [d], k_norm_w [d], w_o [hidden, Hq*d], all float32 arrays."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    d = w.d
    n_qkv = (w.hq + 2 * w.hkv) * d
    x = rng.standard_normal((w.batch, w.seq, w.hidden), dtype=np.float32)
    w_qkv = rng.standard_normal((n_qkv, w.hidden), dtype=np.float32) * 0.02
    qn = 1.0 + rng.standard_normal(d, dtype=np.float32) * 0.1
    kn = 1.0 + rng.standard_normal(d, dtype=np.float32) * 0.1
    w_o = rng.standard_normal((w.hidden, w.hq * d), dtype=np.float32) * 0.02
    return {"x": _finish(x, w.dtype), "w_qkv": _finish(w_qkv, w.dtype),
            "q_norm_w": _finish(qn, w.dtype), "k_norm_w": _finish(kn, w.dtype),
            "w_o": _finish(w_o, w.dtype)}


def host_upstream_grad(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Upstream gradient of the layer output, dout [B, L, hidden] ~ N(0, 1),
    from its own stream (seed + 2000), rounded to the workload's dtype."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 2000)
    g = rng.standard_normal((w.batch, w.seq, w.hidden), dtype=np.float32)
    return _finish(g, w.dtype)


def device_upstream_grad(w: Workload, device="cuda", seed: Optional[int] = None):
    """Same distribution as ``host_upstream_grad``, drawn on the device."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((w.seed if seed is None else seed) + 2000)
    t = torch.randn((w.batch, w.seq, w.hidden), generator=g, device=device,
                    dtype=torch.float32)
    return t.to(torch_dtype(w))


def host_cache(w: Workload, seed: Optional[int] = None,
               fill_unused: float = float("nan")) -> dict:
    """K/V caches [B, Hkv, capacity, d]: rows below ``cache_len`` ~ N(0, 1),
    rows at and above it set to ``fill_unused`` (NaN by default, so that a
    read past the valid rows shows up).  Drawn after the layer inputs from
    its own stream (seed + 1000)."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 1000)
    shape = (w.batch, w.hkv, w.kv_capacity, w.d)
    k = np.full(shape, fill_unused, dtype=np.float32)
    v = np.full(shape, fill_unused, dtype=np.float32)
    n = w.cache_len
    if n:
        k[:, :, :n] = _finish(rng.standard_normal(
            (w.batch, w.hkv, n, w.d), dtype=np.float32), w.dtype)
        v[:, :, :n] = _finish(rng.standard_normal(
            (w.batch, w.hkv, n, w.d), dtype=np.float32), w.dtype)
    return {"k_cache": k, "v_cache": v}


def host_ramp_attention(w: Workload, seed: Optional[int] = None,
                        log2_per_key: float = 0.3, spike_log2: float = 40.0,
                        spike_key: Optional[int] = None) -> dict:
    """Attention inputs q [B, Hq, L, d], k, v [B, Hkv, L, d] whose scores
    grow along the keys: per KV head a unit direction u; q rows are u (the
    group's direction) plus N(0, 0.1^2) noise, key j is u times a ramp that
    raises q.k by ``log2_per_key`` / (log2(e) / sqrt(d)) per key (that many
    log2 units of the softmax) plus the same noise, and in the last sequence
    key ``spike_key`` (default 2 L / 3) is raised by ``spike_log2`` more.  v
    ~ N(0, 1).  Rounded once to the workload's dtype."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 2000)
    B, L, d, hq, hkv = w.batch, w.seq, w.d, w.hq, w.hkv
    per_unit = np.sqrt(d) / np.log2(np.e)  # raw q.k per log2 unit of the softmax
    u = rng.standard_normal((hkv, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    ramp = log2_per_key * per_unit * np.arange(L)
    k = u[None, :, None, :] * ramp[None, None, :, None] + 0.1 * rng.standard_normal((B, hkv, L, d))
    sk = 2 * L // 3 if spike_key is None else spike_key
    k[B - 1, :, sk] += spike_log2 * per_unit * u
    q = np.repeat(u, hq // hkv, axis=0)[None, :, None, :] + 0.1 * rng.standard_normal((B, hq, L, d))
    v = rng.standard_normal((B, hkv, L, d))
    return {n: _finish(a.astype(np.float32), w.dtype) for n, a in (("q", q), ("k", k), ("v", v))}


def torch_dtype(w: Workload):
    import torch
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def to_device(arrays: dict, w: Workload, device="cuda") -> dict:
    """Copy host arrays to the device in the workload's dtype (exact: the
    values are already representable)."""
    import torch
    dt = torch_dtype(w)
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(device=device,
                                                          dtype=dt)
            for k, v in arrays.items()}


def device_layer_inputs(w: Workload, device="cuda", seed: Optional[int] = None):
    """Same distributions as ``host_layer_inputs``, drawn on the device with
    a seeded torch generator (for inputs too large to draw on the host)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(w.seed if seed is None else seed)
    dt = torch_dtype(w)
    d = w.d
    n_qkv = (w.hq + 2 * w.hkv) * d

    def normal(shape, std=1.0, mean=0.0):
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return (t * std + mean).to(dt)

    return {"x": normal((w.batch, w.seq, w.hidden)),
            "w_qkv": normal((n_qkv, w.hidden), 0.02),
            "q_norm_w": normal((d,), 0.1, 1.0),
            "k_norm_w": normal((d,), 0.1, 1.0),
            "w_o": normal((w.hidden, w.hq * d), 0.02)}


def device_cache(w: Workload, device="cuda", seed: Optional[int] = None):
    """K/V caches [B, Hkv, capacity, d] drawn on the device: rows below
    ``cache_len`` ~ N(0, 1), the rest zero.  With ``kv_fp8`` the caches are
    uint8 E4M3 codes of those values (torch's float8_e4m3fn conversion)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((w.seed if seed is None else seed) + 1000)
    dt = torch.float8_e4m3fn if w.kv_fp8 else torch_dtype(w)
    shape = (w.batch, w.hkv, w.kv_capacity, w.d)
    out = {}
    for name in ("k_cache", "v_cache"):
        t = torch.zeros(shape, device=device, dtype=torch.uint8 if w.kv_fp8 else dt)
        if w.cache_len:
            # fill one sequence at a time to bound the float32 staging buffer
            for b in range(w.batch):
                vals = torch.randn((w.hkv, w.cache_len, w.d), generator=g, device=device,
                                   dtype=torch.float32).to(dt)
                t[b, :, :w.cache_len] = vals.view(torch.uint8) if w.kv_fp8 else vals
        out[name] = t
    return out
