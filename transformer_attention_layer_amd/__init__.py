"""Python binding of the MI355X GQA layer library (``libgqa.so``).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the layer runs in the library's gfx950
kernels.  The library must be built (``python -m
transformer_attention_layer_amd.build``); importing the binding without it
raises at the first call, and there is no fallback path.

Entry points carry the names of the C ABI in ``include/gqa.h``:
``qkv_proj_normrope``, ``gqa_attn_core``, ``gqa_o_proj``,
``gqa_layer_forward`` (and ``gqa_layer_forward_noalloc``), the training pair ``gqa_layer_forward_train`` and
``gqa_layer_backward``, plus ``gqa_resolve`` and ``gqa_workspace_bytes``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# GQA_LIB may point at another build of the same library (A/B timing); the
# binding never falls back to anything else when the file is missing.
LIB_PATH = os.environ.get("GQA_LIB", os.path.join(_HERE, "libgqa.so"))

GQA_F32 = 0
GQA_BF16 = 1
WS_QKV, WS_ATTN, WS_LAYER, WS_OPROJ, WS_TRAIN_FORWARD, WS_BACKWARD = 0, 1, 2, 3, 4, 5

STATUS_NAMES = {
    0: "GQA_OK", 1: "GQA_ERR_INVALID_ARG", 2: "GQA_ERR_HEAD_DIM_INDIVISIBLE",
    3: "GQA_ERR_GROUP_INDIVISIBLE", 4: "GQA_ERR_ODD_HEAD_DIM",
    5: "GQA_ERR_UNSUPPORTED_HEAD_DIM", 6: "GQA_ERR_UNSUPPORTED_DTYPE",
    7: "GQA_ERR_UNSUPPORTED_SHAPE", 8: "GQA_ERR_WORKSPACE_TOO_SMALL",
    9: "GQA_ERR_CAPACITY", 10: "GQA_ERR_HIP",
}


class GQAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, f"status {status}")
        super().__init__(f"{self.name}: {detail}")


class _CConfig(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("qk_norm", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("out_f32", ctypes.c_int32),
                ("o_split", ctypes.c_int32), ("rotary_dim", ctypes.c_int32),
                ("kv_fp8", ctypes.c_int32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float), ("o_fp16", ctypes.c_int32)]


class _CSaved(ctypes.Structure):
    _fields_ = [("qkv", ctypes.c_void_p), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


class _CGrads(ctypes.Structure):
    _fields_ = [("dx", ctypes.c_void_p), ("dw_qkv", ctypes.c_void_p),
                ("dq_norm_w", ctypes.c_void_p), ("dk_norm_w", ctypes.c_void_p),
                ("dw_o", ctypes.c_void_p)]


@dataclass(frozen=True)
class GQAConfig:
    """Layer configuration; ``num_kv_heads=None`` means Hq, ``head_dim=None``
    means hidden_size // num_heads."""
    hidden_size: int
    num_heads: int
    num_kv_heads: Optional[int] = None
    head_dim: Optional[int] = None
    rope_theta: float = 1e6
    rms_eps: float = 1e-6
    qk_norm: bool = True
    causal: bool = True
    dtype: str = "bf16"
    out_f32: bool = False   # o_proj output in fp32 (the accumulator) instead of dtype
    o_split: bool = False   # layer forward: attention output as a bf16 hi + lo pair
    rotary_dim: Optional[int] = None  # partial rotary width; None = head_dim
    kv_fp8: bool = False    # K/V caches hold FP8 (E4M3) codes as torch.uint8
    k_scale: float = 1.0    # kv_fp8: an entry stands for value(code) * scale
    v_scale: float = 1.0
    o_fp16: bool = False    # layer forward: attention output as fp16, o_proj on fp16 MFMA

    def c(self) -> _CConfig:
        return _CConfig(self.hidden_size, self.num_heads, self.num_kv_heads or 0,
                        self.head_dim or 0, float(self.rope_theta), float(self.rms_eps),
                        int(bool(self.qk_norm)), int(bool(self.causal)),
                        GQA_BF16 if self.dtype == "bf16" else GQA_F32, int(bool(self.out_f32)),
                        int(bool(self.o_split)), int(self.rotary_dim or 0),
                        int(bool(self.kv_fp8)), float(self.k_scale), float(self.v_scale),
                        int(bool(self.o_fp16)))


_lib = None


def lib() -> ctypes.CDLL:
    """Load ``libgqa.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m transformer_attention_layer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        CP = ctypes.POINTER(_CConfig)
        L.gqa_resolve.argtypes = [CP, CP]
        L.gqa_workspace_bytes.argtypes = [CP, I32, I32, I32, I32]
        L.gqa_workspace_bytes.restype = SZ
        L.qkv_proj_normrope.argtypes = [CP, I32, I32, P, P, P, P, P, P, P, P, I32, P, SZ, P]
        L.gqa_attn_core.argtypes = [CP, I32, I32, P, P, P, P, I32, P, P, SZ, P]
        L.gqa_o_proj.argtypes = [CP, I32, P, P, P, P]
        L.gqa_layer_forward.argtypes = [CP, I32, I32, P, P, P, P, P, P, P, I32, P, P, P, SZ, P]
        L.gqa_layer_forward_noalloc.argtypes = [CP, I32, I32, P, P, P, P, P, P, P, I32, P, P, P]
        SP, GP = ctypes.POINTER(_CSaved), ctypes.POINTER(_CGrads)
        L.gqa_layer_forward_train.argtypes = [CP, I32, I32, P, P, P, P, P, SP, P, P, SZ, P]
        L.gqa_layer_backward.argtypes = [CP, I32, I32, P, P, P, P, P, SP, P, GP, P, SZ, P]
        for f in ("gqa_resolve", "qkv_proj_normrope", "gqa_attn_core", "gqa_o_proj",
                  "gqa_layer_forward", "gqa_layer_forward_noalloc", "gqa_layer_forward_train",
                  "gqa_layer_backward"):
            getattr(L, f).restype = ctypes.c_int
        L.gqa_status_string.argtypes = [ctypes.c_int]
        L.gqa_status_string.restype = ctypes.c_char_p
        L.gqa_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise GQAError(status, lib().gqa_last_error().decode())


def gqa_resolve(cfg: GQAConfig) -> dict:
    """Resolved (num_kv_heads, head_dim) after every configuration check."""
    out = _CConfig()
    cc = cfg.c()
    _check(lib().gqa_resolve(ctypes.byref(cc), ctypes.byref(out)))
    return {f: getattr(out, f) for f, _ in _CConfig._fields_}


def gqa_workspace_bytes(cfg: GQAConfig, batch: int, q_len: int, kv_capacity: int,
                        kind: int) -> int:
    cc = cfg.c()
    return int(lib().gqa_workspace_bytes(ctypes.byref(cc), batch, q_len, kv_capacity, kind))


# ---------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dt(cfg: GQAConfig):
    t = _torch()
    return t.bfloat16 if cfg.dtype == "bf16" else t.float32


def _cache_dt(cfg: GQAConfig):
    """Element type of the K/V caches: FP8 codes are stored as uint8."""
    t = _torch()
    return t.uint8 if cfg.kv_fp8 else _dt(cfg)


def _out_dt(cfg: GQAConfig):
    t = _torch()
    return t.float32 if cfg.out_f32 else _dt(cfg)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, name, dtype, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _i32(t, name, n):
    if t is None:
        return None
    torch = _torch()
    if not t.is_cuda or t.dtype != torch.int32 or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 device tensor of {n} entries")
    return t


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(n: int, device):
    torch = _torch()
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def _res(cfg: GQAConfig):
    r = gqa_resolve(cfg)
    return r["num_kv_heads"], r["head_dim"]


def qkv_proj_normrope(cfg: GQAConfig, x, w_qkv, q_norm_w=None, k_norm_w=None, *,
                      start_pos=None, k_cache=None, v_cache=None, q=None, stream=None):
    """x [B, L, hidden] -> q [B, Hq, L, d]; k, v written into the caches
    [B, Hkv, cap, d] at rows start_pos[b] + t (caches allocated with
    capacity L when not given).  Returns (q, k_cache, v_cache)."""
    torch = _torch()
    hkv, d = _res(cfg)
    B, L, H = x.shape
    dt = _dt(cfg)
    _need(x, "x", dt)
    _need(w_qkv, "w_qkv", dt, ((cfg.num_heads + 2 * hkv) * d, H))
    if cfg.qk_norm:
        _need(q_norm_w, "q_norm_w", dt, (d,))
        _need(k_norm_w, "k_norm_w", dt, (d,))
    cdt = _cache_dt(cfg)
    if k_cache is None:
        k_cache = torch.zeros((B, hkv, L, d), dtype=cdt, device=x.device)
        v_cache = torch.zeros((B, hkv, L, d), dtype=cdt, device=x.device)
    cap = k_cache.shape[2]
    _need(k_cache, "k_cache", cdt, (B, hkv, cap, d))
    _need(v_cache, "v_cache", cdt, (B, hkv, cap, d))
    if q is None:
        q = torch.empty((B, cfg.num_heads, L, d), dtype=dt, device=x.device)
    _need(q, "q", dt, (B, cfg.num_heads, L, d))
    sp = _i32(start_pos, "start_pos", B)
    ws = _workspace(gqa_workspace_bytes(cfg, B, L, cap, WS_QKV), x.device)
    cc = cfg.c()
    _check(lib().qkv_proj_normrope(
        ctypes.byref(cc), B, L, _ptr(x), _ptr(w_qkv),
        _ptr(q_norm_w) if cfg.qk_norm else None, _ptr(k_norm_w) if cfg.qk_norm else None,
        _ptr(sp), _ptr(q), _ptr(k_cache), _ptr(v_cache), cap, _ptr(ws), ws.numel(),
        _stream(stream)))
    return q, k_cache, v_cache


def gqa_attn_core(cfg: GQAConfig, q, k_cache, v_cache, *, kv_len=None, o=None, stream=None):
    """q [B, Hq, Lq, d], caches [B, Hkv, cap, d] -> o [B, Lq, Hq*d]."""
    torch = _torch()
    hkv, d = _res(cfg)
    dt = _dt(cfg)
    B, Hq, Lq, _ = q.shape
    _need(q, "q", dt, (B, cfg.num_heads, Lq, d))
    cap = k_cache.shape[2]
    _need(k_cache, "k_cache", _cache_dt(cfg), (B, hkv, cap, d))
    _need(v_cache, "v_cache", _cache_dt(cfg), (B, hkv, cap, d))
    if o is None:
        o = torch.empty((B, Lq, Hq * d), dtype=dt, device=q.device)
    _need(o, "o", dt, (B, Lq, Hq * d))
    kl = _i32(kv_len, "kv_len", B)
    ws = _workspace(gqa_workspace_bytes(cfg, B, Lq, cap, WS_ATTN), q.device)
    cc = cfg.c()
    _check(lib().gqa_attn_core(ctypes.byref(cc), B, Lq, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(kl), cap, _ptr(o), _ptr(ws), ws.numel(), _stream(stream)))
    return o


def gqa_o_proj(cfg: GQAConfig, o, w_o, *, out=None, stream=None):
    """o [..., Hq*d] -> out [..., hidden] = o W_o^T."""
    torch = _torch()
    hkv, d = _res(cfg)
    dt = _dt(cfg)
    _need(o, "o", dt)
    _need(w_o, "w_o", dt, (cfg.hidden_size, cfg.num_heads * d))
    if o.shape[-1] != cfg.num_heads * d:
        raise ValueError("o's last dimension must be Hq*d")
    tokens = o.numel() // (cfg.num_heads * d)
    if out is None:
        out = torch.empty(tuple(o.shape[:-1]) + (cfg.hidden_size,), dtype=_out_dt(cfg),
                          device=o.device)
    _need(out, "out", _out_dt(cfg))
    cc = cfg.c()
    _check(lib().gqa_o_proj(ctypes.byref(cc), tokens, _ptr(o), _ptr(w_o), _ptr(out),
                            _stream(stream)))
    return out


class LayerWorkspace:
    """A reusable workspace for ``gqa_layer_forward`` (so timed loops do not
    allocate)."""

    def __init__(self, cfg: GQAConfig, batch: int, q_len: int, kv_capacity: int, device="cuda"):
        self.nbytes = gqa_workspace_bytes(cfg, batch, q_len, kv_capacity, WS_LAYER)
        self.buf = _workspace(self.nbytes, device)


def gqa_layer_forward(cfg: GQAConfig, x, w_qkv, q_norm_w, k_norm_w, w_o, *, k_cache=None,
                      v_cache=None, cache_len=None, out=None, workspace: LayerWorkspace = None,
                      stream=None):
    """The layer: x [B, L, hidden] -> out [B, L, hidden].  With caches
    [B, Hkv, cap, d] and ``cache_len`` [B] int32, the new k, v are appended
    at rows cache_len[b].. and attention runs over the whole history.
    Without caches, fresh ones of capacity L are allocated (and returned).
    Returns (out, k_cache, v_cache)."""
    torch = _torch()
    hkv, d = _res(cfg)
    dt = _dt(cfg)
    B, L, H = x.shape
    _need(x, "x", dt, (B, L, cfg.hidden_size))
    _need(w_qkv, "w_qkv", dt, ((cfg.num_heads + 2 * hkv) * d, H))
    _need(w_o, "w_o", dt, (H, cfg.num_heads * d))
    if cfg.qk_norm:
        _need(q_norm_w, "q_norm_w", dt, (d,))
        _need(k_norm_w, "k_norm_w", dt, (d,))
    cdt = _cache_dt(cfg)
    if k_cache is None:
        k_cache = torch.empty((B, hkv, L, d), dtype=cdt, device=x.device)
        v_cache = torch.empty((B, hkv, L, d), dtype=cdt, device=x.device)
    cap = k_cache.shape[2]
    _need(k_cache, "k_cache", cdt, (B, hkv, cap, d))
    _need(v_cache, "v_cache", cdt, (B, hkv, cap, d))
    cl = _i32(cache_len, "cache_len", B)
    if out is None:
        out = torch.empty((B, L, H), dtype=_out_dt(cfg), device=x.device)
    _need(out, "out", _out_dt(cfg), (B, L, H))
    if workspace is None:
        workspace = LayerWorkspace(cfg, B, L, cap, x.device)
    cc = cfg.c()
    _check(lib().gqa_layer_forward(
        ctypes.byref(cc), B, L, _ptr(x), _ptr(w_qkv),
        _ptr(q_norm_w) if cfg.qk_norm else None, _ptr(k_norm_w) if cfg.qk_norm else None,
        _ptr(w_o), _ptr(k_cache), _ptr(v_cache), cap, _ptr(cl), _ptr(out),
        _ptr(workspace.buf), workspace.nbytes, _stream(stream)))
    return out, k_cache, v_cache


def gqa_layer_forward_noalloc(cfg: GQAConfig, x, w_qkv, q_norm_w, k_norm_w, w_o, *, k_cache,
                              v_cache, cache_len=None, out=None, stream=None):
    """``gqa_layer_forward`` without a workspace argument: the library's own
    static scratch memory (one per GPU, shared by every call on that GPU;
    calls that overlap on one GPU race) serves as the workspace, and the C
    call allocates nothing.  The caches are required; ``out`` is allocated
    here when not given.  Raises GQAError (GQA_ERR_WORKSPACE_TOO_SMALL) when
    the call needs more scratch than the library holds.  Returns
    (out, k_cache, v_cache)."""
    torch = _torch()
    hkv, d = _res(cfg)
    dt = _dt(cfg)
    B, L, H = x.shape
    _need(x, "x", dt, (B, L, cfg.hidden_size))
    _need(w_qkv, "w_qkv", dt, ((cfg.num_heads + 2 * hkv) * d, H))
    _need(w_o, "w_o", dt, (H, cfg.num_heads * d))
    if cfg.qk_norm:
        _need(q_norm_w, "q_norm_w", dt, (d,))
        _need(k_norm_w, "k_norm_w", dt, (d,))
    cdt = _cache_dt(cfg)
    if k_cache is None or v_cache is None:
        raise ValueError("k_cache and v_cache are required")
    cap = k_cache.shape[2]
    _need(k_cache, "k_cache", cdt, (B, hkv, cap, d))
    _need(v_cache, "v_cache", cdt, (B, hkv, cap, d))
    cl = _i32(cache_len, "cache_len", B)
    if out is None:
        out = torch.empty((B, L, H), dtype=_out_dt(cfg), device=x.device)
    _need(out, "out", _out_dt(cfg), (B, L, H))
    cc = cfg.c()
    _check(lib().gqa_layer_forward_noalloc(
        ctypes.byref(cc), B, L, _ptr(x), _ptr(w_qkv),
        _ptr(q_norm_w) if cfg.qk_norm else None, _ptr(k_norm_w) if cfg.qk_norm else None,
        _ptr(w_o), _ptr(k_cache), _ptr(v_cache), cap, _ptr(cl), _ptr(out), _stream(stream)))
    return out, k_cache, v_cache


class TrainSaved:
    """Device buffers the training forward writes and the backward reads
    (``gqa_saved`` of the C ABI): qkv [B, L, (Hq+2Hkv)d] fp32 before norm and
    RoPE, q [B, Hq, L, d], k and v [B, Hkv, L, d] after norm and RoPE, o
    [B, L, Hq*d] and lse [B, Hq, L] fp32."""

    def __init__(self, cfg: GQAConfig, batch: int, q_len: int, device="cuda"):
        torch = _torch()
        hkv, d = _res(cfg)
        dt = _dt(cfg)
        B, L, hq = batch, q_len, cfg.num_heads
        self.qkv = torch.empty((B, L, (hq + 2 * hkv) * d), dtype=torch.float32, device=device)
        self.q = torch.empty((B, hq, L, d), dtype=dt, device=device)
        self.k = torch.empty((B, hkv, L, d), dtype=dt, device=device)
        self.v = torch.empty((B, hkv, L, d), dtype=dt, device=device)
        self.o = torch.empty((B, L, hq * d), dtype=dt, device=device)
        self.lse = torch.empty((B, hq, L), dtype=torch.float32, device=device)

    def c(self) -> _CSaved:
        return _CSaved(self.qkv.data_ptr(), self.q.data_ptr(), self.k.data_ptr(),
                       self.v.data_ptr(), self.o.data_ptr(), self.lse.data_ptr())


def gqa_layer_forward_train(cfg: GQAConfig, x, w_qkv, q_norm_w, k_norm_w, w_o, *,
                            saved: TrainSaved = None, out=None, workspace=None, stream=None):
    """The layer forward without a cache that keeps what the backward needs.
    ``workspace``: a uint8 device tensor of gqa_workspace_bytes(...,
    WS_TRAIN_FORWARD) bytes (allocated when omitted).  Returns
    (out [B, L, hidden], saved)."""
    torch = _torch()
    hkv, d = _res(cfg)
    dt = _dt(cfg)
    B, L, H = x.shape
    _need(x, "x", dt, (B, L, cfg.hidden_size))
    _need(w_qkv, "w_qkv", dt, ((cfg.num_heads + 2 * hkv) * d, H))
    _need(w_o, "w_o", dt, (H, cfg.num_heads * d))
    if cfg.qk_norm:
        _need(q_norm_w, "q_norm_w", dt, (d,))
        _need(k_norm_w, "k_norm_w", dt, (d,))
    if saved is None:
        saved = TrainSaved(cfg, B, L, x.device)
    if out is None:
        out = torch.empty((B, L, H), dtype=_out_dt(cfg), device=x.device)
    _need(out, "out", _out_dt(cfg), (B, L, H))
    if workspace is None:
        workspace = _workspace(gqa_workspace_bytes(cfg, B, L, L, WS_TRAIN_FORWARD), x.device)
    cc, cs = cfg.c(), saved.c()
    _check(lib().gqa_layer_forward_train(
        ctypes.byref(cc), B, L, _ptr(x), _ptr(w_qkv),
        _ptr(q_norm_w) if cfg.qk_norm else None, _ptr(k_norm_w) if cfg.qk_norm else None,
        _ptr(w_o), ctypes.byref(cs), _ptr(out), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return out, saved


class BackwardWorkspace:
    """A reusable workspace for ``gqa_layer_backward``."""

    def __init__(self, cfg: GQAConfig, batch: int, q_len: int, device="cuda"):
        self.nbytes = gqa_workspace_bytes(cfg, batch, q_len, q_len, WS_BACKWARD)
        self.buf = _workspace(self.nbytes, device)


def gqa_layer_backward(cfg: GQAConfig, x, w_qkv, q_norm_w, k_norm_w, w_o, saved: TrainSaved,
                       dout, *, grads: dict = None, workspace: BackwardWorkspace = None,
                       stream=None):
    """Gradients of the layer for the upstream gradient dout [B, L, hidden]
    (cfg dtype).  Returns a dict: dx [B, L, hidden] (cfg dtype), dw_qkv,
    dq_norm_w, dk_norm_w (None without QK-norm) and dw_o, all fp32."""
    torch = _torch()
    hkv, d = _res(cfg)
    dt = _dt(cfg)
    B, L, H = x.shape
    _need(x, "x", dt, (B, L, cfg.hidden_size))
    _need(dout, "dout", dt, (B, L, H))
    nq = (cfg.num_heads + 2 * hkv) * d
    _need(w_qkv, "w_qkv", dt, (nq, H))
    _need(w_o, "w_o", dt, (H, cfg.num_heads * d))
    if cfg.qk_norm:
        _need(q_norm_w, "q_norm_w", dt, (d,))
        _need(k_norm_w, "k_norm_w", dt, (d,))
    if grads is None:
        f32 = torch.float32
        grads = {"dx": torch.empty((B, L, H), dtype=dt, device=x.device),
                 "dw_qkv": torch.empty((nq, H), dtype=f32, device=x.device),
                 "dq_norm_w": torch.empty((d,), dtype=f32, device=x.device) if cfg.qk_norm else None,
                 "dk_norm_w": torch.empty((d,), dtype=f32, device=x.device) if cfg.qk_norm else None,
                 "dw_o": torch.empty((H, cfg.num_heads * d), dtype=f32, device=x.device)}
    _need(grads["dx"], "dx", dt, (B, L, H))
    _need(grads["dw_qkv"], "dw_qkv", torch.float32, (nq, H))
    _need(grads["dw_o"], "dw_o", torch.float32, (H, cfg.num_heads * d))
    if cfg.qk_norm:
        _need(grads["dq_norm_w"], "dq_norm_w", torch.float32, (d,))
        _need(grads["dk_norm_w"], "dk_norm_w", torch.float32, (d,))
    if workspace is None:
        workspace = BackwardWorkspace(cfg, B, L, x.device)
    cg = _CGrads(_ptr(grads["dx"]), _ptr(grads["dw_qkv"]),
                 _ptr(grads["dq_norm_w"]) if cfg.qk_norm else None,
                 _ptr(grads["dk_norm_w"]) if cfg.qk_norm else None, _ptr(grads["dw_o"]))
    cc, cs = cfg.c(), saved.c()
    _check(lib().gqa_layer_backward(
        ctypes.byref(cc), B, L, _ptr(x), _ptr(w_qkv),
        _ptr(q_norm_w) if cfg.qk_norm else None, _ptr(k_norm_w) if cfg.qk_norm else None,
        _ptr(w_o), ctypes.byref(cs), _ptr(dout), ctypes.byref(cg), _ptr(workspace.buf),
        workspace.nbytes, _stream(stream)))
    return grads


__all__ = [
    "GQAConfig", "GQAError", "LIB_PATH", "lib", "gqa_resolve", "gqa_workspace_bytes",
    "qkv_proj_normrope", "gqa_attn_core", "gqa_o_proj", "gqa_layer_forward",
    "gqa_layer_forward_noalloc",
    "LayerWorkspace", "GQA_F32", "GQA_BF16", "TrainSaved", "gqa_layer_forward_train",
    "BackwardWorkspace", "gqa_layer_backward",
]
