"""Plain CPU oracle for the forward pass of a grouped-query attention layer
with an explicitly set head_dim.

TEST INFRASTRUCTURE. Only the tests, the smoke check of ``__graft_entry__``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.
The product path (the HIP library and its Python binding) never does, and it
shares no code, table or constant with this file.

What it computes, step by step, follows the sources below; each function
names the passage it implements.

* "Tutorial 07: Multi-Head and Grouped-Query Attention (Full Layer)",
  sections 3 and 4 for what the layer computes: q, k, v projections, a
  per-head RMSNorm of q and k (dim = head_dim), RoPE on q and k, attention
  in float, and the output projection.
* "Attention head partitions: keep each head's dependencies intact" for the
  grouping: attention is computed per KV head, with the query heads it
  serves stacked against its keys and values.
* GPT-NeoX issue "Support explicit attention head_dim independent of
  hidden_size / num_attention_heads", sections "Proposed configuration
  behavior", "Proposed implementation", "Fused QKV projection", "Attention
  output flattening", "Output projection" and "Scaling and RoPE" for the
  shapes, the quotient fallback, the divisibility rules and the scale.
* "num_heads Is Not a Capacity Knob", section "Why the cost does not move",
  for the weight and multiply-accumulate counts, and for the output
  projection as a sum of each head's output through its own slice of W_O.

Readings where the pages are silent (each also listed in the design doc):

1. RMSNorm is the textbook ``v / sqrt(mean(v*v) + eps) * w`` over the d
   entries of one head; one [d] weight for q and one for k, shared by all
   heads.  The pages name RMSNorm(head_dim, weight, eps) but print no formula.
2. k_norm is applied to k's own projection (the tutorial's code in section 4;
   its prose in section 3 has k_norm(projection_q), read as a typo).
3. RoPE is full-width rotate-half: entry i pairs with entry i + d/2 and turns
   by angle ``p * theta**(-2i/d)``.  The pages name RoPE(head_dim,
   max_position_embeddings, rope_theta) but print no pairing rule.  Angles
   are formed in float64.
4. The fused QKV weight is the row concatenation [q_proj; k_proj; v_proj].
5. Query head h reads KV head h // (Hq / Hkv) (contiguous groups).
6. No bias in any projection (``linear(x, W)`` = ``x @ W.T``).
7. With a cache, query i of a chunk of L sits at position cache_len + i and
   sees keys at positions <= its own (bottom-right causal alignment); new
   k and v are appended before attending.
8. The layer returns the o_proj output; the residual add is the caller's.
9. Partial rotary (the NeoX issue keeps its rotary_pct option for RoPE at
   the effective head_dim but does not define it): with rotary_dim r < d, only the first r entries of
   each head rotate, as a rotate-half RoPE of width r (entry i < r/2 pairs
   with i + r/2 and turns by ``p * theta**(-2i/r)``); entries r .. d-1 pass
   through.  r = d is reading 3.

10. FP8 K/V cache ("Head Dimension" article, section 5.2: K and V are cached
   in FP8 precision; nothing more is said): cache entries are OCP E4M3
   codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest
   finite value 448, no infinities, 0x7F/0xFF are NaN).  An entry holds
   ``value(code) * scale`` with one scale per tensor (K, V).  Appending x
   stores the code nearest to x / scale, ties to an even mantissa, with
   magnitudes above 448 saturated to 448.  Attention runs on the stored
   values.
11. Backward pass (GPT-NeoX issue, "Tests and acceptance criteria": forward
   and backward passes; "Attention head partitions ...": gradients of the
   shared KV parameters): the pages name the gradients but print no formula.
   They are read as the exact derivatives of this forward without a cache
   (positions 0..L-1), taken by the chain rule through the steps in reverse;
   a KV head's gradient sums over the query heads it serves, and the shared
   QK-norm weights sum over every token and head.

parity unpinned: reading 1 (the exact RMSNorm formula: eps placement),
reading 3 (the RoPE pairing convention) and reading 9 (which entries a
partial rotary turns) are not fixed by the pages.  The
tests pin them to library routines and mathematical invariants (norm
preservation, relative-position property, identity at p = 0), not to page
values.

Arithmetic runs in float64 by default; ``dtype=np.float32`` runs the same
code in float32, the precision the tutorial's step 6 names for the attention
core.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


# ---------------------------------------------------------------------------
# Configuration
# ---------------------------------------------------------------------------

class ConfigError(ValueError):
    """A configuration the pages say must be rejected."""


@dataclass(frozen=True)
class Resolved:
    hidden: int        # residual width
    hq: int            # query heads
    hkv: int           # key/value heads
    d: int             # effective head_dim
    group: int         # query heads per KV head
    q_width: int       # hq * d
    kv_width: int      # hkv * d
    n_qkv: int         # q_width + 2 * kv_width
    scale: float       # d ** -0.5


def resolve_config(hidden_size: int, num_heads: int,
                   num_kv_heads: Optional[int] = None,
                   head_dim: Optional[int] = None,
                   require_even: bool = True) -> Resolved:
    """Effective head_dim and widths.

    GPT-NeoX issue "Support explicit attention head_dim ...":
    - "Proposed configuration behavior": d = head_dim if set, else
      hidden_size // num_attention_heads; hidden_size % num_attention_heads
      is required only when d must be derived.
    - "Proposed implementation": query width Hq*d, kv width Hkv*d with
      Hkv defaulting to Hq.
    - "Scaling and RoPE": scale d**-0.5; RoPE needs an even d.
    "Attention head partitions: keep each head's dependencies intact": GQA
    groups Hq/Hkv query heads per KV head when that ratio is integral.
    """
    if hidden_size <= 0 or num_heads <= 0:
        raise ConfigError("hidden_size and num_heads must be positive")
    if head_dim is None:
        if hidden_size % num_heads != 0:
            raise ConfigError(
                f"head_dim unset and hidden_size {hidden_size} is not "
                f"divisible by num_heads {num_heads}")
        d = hidden_size // num_heads
    else:
        d = int(head_dim)
        if d <= 0:
            raise ConfigError("head_dim must be positive")
    hkv = num_heads if num_kv_heads is None else int(num_kv_heads)
    if hkv <= 0:
        raise ConfigError("num_kv_heads must be positive")
    if num_heads % hkv != 0:
        raise ConfigError(
            f"num_heads {num_heads} is not a multiple of num_kv_heads {hkv}")
    if require_even and d % 2 != 0:
        raise ConfigError(f"head_dim {d} is odd; RoPE needs an even head_dim")
    return Resolved(hidden=hidden_size, hq=num_heads, hkv=hkv, d=d,
                    group=num_heads // hkv, q_width=num_heads * d,
                    kv_width=hkv * d, n_qkv=(num_heads + 2 * hkv) * d,
                    scale=float(d) ** -0.5)


def weight_shapes(res: Resolved) -> dict:
    """Projection weight shapes, [out, in] as in the GPT-NeoX issue's
    "Checkpoint conversion" section and the tutorial's section 2."""
    return {
        "q_proj": (res.q_width, res.hidden),
        "k_proj": (res.kv_width, res.hidden),
        "v_proj": (res.kv_width, res.hidden),
        "o_proj": (res.hidden, res.q_width),
        "query_key_value": (res.n_qkv, res.hidden),
    }


def attention_param_count(res: Resolved) -> int:
    """Weights of the four projections ("num_heads Is Not a Capacity Knob",
    "Why the cost does not move": four matrices, no biases)."""
    s = weight_shapes(res)
    return sum(a * b for k, (a, b) in s.items() if k != "query_key_value")


def macs_per_token(res: Resolved, n_context: int) -> dict:
    """Multiply-accumulates per token ("Why the cost does not move"): the
    projections cost one MAC per weight, the scores cost d per visible key
    per query head, and the value average d per key per head."""
    proj = attention_param_count(res)
    score = n_context * res.d * res.hq
    value = n_context * res.d * res.hq
    return {"projection": proj, "score_value": score + value}


# ---------------------------------------------------------------------------
# Steps of the layer
# ---------------------------------------------------------------------------

def project(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """linear(x, W) = x @ W.T (tutorial section 4, step 1; no bias)."""
    return np.matmul(x, w.T)


def split_heads(y: np.ndarray, res: Resolved):
    """Split the fused projection on whole-head boundaries, Q | K | V, and
    reshape each to [B, L, heads, d] (GPT-NeoX issue, "Fused QKV
    projection"; tutorial section 4, step 1)."""
    b, l, _ = y.shape
    q = y[..., :res.q_width].reshape(b, l, res.hq, res.d)
    k = y[..., res.q_width:res.q_width + res.kv_width].reshape(
        b, l, res.hkv, res.d)
    v = y[..., res.q_width + res.kv_width:].reshape(b, l, res.hkv, res.d)
    return q, k, v


def weight_blocks(w_qkv: np.ndarray, res: Resolved):
    """The fused weight's row blocks W_q [Hq*d, H], W_k [Hkv*d, H] and W_v
    [Hkv*d, H] (GPT-NeoX issue, "Fused QKV projection": its output width is
    the query width plus twice the KV width; reading 4: rows Q | K | V)."""
    qw, kw = res.q_width, res.kv_width
    return w_qkv[:qw], w_qkv[qw:qw + kw], w_qkv[qw + kw:qw + 2 * kw]


def rms_norm_heads(v: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Per-head RMSNorm over the last axis (tutorial section 3: the norm has
    dim = head_dim and works within each head)."""
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * w


def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    """theta ** (-2i/d) for i < d/2, in float64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / d)


def apply_rope(v: np.ndarray, positions: np.ndarray, theta: float,
               rotary_dim: Optional[int] = None) -> np.ndarray:
    """Rotate-half RoPE of v [B, L, heads, d] at integer positions [B, L]
    (tutorial section 4, step 3; GPT-NeoX issue "Scaling and RoPE": built at
    the effective head_dim, with the rotary_pct option kept).  ``rotary_dim`` r (None =
    d) rotates the first r entries as a width-r RoPE and passes the rest
    (reading 9)."""
    d = v.shape[-1]
    r = d if rotary_dim is None else int(rotary_dim)
    half = r // 2
    ang = positions.astype(np.float64)[..., None] * rope_inv_freq(r, theta)
    cos = np.cos(ang).astype(v.dtype)[:, :, None, :]
    sin = np.sin(ang).astype(v.dtype)[:, :, None, :]
    x1 = v[..., :half]
    x2 = v[..., half:r]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin, v[..., r:]], axis=-1)


def grouped_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                      q_pos: np.ndarray, kv_len: np.ndarray, scale: float,
                      causal: bool = True) -> np.ndarray:
    """softmax(q k^T * scale) v with each KV head serving Hq/Hkv query heads
    (tutorial section 4, step 6; "Attention head partitions ...": a KV head
    and the group of query heads it serves form one unit).

    Computed per KV group: the group's G query heads are stacked into one
    [G*Lq, d] block of query rows, scored against that KV head's keys, and
    each row's softmax weights average its values.

    q [B, Hq, Lq, d]; k, v [B, Hkv, S, d] with S >= kv_len[b]; q_pos [B, Lq]
    holds each query's position.  Query i of batch b sees keys j < kv_len[b],
    and with ``causal`` only those with j <= q_pos[b, i].
    Returns [B, Hq, Lq, d].
    """
    bsz, hq, lq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    out = np.zeros((bsz, hq, lq, v.shape[-1]), dtype=q.dtype)
    for b in range(bsz):
        n = int(kv_len[b])
        visible = np.ones((lq, n), dtype=bool)
        if causal:
            visible = np.arange(n)[None, :] <= q_pos[b][:, None]
        rows_visible = np.tile(visible, (group, 1))           # [G*Lq, n]
        for g in range(hkv):
            heads = slice(g * group, (g + 1) * group)          # the query heads of KV head g
            qg = q[b, heads].reshape(group * lq, d)
            s = np.matmul(qg, k[b, g, :n].T) * q.dtype.type(scale)
            s = np.where(rows_visible, s, -np.inf)
            p = np.exp(s - np.max(s, axis=-1, keepdims=True))
            p = p / np.sum(p, axis=-1, keepdims=True)
            out[b, heads] = np.matmul(p, v[b, g, :n]).reshape(group, lq, -1)
    return out


def merge_heads(o: np.ndarray) -> np.ndarray:
    """[B, Hq, L, d] -> [B, L, Hq*d] (GPT-NeoX issue, "Attention output
    flattening": flatten to the query width, not the residual width)."""
    b, h, l, d = o.shape
    return o.transpose(0, 2, 1, 3).reshape(b, l, h * d)


def project_heads_out(o: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """o_proj of per-head outputs o [B, Hq, L, d]: the sum over heads of each
    head's output times its own d columns of W_o [hidden, Hq*d] ("num_heads
    Is Not a Capacity Knob", "Why the cost does not move": the heads'
    outputs, concatenated, meet W_O, i.e. each head contributes through its
    slice; GPT-NeoX issue, "Output projection": W_o maps the query width
    back to hidden).  Returns [B, L, hidden]."""
    d = o.shape[-1]
    out = np.zeros(o.shape[:1] + o.shape[2:3] + (w_o.shape[0],), dtype=o.dtype)
    for h in range(o.shape[1]):
        out += project(o[:, h], w_o[:, h * d:(h + 1) * d])
    return out


# ---------------------------------------------------------------------------
# FP8 (E4M3) cache entries (reading 10)
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_value(codes) -> np.ndarray:
    """Value of OCP E4M3 codes (reading 10), from the bit fields: sign s,
    exponent e (4 bits, bias 7), mantissa m (3 bits).  e > 0: (1 + m/8) *
    2^(e-7); e = 0: m/8 * 2^-6 (subnormal); e = 15 with m = 7: NaN."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e > 0, (1.0 + m / 8.0) * np.exp2(e - 7.0), m / 8.0 * 2.0 ** -6)
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return sign * mag


def quantize_e4m3(x) -> np.ndarray:
    """Code of the E4M3 value nearest to x, ties to an even mantissa,
    magnitudes above 448 saturated (reading 10).  Within a binade the
    representable magnitudes are multiples of the quantum 2^(e-10) (e the
    biased exponent, at least 1; the subnormals share the quantum 2^-9 of the
    lowest binade), so rounding |x| to the nearest multiple of the quantum,
    half to even, picks the nearest value; a result that reaches the next
    power of two is that power's code.  Returns uint8 codes; x must be
    finite."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_e4m3 needs finite inputs")
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # biased exponent of |x| (1 for the subnormal range and zero)
    with np.errstate(divide="ignore"):
        e = np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0))) + 7.0, 1.0)
    e = np.clip(e, 1.0, 15.0)
    q = np.exp2(e - 10.0)                       # quantum of the binade
    n = np.rint(a / q)                          # half to even
    # n counts quanta: 8..15 within a normal binade; 16 is the next binade's
    # first value; below 8 (only in the lowest binade) a subnormal
    n = n.astype(np.int64)
    e = e.astype(np.int64)
    up = n >= 16
    e = np.where(up, e + 1, e)
    n = np.where(up, n // 2, n)
    normal = n >= 8
    code = np.where(normal, (e << 3) | (n - 8), n)  # subnormal: e field 0, m = n
    code = np.where(sign, code | 0x80, code)
    return code.astype(np.uint8)


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------

def qkv_normrope(res: Resolved, x, w_qkv, q_norm_w, k_norm_w, positions,
                 rope_theta, rms_eps, qk_norm=True, rope=True, rotary_dim=None):
    """q, k, v of the layer (tutorial section 4, steps 1-4): each is x times
    its own row block of the fused weight, split into heads; q and k are
    normalised per head (QK-norm) and rotated at their positions (RoPE).
    Returns q [B, Hq, L, d] and k, v [B, Hkv, L, d] (k after norm and RoPE,
    v raw)."""
    b, l, _ = x.shape
    wq, wk, wv = weight_blocks(w_qkv, res)
    q = project(x, wq).reshape(b, l, res.hq, res.d)
    k = project(x, wk).reshape(b, l, res.hkv, res.d)
    v = project(x, wv).reshape(b, l, res.hkv, res.d)
    if qk_norm:
        q = rms_norm_heads(q, q_norm_w, rms_eps)
        k = rms_norm_heads(k, k_norm_w, rms_eps)
    if rope:
        kw = {} if rotary_dim is None else {"rotary_dim": rotary_dim}
        q = apply_rope(q, positions, rope_theta, **kw)
        k = apply_rope(k, positions, rope_theta, **kw)
    return (q.transpose(0, 2, 1, 3), k.transpose(0, 2, 1, 3),
            v.transpose(0, 2, 1, 3))


def layer_forward(res: Resolved, x, w_qkv, q_norm_w, k_norm_w, w_o, *,
                  rope_theta: float, rms_eps: float, qk_norm: bool = True,
                  causal: bool = True, rope: bool = True,
                  k_cache=None, v_cache=None, cache_len=None,
                  rotary_dim: Optional[int] = None, kv_fp8: bool = False,
                  k_scale: float = 1.0, v_scale: float = 1.0,
                  dtype=np.float64):
    """The layer forward (tutorial section 4, steps 1 to 7): q, k, v, the
    cache update, grouped attention, and the output projection summed over
    heads.

    x [B, L, hidden]; w_qkv [(Hq+2Hkv)d, hidden]; w_o [hidden, Hq*d].
    Without a cache, positions are 0..L-1.  With ``k_cache``/``v_cache``
    [B, Hkv, S, d] and ``cache_len`` [B], token i of sequence b sits at
    position cache_len[b] + i, its k and v are written at that row of a copy
    of the cache (step 5, update_and_fetch), and attention runs over rows
    0 .. cache_len[b] + L - 1.

    Returns (out [B, L, hidden], k_cache', v_cache') where the caches are the
    updated copies (None without a cache).  ``rope=False`` drops step 3 and
    exists only to reduce the layer to textbook multi-head attention in the
    tests; ``rotary_dim`` is reading 9.

    ``kv_fp8`` (reading 10): the caches hold E4M3 codes (uint8) standing for
    code value * k_scale (resp. v_scale); the new rows are appended as the
    codes of k / k_scale and v / v_scale, and attention runs on the stored
    values.  The returned caches are then the updated code arrays.
    """
    x = np.asarray(x, dtype=dtype)
    w_qkv = np.asarray(w_qkv, dtype=dtype)
    w_o = np.asarray(w_o, dtype=dtype)
    qn = None if q_norm_w is None else np.asarray(q_norm_w, dtype=dtype)
    kn = None if k_norm_w is None else np.asarray(k_norm_w, dtype=dtype)
    bsz, seq, _ = x.shape
    if cache_len is None:
        start = np.zeros(bsz, dtype=np.int64)
    else:
        start = np.asarray(cache_len, dtype=np.int64)
    positions = start[:, None] + np.arange(seq, dtype=np.int64)[None, :]
    kw = {} if rotary_dim is None else {"rotary_dim": rotary_dim}
    q, k, v = qkv_normrope(res, x, w_qkv, qn, kn, positions, rope_theta,
                           rms_eps, qk_norm=qk_norm, rope=rope, **kw)
    if k_cache is None:
        kk, vv = k, v
        kv_len = np.full(bsz, seq, dtype=np.int64)
        k_out = v_out = None
    elif kv_fp8:
        kc = np.array(k_cache, dtype=np.uint8, copy=True)
        vc = np.array(v_cache, dtype=np.uint8, copy=True)
        for b in range(bsz):
            s0 = int(start[b])
            kc[b, :, s0:s0 + seq] = quantize_e4m3(np.asarray(k[b], np.float64) / k_scale)
            vc[b, :, s0:s0 + seq] = quantize_e4m3(np.asarray(v[b], np.float64) / v_scale)
        kv_len = start + seq
        # rows at or past kv_len are never read; their codes may be anything
        kk = np.zeros(kc.shape, dtype=dtype)
        vv = np.zeros(vc.shape, dtype=dtype)
        for b in range(bsz):
            n = int(kv_len[b])
            kk[b, :, :n] = e4m3_value(kc[b, :, :n]) * k_scale
            vv[b, :, :n] = e4m3_value(vc[b, :, :n]) * v_scale
        k_out, v_out = kc, vc
    else:
        kk = np.array(k_cache, dtype=dtype, copy=True)
        vv = np.array(v_cache, dtype=dtype, copy=True)
        for b in range(bsz):
            s0 = int(start[b])
            kk[b, :, s0:s0 + seq] = k[b]
            vv[b, :, s0:s0 + seq] = v[b]
        kv_len = start + seq
        k_out, v_out = kk, vv
    o = grouped_attention(q, kk, vv, positions, kv_len, res.scale, causal)
    out = project_heads_out(o, w_o)
    return out, k_out, v_out


def layer_forward_rows(res: Resolved, x, w_qkv, q_norm_w, k_norm_w, w_o, rows,
                       *, rope_theta: float, rms_eps: float,
                       qk_norm: bool = True, rotary_dim: Optional[int] = None,
                       dtype=np.float64):
    """Exact causal prefill output (no cache, positions 0..L-1) for chosen
    (b, t) rows only.

    Row t of the output depends only on x[b, t] (through q) and x[b, :t+1]
    (through k and v), because the causal mask hides later keys.  So the
    same steps as ``layer_forward``, run on the prefix x[b, :t+1] and read
    at its last position, give row t exactly.  Returns an array [len(rows),
    hidden].
    """
    rows = list(rows)
    out = np.zeros((len(rows), res.hidden), dtype=dtype)
    by_b: dict = {}
    for i, (b, t) in enumerate(rows):
        by_b.setdefault(int(b), []).append((i, int(t)))
    for b, items in by_b.items():
        tmax = max(t for _, t in items)
        xb = np.asarray(x[b:b + 1, :tmax + 1], dtype=dtype)
        wq, wk, wv = weight_blocks(np.asarray(w_qkv, dtype=dtype), res)
        k = project(xb, wk).reshape(1, tmax + 1, res.hkv, res.d)
        v = project(xb, wv).reshape(1, tmax + 1, res.hkv, res.d)
        pos_all = np.arange(tmax + 1, dtype=np.int64)[None, :]
        if qk_norm:
            k = rms_norm_heads(k, np.asarray(k_norm_w, dtype=dtype), rms_eps)
        kw = {} if rotary_dim is None else {"rotary_dim": rotary_dim}
        k = apply_rope(k, pos_all, rope_theta, **kw)
        k = k.transpose(0, 2, 1, 3)
        v = v.transpose(0, 2, 1, 3)
        ts = np.array([t for _, t in items], dtype=np.int64)
        xq = np.asarray(x[b:b + 1, ts], dtype=dtype)
        q = project(xq, wq).reshape(1, len(ts), res.hq, res.d)
        if qk_norm:
            q = rms_norm_heads(q, np.asarray(q_norm_w, dtype=dtype), rms_eps)
        q = apply_rope(q, ts[None, :], rope_theta, **kw).transpose(0, 2, 1, 3)
        o = grouped_attention(q, k, v, ts[None, :],
                              np.array([tmax + 1]), res.scale, True)
        o_rows = project_heads_out(o, np.asarray(w_o, dtype=dtype))[0]
        for j, (i, _) in enumerate(items):
            out[i] = o_rows[j]
    return out


# ---------------------------------------------------------------------------
# Backward pass (reading 11): gradients of the layer without a cache
# ---------------------------------------------------------------------------

def project_backward(x, w, dy):
    """Gradients of y = x @ W.T (tutorial section 4, steps 1 and 7) for the
    upstream gradient dy: dx = dy @ W and dW = dy^T x, summed over every
    token.  Returns (dx, dW)."""
    dx = np.matmul(dy, w)
    dw = np.matmul(dy.reshape(-1, dy.shape[-1]).T, x.reshape(-1, x.shape[-1]))
    return dx, dw


def rms_norm_heads_backward(v, w, eps, dy):
    """Gradients of ``rms_norm_heads(v, w, eps)`` (reading 1) for dy.

    With r = (mean(v*v) + eps)^(-1/2) per head row, out_j = v_j r w_j and
    d out_j / d v_i = w_j r (delta_ij - v_i v_j r^2 / d).  Hence
    dv_i = r (w_i dy_i - v_i r^2 mean_j(w_j dy_j v_j)), and the weight, shared
    by all rows, gets dw_j = sum over rows of dy_j v_j r.  Returns (dv, dw)."""
    r = 1.0 / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    wd = w * dy
    dv = r * (wd - v * r * r * np.mean(wd * v, axis=-1, keepdims=True))
    dw = np.sum((dy * v * r).reshape(-1, v.shape[-1]), axis=0)
    return dv, dw


def apply_rope_backward(g, positions, theta: float,
                        rotary_dim: Optional[int] = None):
    """Gradient through ``apply_rope`` (readings 3 and 9) for g [B, L, heads,
    d].  Each pair (i, i + r/2) is turned by a rotation matrix
    [[cos, -sin], [sin, cos]]; its transpose [[cos, sin], [-sin, cos]] carries
    the gradient back.  Entries past the rotary width pass through."""
    d = g.shape[-1]
    r = d if rotary_dim is None else int(rotary_dim)
    half = r // 2
    ang = positions.astype(np.float64)[..., None] * rope_inv_freq(r, theta)
    cos = np.cos(ang).astype(g.dtype)[:, :, None, :]
    sin = np.sin(ang).astype(g.dtype)[:, :, None, :]
    g1 = g[..., :half]
    g2 = g[..., half:r]
    return np.concatenate([g1 * cos + g2 * sin, g2 * cos - g1 * sin, g[..., r:]], axis=-1)


def grouped_attention_backward(q, k, v, q_pos, kv_len, scale: float,
                               causal: bool, do):
    """Gradients of ``grouped_attention`` for the upstream gradient do
    [B, Hq, Lq, d] (tutorial section 4, step 6; the group map of reading 5).

    Per query head h with KV head g = h // (Hq/Hkv): s = q k^T * scale over
    the visible keys, p = softmax(s) by rows, o = p v.  Then dv_g += p^T do,
    dp = do v^T, and the softmax Jacobian gives ds = p * (dp - sum_j p dp)
    row by row; dq = ds k * scale and dk_g += ds^T q * scale.  A KV head's
    gradients sum the contributions of every query head it serves.
    Returns (dq, dk, dv) shaped like q, k, v."""
    bsz, hq, lq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(bsz):
        n = int(kv_len[b])
        key_idx = np.arange(n)
        visible = np.ones((lq, n), dtype=bool)
        if causal:
            visible = key_idx[None, :] <= q_pos[b][:, None]
        for h in range(hq):
            g = h // group
            s = np.matmul(q[b, h], k[b, g, :n].T) * scale
            s = np.where(visible, s, -np.inf)
            m = np.max(s, axis=-1, keepdims=True)
            p = np.exp(s - m)
            p = p / np.sum(p, axis=-1, keepdims=True)
            dv[b, g, :n] += np.matmul(p.T, do[b, h])
            dp = np.matmul(do[b, h], v[b, g, :n].T)
            ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
            dq[b, h] = np.matmul(ds, k[b, g, :n]) * scale
            dk[b, g, :n] += np.matmul(ds.T, q[b, h]) * scale
    return dq, dk, dv


def layer_backward(res: Resolved, x, w_qkv, q_norm_w, k_norm_w, w_o, dout, *,
                   rope_theta: float, rms_eps: float, qk_norm: bool = True,
                   causal: bool = True, rotary_dim: Optional[int] = None,
                   dtype=np.float64):
    """Gradients of ``layer_forward`` without a cache (positions 0..L-1) for
    the upstream gradient dout [B, L, hidden] (reading 11): the chain rule
    through the forward's steps in reverse order -- o_proj, attention, RoPE,
    QK-norm, the fused projection.

    Returns a dict with dx [B, L, hidden], dw_qkv [(Hq+2Hkv)d, hidden],
    dq_norm_w and dk_norm_w [d] (None without QK-norm) and dw_o
    [hidden, Hq*d]."""
    x = np.asarray(x, dtype=dtype)
    w_qkv = np.asarray(w_qkv, dtype=dtype)
    w_o = np.asarray(w_o, dtype=dtype)
    dout = np.asarray(dout, dtype=dtype)
    bsz, seq, _ = x.shape
    positions = np.tile(np.arange(seq, dtype=np.int64), (bsz, 1))
    kw = {} if rotary_dim is None else {"rotary_dim": rotary_dim}
    # forward, keeping what the backward reads
    y = project(x, w_qkv)
    q0, k0, v0 = split_heads(y, res)
    qn, kn = q0, k0
    if qk_norm:
        qnw = np.asarray(q_norm_w, dtype=dtype)
        knw = np.asarray(k_norm_w, dtype=dtype)
        qn = rms_norm_heads(q0, qnw, rms_eps)
        kn = rms_norm_heads(k0, knw, rms_eps)
    qr = apply_rope(qn, positions, rope_theta, **kw)
    kr = apply_rope(kn, positions, rope_theta, **kw)
    qh, kh, vh = (qr.transpose(0, 2, 1, 3), kr.transpose(0, 2, 1, 3),
                  v0.transpose(0, 2, 1, 3))
    kv_len = np.full(bsz, seq, dtype=np.int64)
    o = grouped_attention(qh, kh, vh, positions, kv_len, res.scale, causal)
    om = merge_heads(o)
    # backward
    dom, dw_o = project_backward(om, w_o, dout)
    do = dom.reshape(bsz, seq, res.hq, res.d).transpose(0, 2, 1, 3)
    dqh, dkh, dvh = grouped_attention_backward(qh, kh, vh, positions, kv_len,
                                               res.scale, causal, do)
    dqn = apply_rope_backward(dqh.transpose(0, 2, 1, 3), positions, rope_theta, **kw)
    dkn = apply_rope_backward(dkh.transpose(0, 2, 1, 3), positions, rope_theta, **kw)
    dq_norm_w = dk_norm_w = None
    dq0, dk0 = dqn, dkn
    if qk_norm:
        dq0, dq_norm_w = rms_norm_heads_backward(q0, qnw, rms_eps, dqn)
        dk0, dk_norm_w = rms_norm_heads_backward(k0, knw, rms_eps, dkn)
    dy = np.concatenate([dq0.reshape(bsz, seq, -1), dk0.reshape(bsz, seq, -1),
                         dvh.transpose(0, 2, 1, 3).reshape(bsz, seq, -1)], axis=-1)
    dx, dw_qkv = project_backward(x, w_qkv, dy)
    return {"dx": dx, "dw_qkv": dw_qkv, "dq_norm_w": dq_norm_w,
            "dk_norm_w": dk_norm_w, "dw_o": dw_o}
