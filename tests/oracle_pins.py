"""Pins of the CPU oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own formulas.

Each ``check_*`` function raises AssertionError when the oracle disagrees.
They are plain functions so that ``test_oracle_mutations`` can rerun them
against an oracle with a planted mistake and show that some pin fails.
All access to the oracle goes through the module object ``O`` so that a
patched function is the one exercised.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from oracle import gqa_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def golden():
    with open(os.path.join(HERE, "golden", "page_figures.json")) as f:
        return json.load(f)


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _layer_case(seed=0, b=2, l=9, hidden=24, hq=4, hkv=2, d=8):
    rng = np.random.default_rng(seed)
    res = O.resolve_config(hidden, hq, hkv, d)
    x = _rand(rng, b, l, hidden)
    w_qkv = _rand(rng, res.n_qkv, hidden, scale=0.3)
    qn = 1.0 + _rand(rng, d, scale=0.1)
    kn = 1.0 + _rand(rng, d, scale=0.1)
    w_o = _rand(rng, hidden, res.q_width, scale=0.3)
    return res, x, w_qkv, qn, kn, w_o


# ---------------------------------------------------------------------------
# Configuration, shapes and counts (page figures)
# ---------------------------------------------------------------------------

def check_geometries():
    g = golden()
    q = g["qwen3_0_6b_geometry"]
    r = O.resolve_config(q["hidden_size"], q["num_attention_heads"],
                         q["num_kv_heads"], q["head_dim"])
    assert r.d == q["head_dim"]
    assert r.q_width == q["query_hidden_size"]
    assert r.kv_width == q["kv_hidden_size"]
    assert r.n_qkv == q["qkv_out"]
    s = O.weight_shapes(r)
    assert s["o_proj"] == (q["o_proj_out"], q["o_proj_in"])
    assert s["query_key_value"] == (q["qkv_out"], q["hidden_size"])
    qp = q["quotient_path"]
    r0 = O.resolve_config(q["hidden_size"], q["num_attention_heads"],
                          q["num_kv_heads"], None)
    assert r0.d == qp["head_dim"] and r0.n_qkv == qp["qkv_out"]
    assert r0.kv_width == qp["kv_hidden_size"] and r0.q_width == qp["o_proj_in"]

    q4 = g["qwen3_4b_geometry"]
    r = O.resolve_config(q4["hidden_size"], q4["num_attention_heads"], None,
                         q4["head_dim"])
    s = O.weight_shapes(r)
    assert list(s["q_proj"]) == q4["q_proj_weight"]
    assert list(s["o_proj"]) == q4["o_proj_weight"]
    r0 = O.resolve_config(q4["hidden_size"], q4["num_attention_heads"])
    assert r0.d == q4["quotient"]

    q8 = g["qwen3_8b_geometry"]
    r = O.resolve_config(q8["hidden_size"], q8["num_attention_heads"],
                         q8["num_kv_heads"], q8["head_dim"])
    s = O.weight_shapes(r)
    assert list(s["q_proj"]) == q8["w_q"] and list(s["k_proj"]) == q8["w_k"]
    assert list(s["v_proj"]) == q8["w_v"] and list(s["o_proj"]) == q8["w_o"]
    assert O.resolve_config(q8["hidden_size"], q8["num_attention_heads"],
                            q8["num_kv_heads"]).d == q8["head_dim"]
    # the tutorial's reshape flow, run through the oracle's own steps
    fl = q8["reshape_flow"]
    res_small = O.resolve_config(q8["hidden_size"], q8["num_attention_heads"],
                                 q8["num_kv_heads"], q8["head_dim"])
    y = np.zeros(fl["x"][:2] + [res_small.n_qkv])
    qh, kh, vh = O.split_heads(y, res_small)
    assert list(qh.shape) == fl["heads"]
    assert list(qh.transpose(0, 2, 1, 3).shape) == fl["transposed"]
    assert list(O.merge_heads(qh.transpose(0, 2, 1, 3)).shape) == fl["flat"]

    gm = g["gemma3_geometry"]
    r = O.resolve_config(gm["hidden_size"], gm["num_attention_heads"], None,
                         gm["head_dim"])
    assert r.d == gm["head_dim"]
    assert O.resolve_config(gm["hidden_size"], gm["num_attention_heads"]).d \
        == gm["quotient"]


def check_resolve_errors():
    # divisibility is required only when head_dim must be derived
    O.resolve_config(1000, 16, 8, 128)
    try:
        O.resolve_config(1000, 16, 8, None)
    except O.ConfigError:
        pass
    else:
        raise AssertionError("indivisible hidden_size accepted with head_dim unset")
    for bad in [dict(num_kv_heads=3), dict(head_dim=127)]:
        try:
            O.resolve_config(1024, 16, bad.get("num_kv_heads", 8),
                             bad.get("head_dim", 128))
        except O.ConfigError:
            pass
        else:
            raise AssertionError(f"{bad} accepted")
    r = O.resolve_config(1024, 16)
    assert r.hkv == 16 and r.group == 1
    assert abs(O.resolve_config(256, 4, 2, 128).scale - 128 ** -0.5) < 1e-15


def check_param_counts():
    g = golden()
    c = g["param_counts_d_model_512_quotient"]
    for case in c["cases"]:
        # d = 512/512 = 1 at the far end: odd, so no RoPE check here
        r = O.resolve_config(c["d_model"], case["heads"], require_even=False)
        assert O.attention_param_count(r) == case["params"], case
    c = g["param_counts_d_model_512_head_dim_128"]
    for case in c["cases"]:
        r = O.resolve_config(c["d_model"], case["heads"], None, c["head_dim"])
        assert O.attention_param_count(r) == case["params"], case


def check_macs():
    c = golden()["macs_per_token_d_model_512"]
    for h in c["heads_checked"]:
        r = O.resolve_config(c["d_model"], h, require_even=False)
        for case in c["score_value_cases"]:
            m = O.macs_per_token(r, case["n"])
            assert m["score_value"] == case["macs"], (h, case)
            assert m["projection"] == c["projection_macs"]


# ---------------------------------------------------------------------------
# Steps against brute force and library routines
# ---------------------------------------------------------------------------

def check_projection_bruteforce():
    rng = np.random.default_rng(1)
    x = _rand(rng, 2, 3, 5)
    w = _rand(rng, 4, 5)
    y = O.project(x, w)
    for b in range(2):
        for t in range(3):
            for n in range(4):
                acc = 0.0
                for k in range(5):
                    acc += x[b, t, k] * w[n, k]
                assert abs(y[b, t, n] - acc) < 1e-12


def _brute_attention(q, k, v, q_pos, kv_len, scale, causal):
    """Pure-Python loops with math.exp (no numpy reductions)."""
    bsz, hq, lq, d = q.shape
    hkv = k.shape[1]
    per = hq // hkv
    out = np.zeros_like(q)
    for b in range(bsz):
        for h in range(hq):
            g = h // per
            for i in range(lq):
                keys = [j for j in range(int(kv_len[b]))
                        if (not causal) or j <= q_pos[b][i]]
                scores = []
                for j in keys:
                    s = 0.0
                    for e in range(d):
                        s += q[b, h, i, e] * k[b, g, j, e]
                    scores.append(s * scale)
                mx = max(scores)
                ws = [math.exp(s - mx) for s in scores]
                tot = sum(ws)
                for e in range(d):
                    acc = 0.0
                    for w_, j in zip(ws, keys):
                        acc += w_ * v[b, g, j, e]
                    out[b, h, i, e] = acc / tot
    return out


def check_attention_bruteforce():
    rng = np.random.default_rng(2)
    q = _rand(rng, 1, 4, 7, 8)
    k = _rand(rng, 1, 2, 7, 8)
    v = _rand(rng, 1, 2, 7, 8)
    pos = np.arange(7)[None, :]
    for causal in (True, False):
        got = O.grouped_attention(q, k, v, pos, np.array([7]), 8 ** -0.5, causal)
        ref = _brute_attention(q, k, v, pos, [7], 8 ** -0.5, causal)
        assert np.max(np.abs(got - ref)) < 1e-12
    # a chunk of 3 queries at the end of 7 cached keys (bottom-right aligned)
    qc = q[:, :, :3]
    pos = np.array([[4, 5, 6]])
    got = O.grouped_attention(qc, k, v, pos, np.array([7]), 0.3, True)
    ref = _brute_attention(qc, k, v, pos, [7], 0.3, True)
    assert np.max(np.abs(got - ref)) < 1e-12


def check_attention_vs_torch_sdpa():
    rng = np.random.default_rng(3)
    for hq, hkv in [(4, 4), (4, 2), (8, 1)]:
        q = _rand(rng, 2, hq, 11, 16)
        k = _rand(rng, 2, hkv, 11, 16)
        v = _rand(rng, 2, hkv, 11, 16)
        pos = np.tile(np.arange(11), (2, 1))
        got = O.grouped_attention(q, k, v, pos, np.array([11, 11]), 0.25, True)
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=True, scale=0.25, enable_gqa=True).numpy()
        assert np.max(np.abs(got - ref)) < 1e-12, (hq, hkv)
    # queries at the tail of a longer key range: explicit bottom-right mask
    q = _rand(rng, 1, 4, 3, 16)
    k = _rand(rng, 1, 2, 10, 16)
    v = _rand(rng, 1, 2, 10, 16)
    pos = np.array([[7, 8, 9]])
    mask = torch.from_numpy(np.arange(10)[None, :] <= pos[0][:, None])
    got = O.grouped_attention(q, k, v, pos, np.array([10]), 0.25, True)
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=mask, scale=0.25, enable_gqa=True).numpy()
    assert np.max(np.abs(got - ref)) < 1e-12


def check_layer_mha_reduces_to_torch_mha():
    """Hkv = Hq, d = hidden/Hq, no QK-norm and no RoPE: the layer is the
    Concat(head_i) W_O multi-head attention of "num_heads Is Not a Capacity
    Knob", "Why the cost does not move"; torch's packed in_proj weight uses
    the same q | k | v row order."""
    rng = np.random.default_rng(4)
    hidden, heads, L = 32, 4, 10
    res = O.resolve_config(hidden, heads)
    x = _rand(rng, 2, L, hidden)
    w_qkv = _rand(rng, res.n_qkv, hidden, scale=0.3)
    w_o = _rand(rng, hidden, res.q_width, scale=0.3)
    got, _, _ = O.layer_forward(res, x, w_qkv, None, None, w_o, rope_theta=1e4,
                                rms_eps=1e-6, qk_norm=False, rope=False)
    xt = torch.from_numpy(x).transpose(0, 1)   # [L, B, E]
    mask = torch.triu(torch.ones(L, L, dtype=torch.bool), diagonal=1)
    ref, _ = F.multi_head_attention_forward(
        xt, xt, xt, hidden, heads, torch.from_numpy(w_qkv), None, None, None,
        False, 0.0, torch.from_numpy(w_o), None, training=False,
        need_weights=False, attn_mask=mask)
    ref = ref.transpose(0, 1).numpy()
    assert np.max(np.abs(got - ref)) < 1e-12


def _torch_rope_complex(v, positions, theta):
    """RoPE as complex multiplication: z_i = v_i + 1j*v_{i+d/2} times
    exp(1j * p * theta**(-2i/d))."""
    d = v.shape[-1]
    half = d // 2
    t = torch.from_numpy(v)
    z = torch.complex(t[..., :half], t[..., half:])
    i = torch.arange(half, dtype=torch.float64)
    ang = torch.from_numpy(positions).double()[..., None] * \
        torch.pow(torch.tensor(theta, dtype=torch.float64), -2.0 * i / d)
    rot = torch.polar(torch.ones_like(ang), ang)[:, :, None, :]
    z = z * rot
    return torch.cat([z.real, z.imag], dim=-1).numpy()


def check_layer_vs_torch_composition():
    """The whole layer with Hq*d != hidden, QK-norm, RoPE, GQA and a causal
    mask, composed from torch library routines (F.linear, F.rms_norm, RoPE as
    complex multiplication, SDPA with enable_gqa), in float64."""
    res, x, w_qkv, qn, kn, w_o = _layer_case(seed=5, b=2, l=9, hidden=24,
                                             hq=4, hkv=2, d=8)
    theta, eps = 1e4, 1e-6
    got, _, _ = O.layer_forward(res, x, w_qkv, qn, kn, w_o, rope_theta=theta,
                                rms_eps=eps)
    b, l, _ = x.shape
    y = F.linear(torch.from_numpy(x), torch.from_numpy(w_qkv))
    q = y[..., :res.q_width].reshape(b, l, res.hq, res.d)
    k = y[..., res.q_width:res.q_width + res.kv_width].reshape(b, l, res.hkv, res.d)
    v = y[..., res.q_width + res.kv_width:].reshape(b, l, res.hkv, res.d)
    q = F.rms_norm(q, (res.d,), torch.from_numpy(qn), eps)
    k = F.rms_norm(k, (res.d,), torch.from_numpy(kn), eps)
    pos = np.tile(np.arange(l), (b, 1))
    q = torch.from_numpy(_torch_rope_complex(q.numpy(), pos, theta))
    k = torch.from_numpy(_torch_rope_complex(k.numpy(), pos, theta))
    o = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2),
                                       v.transpose(1, 2), is_causal=True,
                                       enable_gqa=True)
    ref = F.linear(o.transpose(1, 2).reshape(b, l, res.q_width),
                   torch.from_numpy(w_o)).numpy()
    assert np.max(np.abs(got - ref)) < 1e-10


def check_rmsnorm():
    rng = np.random.default_rng(6)
    v = _rand(rng, 3, 5, 4, 16, scale=3.0)
    w = 1.0 + _rand(rng, 16, scale=0.1)
    got = O.rms_norm_heads(v, w, 1e-6)
    ref = F.rms_norm(torch.from_numpy(v), (16,), torch.from_numpy(w), 1e-6).numpy()
    assert np.max(np.abs(got - ref)) < 1e-12
    unit = O.rms_norm_heads(v, np.ones(16), 0.0)
    assert np.max(np.abs(np.sqrt(np.mean(unit ** 2, axis=-1)) - 1.0)) < 1e-12
    # scale invariance: norm(c * v) == norm(v) for c > 0 (eps = 0)
    assert np.max(np.abs(O.rms_norm_heads(7.5 * v, w, 0.0)
                         - O.rms_norm_heads(v, w, 0.0))) < 1e-12


def check_rope():
    rng = np.random.default_rng(7)
    v = _rand(rng, 2, 6, 3, 16)
    pos = np.array([[0, 1, 2, 100, 5000, 32768], [7, 7, 8, 9, 10, 65535]])
    theta = 1e6
    got = O.apply_rope(v, pos, theta)
    # identity at position 0
    z = O.apply_rope(v, np.zeros_like(pos), theta)
    assert np.max(np.abs(z - v)) < 1e-15
    # norm preserving per head
    assert np.max(np.abs(np.linalg.norm(got, axis=-1)
                         - np.linalg.norm(v, axis=-1))) < 1e-10
    # complex-multiplication form
    ref = _torch_rope_complex(v, pos, theta)
    assert np.max(np.abs(got - ref)) < 1e-10
    # relative position: <R(p) a, R(p') b> depends only on p' - p
    a = _rand(rng, 1, 1, 1, 16)
    bb = _rand(rng, 1, 1, 1, 16)
    dots = []
    for shift in (0, 13, 4096):
        ra = O.apply_rope(a, np.array([[3 + shift]]), theta)
        rb = O.apply_rope(bb, np.array([[11 + shift]]), theta)
        dots.append(float(np.sum(ra * rb)))
    assert max(dots) - min(dots) < 1e-10


def check_partial_rope():
    """Partial rotary (reading 9) against closed forms: with rotary_dim 2 the
    single pair (0, 1) turns by angle p (theta**0); with rotary_dim 4 the
    pairs (0, 2) and (1, 3) turn by p and p * theta**(-1/2); the entries past
    rotary_dim are untouched, and rotary_dim = d is the full RoPE."""
    rng = np.random.default_rng(11)
    theta = 1e4
    pos = np.array([[0, 1, 3, 1000]])
    v = _rand(rng, 1, 4, 2, 8)
    for r, pairs in ((2, [(0, 1, 1.0)]), (4, [(0, 2, 1.0), (1, 3, theta ** -0.5)])):
        got = O.apply_rope(v, pos, theta, rotary_dim=r)
        assert np.array_equal(got[..., r:], v[..., r:])
        for i, j, f in pairs:
            a = pos[0][:, None] * f  # [L, 1], one angle per position
            c, s_ = np.cos(a), np.sin(a)
            x1, x2 = v[0, :, :, i], v[0, :, :, j]
            assert np.max(np.abs(got[0, :, :, i] - (x1 * c - x2 * s_))) < 1e-12
            assert np.max(np.abs(got[0, :, :, j] - (x2 * c + x1 * s_))) < 1e-12
    assert np.array_equal(O.apply_rope(v, pos, theta, rotary_dim=8), O.apply_rope(v, pos, theta))


def check_position_shift_invariance():
    """Shifting every position by the same offset leaves scores, and so the
    attention output, unchanged (RoPE's relative-position property)."""
    res, x, w_qkv, qn, kn, w_o = _layer_case(seed=8)
    b, l, _ = x.shape
    outs = []
    for shift in (0, 1000):
        pos = np.tile(np.arange(l), (b, 1)) + shift
        q, k, v = O.qkv_normrope(res, x, w_qkv, qn, kn, pos, 1e4, 1e-6)
        o = O.grouped_attention(q, k, v, pos - shift, np.full(b, l), res.scale)
        outs.append(o)
    assert np.max(np.abs(outs[0] - outs[1])) < 1e-10


def check_causality():
    """Changing x at t' leaves rows t < t' unchanged (a nontrivial sequence
    length, per "Attention head partitions ...": a single token cannot show
    a future-token leak)."""
    res, x, w_qkv, qn, kn, w_o = _layer_case(seed=9, l=12)
    base, _, _ = O.layer_forward(res, x, w_qkv, qn, kn, w_o, rope_theta=1e4,
                                 rms_eps=1e-6)
    for tp in (3, 11):
        x2 = x.copy()
        x2[:, tp] += 5.0
        pert, _, _ = O.layer_forward(res, x2, w_qkv, qn, kn, w_o,
                                     rope_theta=1e4, rms_eps=1e-6)
        assert np.max(np.abs(pert[:, :tp] - base[:, :tp])) < 1e-12
        assert np.max(np.abs(pert[:, tp] - base[:, tp])) > 1e-3


def check_gqa_equals_repeated_kv():
    """GQA equals MHA with each KV head repeated for its Hq/Hkv query heads
    (contiguous groups), on per-head-distinguishable values."""
    rng = np.random.default_rng(10)
    hq, hkv, L, d = 8, 2, 9, 6
    q = _rand(rng, 1, hq, L, d)
    k = _rand(rng, 1, hkv, L, d)
    v = _rand(rng, 1, hkv, L, d) + np.arange(hkv)[None, :, None, None] * 10.0
    pos = np.arange(L)[None, :]
    got = O.grouped_attention(q, k, v, pos, np.array([L]), 0.4)
    kr = np.repeat(k, hq // hkv, axis=1)
    vr = np.repeat(v, hq // hkv, axis=1)
    ref = O.grouped_attention(q, kr, vr, pos, np.array([L]), 0.4)
    assert np.max(np.abs(got - ref)) < 1e-12
    # heads are distinguishable: query head h's output carries KV head h//4's offset
    means = got.mean(axis=(2, 3))[0]
    for h in range(hq):
        assert abs(means[h] - 10.0 * (h // (hq // hkv))) < 3.0


def check_rank_ceiling():
    """rank(q k^T) <= d_head ("num_heads Is Not a Capacity Knob", "What a
    head cannot express")."""
    res, x, w_qkv, qn, kn, w_o = _layer_case(seed=11, b=1, l=40, hidden=24,
                                             hq=2, hkv=1, d=4)
    pos = np.arange(40)[None, :]
    q, k, v = O.qkv_normrope(res, x, w_qkv, qn, kn, pos, 1e4, 1e-6)
    s = q[0, 0] @ k[0, 0].T
    assert np.linalg.matrix_rank(s) <= res.d
    assert np.linalg.matrix_rank(s) == res.d


def check_one_dim_head():
    """With d_head = 1 and no RoPE every query ranks the visible keys the
    same way, reversed when its own coordinate is negative."""
    rng = np.random.default_rng(12)
    L = 16
    a = _rand(rng, 1, 1, L, 1)
    bk = _rand(rng, 1, 1, L, 1)
    v = np.eye(L)[None, None]          # value j = one-hot(j): output = weights
    pos = np.arange(L)[None, :]
    w = O.grouped_attention(a, bk, v, pos, np.array([L]), 1.0)[0, 0]
    for t in range(1, L):
        order_keys = np.argsort(bk[0, 0, :t + 1, 0], kind="stable")
        order_w = np.argsort(w[t, :t + 1], kind="stable")
        if a[0, 0, t, 0] > 0:
            assert list(order_w) == list(order_keys)
        else:
            assert list(order_w) == list(order_keys[::-1])


def check_sum_over_heads():
    """out = sum_h O_h W_o[:, h*d:(h+1)*d]^T; zeroing one head's W_o slice
    removes exactly that head's term ("Why the cost does not move")."""
    res, x, w_qkv, qn, kn, w_o = _layer_case(seed=13)
    b, l, _ = x.shape
    pos = np.tile(np.arange(l), (b, 1))
    q, k, v = O.qkv_normrope(res, x, w_qkv, qn, kn, pos, 1e4, 1e-6)
    o = O.grouped_attention(q, k, v, pos, np.full(b, l), res.scale)
    full, _, _ = O.layer_forward(res, x, w_qkv, qn, kn, w_o, rope_theta=1e4,
                                 rms_eps=1e-6)
    terms = [o[:, h] @ w_o[:, h * res.d:(h + 1) * res.d].T for h in range(res.hq)]
    assert np.max(np.abs(sum(terms) - full)) < 1e-12
    w_pruned = w_o.copy()
    w_pruned[:, 1 * res.d:2 * res.d] = 0.0
    pruned, _, _ = O.layer_forward(res, x, w_qkv, qn, kn, w_pruned,
                                   rope_theta=1e4, rms_eps=1e-6)
    assert np.max(np.abs(pruned - (full - terms[1]))) < 1e-12


def check_prefill_equals_decode():
    """Prefill over L tokens equals prefill of a prefix followed by cached
    chunks (step 5, update_and_fetch, appends before attending)."""
    res, x, w_qkv, qn, kn, w_o = _layer_case(seed=14, b=2, l=10)
    kw = dict(rope_theta=1e4, rms_eps=1e-6)
    full, _, _ = O.layer_forward(res, x, w_qkv, qn, kn, w_o, **kw)
    cap = 10
    kc = np.full((2, res.hkv, cap, res.d), np.nan)
    vc = np.full((2, res.hkv, cap, res.d), np.nan)
    o1, kc, vc = O.layer_forward(res, x[:, :6], w_qkv, qn, kn, w_o, k_cache=kc,
                                 v_cache=vc, cache_len=np.array([0, 0]), **kw)
    o2, kc, vc = O.layer_forward(res, x[:, 6:9], w_qkv, qn, kn, w_o, k_cache=kc,
                                 v_cache=vc, cache_len=np.array([6, 6]), **kw)
    o3, kc, vc = O.layer_forward(res, x[:, 9:], w_qkv, qn, kn, w_o, k_cache=kc,
                                 v_cache=vc, cache_len=np.array([9, 9]), **kw)
    got = np.concatenate([o1, o2, o3], axis=1)
    assert np.max(np.abs(got - full)) < 1e-12


def check_quotient_equals_explicit():
    rng = np.random.default_rng(15)
    r0 = O.resolve_config(32, 4, 2, None)
    r1 = O.resolve_config(32, 4, 2, 8)
    assert r0 == r1
    x = _rand(rng, 1, 7, 32)
    w_qkv = _rand(rng, r0.n_qkv, 32, scale=0.3)
    w_o = _rand(rng, 32, r0.q_width, scale=0.3)
    a, _, _ = O.layer_forward(r0, x, w_qkv, None, None, w_o, rope_theta=5e5,
                              rms_eps=1e-6, qk_norm=False)
    b, _, _ = O.layer_forward(r1, x, w_qkv, None, None, w_o, rope_theta=5e5,
                              rms_eps=1e-6, qk_norm=False)
    assert np.array_equal(a, b)


def check_rows_mode():
    res, x, w_qkv, qn, kn, w_o = _layer_case(seed=16, b=2, l=11)
    kw = dict(rope_theta=1e4, rms_eps=1e-6)
    full, _, _ = O.layer_forward(res, x, w_qkv, qn, kn, w_o, **kw)
    rows = [(0, 0), (0, 5), (1, 10), (1, 3), (0, 10)]
    got = O.layer_forward_rows(res, x, w_qkv, qn, kn, w_o, rows, **kw)
    for i, (b, t) in enumerate(rows):
        assert np.max(np.abs(got[i] - full[b, t])) < 1e-12


# ---------------------------------------------------------------------------
# FP8 (E4M3) cache entries (reading 10)
# ---------------------------------------------------------------------------

def check_e4m3_closed_forms():
    """Values fixed by the format's definition (1 sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits, no infinities): 1.0, the largest finite
    448, the smallest normal 2^-6, the smallest subnormal 2^-9, the NaN
    codes, signed zero, 254 finite values in increasing order."""
    v = O.e4m3_value(np.arange(256))
    fixed = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0x7E: 448.0, 0x08: 2.0 ** -6,
             0x07: 7 * 2.0 ** -9, 0x01: 2.0 ** -9, 0x30: 0.5, 0xB8: -1.0, 0xFE: -448.0}
    for c, want in fixed.items():
        assert v[c] == want, (hex(c), v[c], want)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[0x80:0xFF], -pos)


def _e4m3_nearest_bruteforce(x):
    """Nearest finite E4M3 value by searching the value table: saturate,
    take the smallest distance, break ties toward the even code."""
    table = O.e4m3_value(np.arange(0x7F))  # the 127 non-negative finite values
    out = []
    for xi in np.asarray(x, dtype=np.float64):
        a = min(abs(xi), 448.0)
        dist = np.abs(table - a)
        best = np.flatnonzero(dist == dist.min())
        c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
        if np.signbit(xi):
            c |= 0x80
        out.append(c)
    return np.array(out, dtype=np.uint8)


def check_e4m3_quantize_bruteforce():
    """The quantizer against a search over the value table: every finite
    value, every midpoint between neighbours (ties), points just either side
    of them, out-of-range magnitudes and random values over the range."""
    v = O.e4m3_value(np.arange(0x7F))
    mids = 0.5 * (v[:-1] + v[1:])
    pts = np.concatenate([v, mids, np.nextafter(mids, 0.0), np.nextafter(mids, 1e9),
                          [448.0, 460.0, 464.0, 500.0, 1e6, 2.0 ** -10, 1e-30, 0.0]])
    rng = np.random.default_rng(40)
    pts = np.concatenate([pts, rng.standard_normal(4000) * np.exp2(rng.integers(-12, 10, 4000))])
    pts = np.concatenate([pts, -pts])
    got = O.quantize_e4m3(pts)
    want = _e4m3_nearest_bruteforce(pts)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(pts[i], int(got[i]), int(want[i])) for i in bad[:5]]
    # the stored value is within half a quantum of the (saturated) input
    a = np.minimum(np.abs(pts), 448.0)
    err = np.abs(np.abs(O.e4m3_value(got)) - a)
    q = np.exp2(np.clip(np.floor(np.log2(np.maximum(a, 2.0 ** -9))), -6, 8) - 3)
    assert np.all(err <= q / 2 + 1e-300)


def check_fp8_cache_layer():
    """With kv_fp8, the appended rows are the codes of k / k_scale and
    v / v_scale, and the output is the plain layer's run on caches holding
    the stored values (attention reads the cache, not the fresh rows); with
    a power-of-two scale the codes are the unscaled codes' exponents
    shifted."""
    res, x, w_qkv, qn, kn, w_o = _layer_case(seed=41, b=2, l=3)
    kw = dict(rope_theta=1e4, rms_eps=1e-6)
    cap, c0 = 9, np.array([4, 6])
    rng = np.random.default_rng(42)
    kc = O.quantize_e4m3(rng.standard_normal((2, res.hkv, cap, res.d)))
    vc = O.quantize_e4m3(rng.standard_normal((2, res.hkv, cap, res.d)))
    ks, vs = 0.5, 3.0
    out, kc2, vc2 = O.layer_forward(res, x, w_qkv, qn, kn, w_o, k_cache=kc, v_cache=vc,
                                    cache_len=c0, kv_fp8=True, k_scale=ks, v_scale=vs, **kw)
    pos = c0[:, None] + np.arange(3)[None, :]
    q, k, v = O.qkv_normrope(res, x, w_qkv, qn, kn, pos, kw["rope_theta"], kw["rms_eps"])
    for b in range(2):
        s0 = int(c0[b])
        assert np.array_equal(kc2[b, :, s0:s0 + 3], O.quantize_e4m3(k[b] / ks))
        assert np.array_equal(vc2[b, :, s0:s0 + 3], O.quantize_e4m3(v[b] / vs))
        assert np.array_equal(kc2[b, :, :s0], kc[b, :, :s0])
    kvals = O.e4m3_value(kc2) * ks
    vvals = O.e4m3_value(vc2) * vs
    o = O.grouped_attention(q, kvals, vvals, pos, c0 + 3, res.scale, True)
    ref = O.project(O.merge_heads(o), w_o)
    assert np.max(np.abs(out - ref)) < 1e-12
    # scale 1/2 on values in the normal range doubles them: exponent + 1
    xs = np.array([0.3, -1.7, 5.0, 100.0])
    assert np.array_equal(O.quantize_e4m3(xs / 0.5), O.quantize_e4m3(xs) + 8)


# ---------------------------------------------------------------------------
# Backward pass (reading 11)
# ---------------------------------------------------------------------------

def _layer_loss(res, x, w_qkv, qn, kn, w_o, dout, **kw):
    out, _, _ = O.layer_forward(res, x, w_qkv, qn, kn, w_o, **kw)
    return float(np.sum(out * dout))


BWD_CASES = [
    # (seed, b, l, hidden, hq, hkv, d, qk_norm, causal, rotary_dim)
    (20, 2, 5, 12, 4, 2, 6, True, True, None),     # GQA, Hq*d != hidden
    (21, 1, 6, 16, 4, 1, 8, True, False, 4),       # MQA, no mask, partial rotary
    (22, 2, 4, 8, 2, 2, 4, False, True, None),     # MHA without QK-norm
]


def check_layer_backward_finite_differences():
    """Every gradient of the layer against central differences of
    sum(dout * layer_forward(...)) in float64, on sampled entries of each
    input and parameter (step 1e-6: truncation and rounding stay near 1e-9
    for these O(1) values).  The difference quotient uses only the forward,
    so a mistake anywhere in the backward shows."""
    for seed, b, l, hid, hq, hkv, d, qkn, causal, rot in BWD_CASES:
        rng = np.random.default_rng(seed)
        res, x, w_qkv, qn, kn, w_o = _layer_case(seed=seed, b=b, l=l, hidden=hid,
                                                 hq=hq, hkv=hkv, d=d)
        dout = _rand(rng, b, l, hid)
        kw = dict(rope_theta=100.0, rms_eps=1e-6, qk_norm=qkn, causal=causal,
                  rotary_dim=rot)
        g = O.layer_backward(res, x, w_qkv, qn if qkn else None, kn if qkn else None,
                             w_o, dout, **kw)
        args = {"x": x, "w_qkv": w_qkv, "qn": qn, "kn": kn, "w_o": w_o}
        keys = {"x": "dx", "w_qkv": "dw_qkv", "qn": "dq_norm_w", "kn": "dk_norm_w",
                "w_o": "dw_o"}
        h = 1e-6
        for name, key in keys.items():
            if not qkn and name in ("qn", "kn"):
                assert g[key] is None
                continue
            arr = args[name]
            assert g[key].shape == arr.shape, (key, g[key].shape, arr.shape)
            flat = rng.choice(arr.size, size=min(arr.size, 24), replace=False)
            for fi in flat:
                idx = np.unravel_index(fi, arr.shape)
                vals = []
                for sgn in (1.0, -1.0):
                    a = arr.copy()
                    a[idx] += sgn * h
                    call = dict(args, **{name: a})
                    vals.append(_layer_loss(res, call["x"], call["w_qkv"],
                                            call["qn"] if qkn else None,
                                            call["kn"] if qkn else None,
                                            call["w_o"], dout, **kw))
                fd = (vals[0] - vals[1]) / (2 * h)
                assert abs(fd - g[key][idx]) < 1e-6 * max(1.0, abs(fd)), \
                    (seed, key, idx, fd, g[key][idx])


def check_layer_backward_vs_torch_autograd():
    """All five gradients against torch autograd through an independent
    float64 composition of library routines (F.linear, F.rms_norm, RoPE as
    complex multiplication, SDPA with enable_gqa), GQA with a causal mask."""
    res, x, w_qkv, qn, kn, w_o = _layer_case(seed=23, b=2, l=7, hidden=24, hq=6, hkv=2, d=8)
    rng = np.random.default_rng(24)
    dout = _rand(rng, 2, 7, 24)
    theta, eps = 1e3, 1e-6
    g = O.layer_backward(res, x, w_qkv, qn, kn, w_o, dout, rope_theta=theta, rms_eps=eps)
    t = {n: torch.from_numpy(a.copy()).requires_grad_(True)
         for n, a in (("x", x), ("w_qkv", w_qkv), ("qn", qn), ("kn", kn), ("w_o", w_o))}
    b, l, _ = x.shape
    y = F.linear(t["x"], t["w_qkv"])
    q = y[..., :res.q_width].reshape(b, l, res.hq, res.d)
    k = y[..., res.q_width:res.q_width + res.kv_width].reshape(b, l, res.hkv, res.d)
    v = y[..., res.q_width + res.kv_width:].reshape(b, l, res.hkv, res.d)
    q = F.rms_norm(q, (res.d,), t["qn"], eps)
    k = F.rms_norm(k, (res.d,), t["kn"], eps)
    half = res.d // 2
    i = torch.arange(half, dtype=torch.float64)
    ang = torch.arange(l, dtype=torch.float64)[:, None] * \
        torch.pow(torch.tensor(theta, dtype=torch.float64), -2.0 * i / res.d)
    rot = torch.polar(torch.ones_like(ang), ang)[None, :, None, :]

    def rope(u):
        z = torch.complex(u[..., :half], u[..., half:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    o = F.scaled_dot_product_attention(rope(q).transpose(1, 2), rope(k).transpose(1, 2),
                                       v.transpose(1, 2), is_causal=True, enable_gqa=True)
    out = F.linear(o.transpose(1, 2).reshape(b, l, res.q_width), t["w_o"])
    out.backward(torch.from_numpy(dout))
    for name, key in (("x", "dx"), ("w_qkv", "dw_qkv"), ("qn", "dq_norm_w"),
                      ("kn", "dk_norm_w"), ("w_o", "dw_o")):
        ref = t[name].grad.numpy()
        assert np.max(np.abs(g[key] - ref)) < 1e-10 * max(1.0, np.abs(ref).max()), key


def check_attention_backward_group_sum():
    """The gradient of a shared KV head is the sum, over the query heads it
    serves, of the gradients of the repeated-KV multi-head layer, and the
    query gradients are those of that layer (per-head-distinguishable
    values, causal, a ragged key range)."""
    rng = np.random.default_rng(25)
    hq, hkv, L, d = 6, 2, 8, 4
    q = _rand(rng, 2, hq, L, d)
    k = _rand(rng, 2, hkv, L, d) + np.arange(hkv)[None, :, None, None]
    v = _rand(rng, 2, hkv, L, d) + 3.0 * np.arange(hkv)[None, :, None, None]
    do = _rand(rng, 2, hq, L, d)
    pos = np.tile(np.arange(L), (2, 1))
    kvl = np.array([L, L])
    dq, dk, dv = O.grouped_attention_backward(q, k, v, pos, kvl, 0.5, True, do)
    grp = hq // hkv
    rq, rk, rv = O.grouped_attention_backward(q, np.repeat(k, grp, axis=1),
                                              np.repeat(v, grp, axis=1), pos, kvl, 0.5,
                                              True, do)
    assert np.max(np.abs(dq - rq)) < 1e-12
    assert np.max(np.abs(dk - rk.reshape(2, hkv, grp, L, d).sum(2))) < 1e-12
    assert np.max(np.abs(dv - rv.reshape(2, hkv, grp, L, d).sum(2))) < 1e-12
    # under the causal mask the last key gets gradient only from the last query
    only_last = do.copy()
    only_last[:, :, :-1] = 0.0
    _, _, dv_last = O.grouped_attention_backward(q, k, v, pos, kvl, 0.5, True, only_last)
    do0 = do.copy()
    do0[:, :, -1] = 0.0
    _, dk0, dv0 = O.grouped_attention_backward(q, k, v, pos, kvl, 0.5, True, do0)
    assert np.max(np.abs(dv0[:, :, -1])) < 1e-15 and np.max(np.abs(dk0[:, :, -1])) < 1e-15
    assert np.max(np.abs(dv_last[:, :, -1])) > 1e-3


def check_norm_rope_backward_invariants():
    """RMSNorm with eps = 0 is invariant to scaling its input, so its input
    gradient is orthogonal to the input row; RoPE is a rotation, so its
    backward inverts it and keeps norms."""
    rng = np.random.default_rng(26)
    v = _rand(rng, 2, 3, 4, 16, scale=2.0)
    w = 1.0 + _rand(rng, 16, scale=0.2)
    dy = _rand(rng, 2, 3, 4, 16)
    dv, dw = O.rms_norm_heads_backward(v, w, 0.0, dy)
    assert np.max(np.abs(np.sum(dv * v, axis=-1))) < 1e-12
    # the weight gradient is the upstream gradient times the normalised input
    unit = O.rms_norm_heads(v, np.ones(16), 0.0)
    assert np.max(np.abs(dw - np.sum((dy * unit).reshape(-1, 16), axis=0))) < 1e-12
    pos = np.array([[0, 3, 40000], [1, 5, 65535]])
    u = _rand(rng, 2, 3, 4, 16)
    for rot in (None, 8):
        back = O.apply_rope_backward(O.apply_rope(u, pos, 1e4, rotary_dim=rot), pos, 1e4,
                                     rotary_dim=rot)
        assert np.max(np.abs(back - u)) < 1e-12
        gb = O.apply_rope_backward(u, pos, 1e4, rotary_dim=rot)
        assert np.max(np.abs(np.linalg.norm(gb, axis=-1) - np.linalg.norm(u, axis=-1))) < 1e-12


ALL_CHECKS = [
    check_geometries, check_resolve_errors, check_param_counts, check_macs,
    check_projection_bruteforce, check_attention_bruteforce,
    check_attention_vs_torch_sdpa, check_layer_mha_reduces_to_torch_mha,
    check_layer_vs_torch_composition, check_rmsnorm, check_rope, check_partial_rope,
    check_position_shift_invariance, check_causality,
    check_gqa_equals_repeated_kv, check_rank_ceiling, check_one_dim_head,
    check_sum_over_heads, check_prefill_equals_decode,
    check_quotient_equals_explicit, check_rows_mode,
    check_e4m3_closed_forms, check_e4m3_quantize_bruteforce, check_fp8_cache_layer,
    check_layer_backward_finite_differences, check_layer_backward_vs_torch_autograd,
    check_attention_backward_group_sum, check_norm_rope_backward_invariants,
]
