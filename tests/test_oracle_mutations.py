"""Plant plausible mistakes in the CPU oracle and show that at least one pin
fails for each.  Every mistake is planted in the oracle, on the CPU, through
pytest's monkeypatch (undone after each case)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle_pins as P  # noqa: E402
from oracle import gqa_oracle as O  # noqa: E402

_orig = {name: getattr(O, name) for name in (
    "resolve_config", "attention_param_count", "macs_per_token", "project",
    "split_heads", "rms_norm_heads", "rope_inv_freq", "apply_rope",
    "grouped_attention", "merge_heads", "qkv_normrope", "e4m3_value", "quantize_e4m3",
    "weight_blocks", "project_heads_out",
    "project_backward", "rms_norm_heads_backward", "apply_rope_backward",
    "grouped_attention_backward")}


def _k_norm_uses_q_weight(res, x, w_qkv, qn, kn, positions, theta, eps,
                          qk_norm=True, rope=True, rotary_dim=None):
    return _orig["qkv_normrope"](res, x, w_qkv, qn, qn, positions, theta, eps,
                                 qk_norm=qk_norm, rope=rope, rotary_dim=rotary_dim)


def _attention_with(group_map=None, scale_fn=None, causal_shift=0,
                    normalize=True, softmax_axis=-1):
    def attn(q, k, v, q_pos, kv_len, scale, causal=True):
        bsz, hq, lq, d = q.shape
        hkv = k.shape[1]
        group = hq // hkv
        out = np.zeros((bsz, hq, lq, v.shape[-1]), dtype=q.dtype)
        sc = scale if scale_fn is None else scale_fn(d)
        for b in range(bsz):
            n = int(kv_len[b])
            vis = np.arange(n)[None, :] <= (q_pos[b][:, None] + causal_shift)
            if not causal:
                vis = np.ones_like(vis)
            for h in range(hq):
                g = h // group if group_map is None else group_map(h, hkv, group)
                s = q[b, h] @ k[b, g, :n].T * sc
                s = np.where(vis, s, -np.inf)
                m = np.max(s, axis=-1, keepdims=True)
                p = np.exp(s - m)
                if normalize:
                    p = p / np.sum(p, axis=softmax_axis, keepdims=True)
                p = np.nan_to_num(p)
                out[b, h] = p @ v[b, g, :n]
        return out
    return attn


def _rope_with(sign=1.0, interleaved=False, freq_factor=2.0, freq_over_head_dim=False):
    def rope(v, positions, theta, rotary_dim=None):
        d = v.shape[-1]
        r = d if rotary_dim is None else rotary_dim
        half = r // 2
        i = np.arange(half, dtype=np.float64)
        ang = positions.astype(np.float64)[..., None] * \
            np.power(np.float64(theta), -freq_factor * i / (d if freq_over_head_dim else r)) * sign
        cos = np.cos(ang)[:, :, None, :]
        sin = np.sin(ang)[:, :, None, :]
        if interleaved:
            x1, x2 = v[..., 0:r:2], v[..., 1:r:2]
            y = v.copy()
            y[..., 0:r:2] = x1 * cos - x2 * sin
            y[..., 1:r:2] = x2 * cos + x1 * sin
            return y
        x1, x2 = v[..., :half], v[..., half:r]
        return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin, v[..., r:]], -1)
    return rope


def _split_kv_swapped(y, res):
    q, k, v = _orig["split_heads"](y, res)
    if k.shape == v.shape:
        return q, v, k
    return q, k, v


def _blocks_k_v_swapped(w_qkv, res):
    """The fused weight's K and V row blocks taken in the wrong order."""
    wq, wk, wv = _orig["weight_blocks"](w_qkv, res)
    return wq, wv, wk


def _heads_out_slices_shifted(o, w_o):
    """Head h multiplied by the W_o columns of head h + 1 (cyclically)."""
    d, hq = o.shape[-1], o.shape[1]
    w = np.concatenate([w_o[:, d:], w_o[:, :d]], axis=1) if hq > 1 else w_o
    return _orig["project_heads_out"](o, w)


def _resolve_always_quotient(hidden_size, num_heads, num_kv_heads=None,
                             head_dim=None, require_even=True):
    return _orig["resolve_config"](hidden_size, num_heads, num_kv_heads,
                                   None if hidden_size % num_heads == 0 else head_dim,
                                   require_even)


def _params_without_o_proj(res):
    s = O.weight_shapes(res)
    return sum(a * b for k, (a, b) in s.items()
               if k not in ("query_key_value", "o_proj"))


def _macs_score_only(res, n):
    m = _orig["macs_per_token"](res, n)
    return {"projection": m["projection"], "score_value": m["score_value"] // 2}


def _e4m3_value_bias8(codes):
    """FNUZ-style reading of the codes (bias 8): every value halved."""
    return _orig["e4m3_value"](codes) / 2.0


def _quantize_half_up(x):
    """Rounds halves away from zero instead of to even."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    e = np.clip(np.floor(np.log2(np.where(a > 0, a, 1.0))) + 7.0, 1.0, 15.0)
    q = np.exp2(e - 10.0)
    y = np.sign(x) * np.floor(a / q + 0.5) * q
    return _orig["quantize_e4m3"](y)


def _quantize_no_saturation(x):
    """Values above 448 become NaN codes instead of saturating."""
    x = np.asarray(x, dtype=np.float64)
    c = _orig["quantize_e4m3"](x)
    return np.where(np.abs(x) > 464.0, np.where(x < 0, 0xFF, 0x7F), c).astype(np.uint8)


def _norm_bwd_without_mean_term(v, w, eps, dy):
    """Treats r as a constant: drops the term through mean(v*v)."""
    dv, dw = _orig["rms_norm_heads_backward"](v, w, eps, dy)
    r = 1.0 / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    return r * w * dy, dw


def _rope_bwd_forward_rotation(g, positions, theta, rotary_dim=None):
    """Carries the gradient back through the forward rotation, not its
    transpose."""
    return _orig["apply_rope"](g, positions, theta, rotary_dim=rotary_dim)


def _attn_bwd_with(last_head_only=False, no_centering=False, dk_unscaled=False):
    def bwd(q, k, v, q_pos, kv_len, scale, causal, do):
        bsz, hq, lq, d = q.shape
        hkv = k.shape[1]
        group = hq // hkv
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(bsz):
            n = int(kv_len[b])
            vis = np.arange(n)[None, :] <= q_pos[b][:, None] if causal else \
                np.ones((lq, n), dtype=bool)
            for h in range(hq):
                g = h // group
                s = np.where(vis, q[b, h] @ k[b, g, :n].T * scale, -np.inf)
                p = np.exp(s - s.max(-1, keepdims=True))
                p /= p.sum(-1, keepdims=True)
                dp = do[b, h] @ v[b, g, :n].T
                ds = p * dp if no_centering else p * (dp - np.sum(p * dp, -1, keepdims=True))
                dq[b, h] = ds @ k[b, g, :n] * scale
                cdk = ds.T @ q[b, h] * (1.0 if dk_unscaled else scale)
                cdv = p.T @ do[b, h]
                if last_head_only:
                    dk[b, g, :n], dv[b, g, :n] = cdk, cdv
                else:
                    dk[b, g, :n] += cdk
                    dv[b, g, :n] += cdv
        return dq, dk, dv
    return bwd


def _proj_bwd_first_sequence_only(x, w, dy):
    """Weight gradient summed over the first sequence's tokens only."""
    dx, _ = _orig["project_backward"](x, w, dy)
    return dx, dy[0].reshape(-1, dy.shape[-1]).T @ x[0].reshape(-1, x.shape[-1])


MUTATIONS = {
    "norm_bwd_drops_mean_term": ("rms_norm_heads_backward", _norm_bwd_without_mean_term),
    "rope_bwd_forward_rotation": ("apply_rope_backward", _rope_bwd_forward_rotation),
    "attn_bwd_kv_grad_last_head_only": ("grouped_attention_backward",
                                        _attn_bwd_with(last_head_only=True)),
    "attn_bwd_softmax_not_centred": ("grouped_attention_backward",
                                     _attn_bwd_with(no_centering=True)),
    "attn_bwd_dk_unscaled": ("grouped_attention_backward", _attn_bwd_with(dk_unscaled=True)),
    "proj_bwd_first_sequence_only": ("project_backward", _proj_bwd_first_sequence_only),
    "k_norm_with_q_weight": ("qkv_normrope", _k_norm_uses_q_weight),
    "group_map_modulo": ("grouped_attention",
                         _attention_with(group_map=lambda h, hkv, g: h % hkv)),
    "scale_one_over_d": ("grouped_attention",
                         _attention_with(scale_fn=lambda d: 1.0 / d)),
    "causal_sees_next_token": ("grouped_attention",
                               _attention_with(causal_shift=1)),
    "softmax_not_normalised": ("grouped_attention",
                               _attention_with(normalize=False)),
    "softmax_over_queries": ("grouped_attention",
                             _attention_with(softmax_axis=0)),
    "rope_sign_flipped": ("apply_rope", _rope_with(sign=-1.0)),
    "rope_interleaved_pairs": ("apply_rope", _rope_with(interleaved=True)),
    "rope_freq_dropped_factor_2": ("apply_rope", _rope_with(freq_factor=1.0)),
    "partial_rope_freq_over_head_dim": ("apply_rope", _rope_with(freq_over_head_dim=True)),
    "rmsnorm_eps_outside_sqrt": (
        "rms_norm_heads",
        lambda v, w, eps: v / (np.sqrt(np.mean(v * v, -1, keepdims=True)) + eps) * w),
    "rmsnorm_over_heads": (
        "rms_norm_heads",
        lambda v, w, eps: v / np.sqrt(np.mean(v * v, axis=(-2, -1), keepdims=True)
                                      + eps) * w),
    "flatten_without_transpose": (
        "merge_heads", lambda o: o.reshape(o.shape[0], o.shape[2], -1)),
    "k_v_swapped": ("split_heads", _split_kv_swapped),
    "k_v_weight_blocks_swapped": ("weight_blocks", _blocks_k_v_swapped),
    "o_proj_head_slices_shifted": ("project_heads_out", _heads_out_slices_shifted),
    "projection_transposed_operand": (
        "project", lambda x, w: np.matmul(x, w.T) if w.shape[0] != w.shape[1]
        else np.matmul(x, w)),
    "head_dim_always_derived": ("resolve_config", _resolve_always_quotient),
    "params_miss_o_proj": ("attention_param_count", _params_without_o_proj),
    "macs_miss_value_term": ("macs_per_token", _macs_score_only),
    "e4m3_bias_8": ("e4m3_value", _e4m3_value_bias8),
    "e4m3_ties_away_from_zero": ("quantize_e4m3", _quantize_half_up),
    "e4m3_no_saturation": ("quantize_e4m3", _quantize_no_saturation),
}


def _run_all_checks():
    failed = []
    for chk in P.ALL_CHECKS:
        try:
            chk()
        except KeyError:  # a broken mutation, not a caught mistake
            raise
        except Exception as e:  # AssertionError, or a crash from bad shapes
            failed.append((chk.__name__, type(e).__name__))
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = _run_all_checks()
    assert failed, f"no pin caught the planted mistake {name}"


def test_unmutated_oracle_passes_all_pins():
    assert _run_all_checks() == []
