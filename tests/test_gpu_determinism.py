"""Race detection by repetition: each path run twice on the same inputs must
give bitwise identical results.  A kernel that reads LDS before every wave
has written it, or sums in an order that depends on timing, shows up as a
difference between two runs.  Covers the split-KV decode (bf16 and FP8
caches) with its merge of the splits' partial results, the few-token
projections with their K split over workgroups and its summing pass, and
the prefill attention core."""
import dataclasses
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gqa_inputs as GI  # noqa: E402
from gpu_util import announce, cfg_of  # noqa: E402
from oracle import gqa_oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_attention_layer_amd as T
    T.lib()
    yield


def T_():
    import transformer_attention_layer_amd as T
    return T


def _decode_twice(w, kv_fp8=False):
    T = T_()
    h = GI.host_layer_inputs(w)
    d = GI.to_device(h, w)
    cache = GI.host_cache(w, fill_unused=0.0)
    if kv_fp8:
        c = {k: torch.from_numpy(O.quantize_e4m3(v)).cuda() for k, v in cache.items()}
    else:
        c = GI.to_device(cache, w)
    cl = torch.full((w.batch,), w.cache_len, dtype=torch.int32, device="cuda")
    cfg = cfg_of(w)
    if kv_fp8:
        cfg = dataclasses.replace(cfg, kv_fp8=True)
    outs = []
    for _ in range(2):
        # the append rewrites the same rows each time
        out, _, _ = T.gqa_layer_forward(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"],
                                        d["w_o"], k_cache=c["k_cache"], v_cache=c["v_cache"],
                                        cache_len=cl)
        outs.append(out.clone())
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("name,w", [
    ("gqa_5_splits", GI.WORKLOADS["decode_h2560_gqa"].with_(batch=2, cache_len=5000)),
    ("mqa_69_splits", GI.WORKLOADS["decode_h2560_mqa"].with_(batch=1, cache_len=70000)),
    ("gqa_8seq_8k", GI.WORKLOADS["decode_h2560_gqa"].with_(batch=8, cache_len=8191)),
    ("gqa_q4", GI.WORKLOADS["decode_h2560_gqa"].with_(batch=3, seq=4, cache_len=3000)),
    ("gqa_rotated_d64", GI.WORKLOADS["decode_h2560_gqa"].with_(batch=96, cache_len=3500, hq=8,
                                                               hkv=4, head_dim=64)),
])
def test_decode_repeat_bitwise(name, w):
    announce(f"[repeat] decode {name}")
    a, b = _decode_twice(w)
    assert torch.equal(a, b)


@pytest.mark.parametrize("name,w", [
    ("gqa_fp8", GI.WORKLOADS["decode_h2560_gqa_fp8"].with_(batch=4, cache_len=6000)),
    ("mqa_fp8", GI.WORKLOADS["decode_h2560_mqa_fp8"].with_(batch=2, cache_len=20000)),
])
def test_fp8_decode_repeat_bitwise(name, w):
    announce(f"[repeat] fp8 decode {name}")
    a, b = _decode_twice(w.with_(kv_fp8=False), kv_fp8=True)
    assert torch.equal(a, b)


@pytest.mark.parametrize("tokens", [17, 64, 200])
def test_few_token_projections_repeat_bitwise(tokens):
    """qkv_proj_normrope and gqa_layer_forward on few tokens (the
    weight-streaming GEMMs, K split over workgroups for narrow outputs)."""
    T = T_()
    for base, kw in (("prefill_h1024", {"o_split": True}), ("wide_h5120", {"hq": 40, "hkv": 8})):
        w = GI.WORKLOADS[base].with_(batch=1, seq=tokens, **kw)
        announce(f"[repeat] few tokens {base} {kw} T={tokens}")
        d = GI.to_device(GI.host_layer_inputs(w), w)
        cfg = cfg_of(w)
        q1, k1, v1 = T.qkv_proj_normrope(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"])
        q2, k2, v2 = T.qkv_proj_normrope(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"])
        o1, _, _ = T.gqa_layer_forward(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"],
                                       d["w_o"])
        o2, _, _ = T.gqa_layer_forward(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"],
                                       d["w_o"])
        torch.cuda.synchronize()
        assert torch.equal(q1, q2) and torch.equal(k1, k2) and torch.equal(v1, v2)
        assert torch.equal(o1, o2)


@pytest.mark.parametrize("hq,hkv", [(16, 8), (16, 2), (32, 1)])
def test_prefill_attention_repeat_bitwise(hq, hkv):
    """gqa_attn_core on random q, k, v: several query tiles, a ragged tail,
    GQA groups 2, 8 and 32."""
    T = T_()
    w = GI.WORKLOADS["prefill_h1024"].with_(batch=2, seq=333, hq=hq, hkv=hkv)
    announce(f"[repeat] prefill attention {hq}/{hkv}")
    rng = np.random.default_rng(5)
    q = GI.round_bf16(rng.standard_normal((2, hq, 333, 128), dtype=np.float32))
    k = GI.round_bf16(rng.standard_normal((2, hkv, 333, 128), dtype=np.float32))
    v = GI.round_bf16(rng.standard_normal((2, hkv, 333, 128), dtype=np.float32))
    d = GI.to_device({"q": q, "k": k, "v": v}, w)
    cfg = cfg_of(w)
    a = T.gqa_attn_core(cfg, d["q"], d["k"], d["v"])
    b = T.gqa_attn_core(cfg, d["q"], d["k"], d["v"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
