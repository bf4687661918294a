"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, element by element, at sizes the oracle finishes in
seconds; every case spans several tiles and a ragged tail."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gqa_inputs as GI  # noqa: E402
from gpu_util import (announce, assert_close, cfg_of, oracle_layer, resolved,  # noqa: E402
                      to_np)
from oracle import gqa_oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_attention_layer_amd as T
    T.lib()  # fail loudly if the library is missing
    yield


def T_():
    import transformer_attention_layer_amd as T
    return T


# reduced-size versions of every workload (same model shapes, shorter runs)
SMALL = {
    "tiny_f32": GI.WORKLOADS["tiny_f32"],
    "prefill_h1024": GI.WORKLOADS["prefill_h1024"].with_(batch=2, seq=200),
    "quotient_h4096": GI.WORKLOADS["quotient_h4096"].with_(batch=1, seq=300),
    "wide_h5120": GI.WORKLOADS["wide_h5120"].with_(batch=1, seq=260),
    "decode_h2560_gqa": GI.WORKLOADS["decode_h2560_gqa"].with_(batch=3, cache_len=1000),
    "decode_h2560_mqa": GI.WORKLOADS["decode_h2560_mqa"].with_(batch=2, cache_len=777),
    # key splits merged by the decode combine: 5 (an odd count, so the
    # combine's lane groups take different numbers of splits) and 69 (more
    # than one 64-split chunk of weights)
    "decode_gqa_5_splits": GI.WORKLOADS["decode_h2560_gqa"].with_(batch=2, cache_len=5000),
    "decode_mqa_69_splits": GI.WORKLOADS["decode_h2560_mqa"].with_(batch=1, cache_len=70000),
    # bf16 head sizes other than 128 (separate norm/RoPE pass, vector-unit attention)
    "bf16_d64": GI.WORKLOADS["prefill_h1024"].with_(batch=2, seq=150, hq=8, hkv=2, head_dim=64),
    "bf16_d256": GI.WORKLOADS["prefill_h1024"].with_(batch=1, seq=130, hq=4, hkv=2, head_dim=256),
    "bf16_d80_quotient": GI.WORKLOADS["quotient_h4096"].with_(batch=1, seq=90, hidden=640, hq=8,
                                                             hkv=4, o_fp16=False, o_split=True),
    "bf16_d64_decode": GI.WORKLOADS["decode_h2560_gqa"].with_(batch=2, cache_len=300, hq=8, hkv=4,
                                                              head_dim=64),
    # more decode waves than the GPU holds at once (384 streams x 4 splits of
    # 896 keys, the last one ragged): each wave starts its chunk at its own
    # tile and wraps round, so partial tiles fall mid-walk
    "decode_rotated_d64": GI.WORKLOADS["decode_h2560_gqa"].with_(batch=96, cache_len=3500, hq=8,
                                                                 hkv=4, head_dim=64),
    # ... with 4 new tokens per sequence, so causally masked keys sit in
    # tiles that the rotated walks reach mid-way
    "decode_rotated_q4_d64": GI.WORKLOADS["decode_h2560_gqa"].with_(batch=96, seq=4, cache_len=3500,
                                                                    hq=8, hkv=4, head_dim=64),
    # head_dim 256 through the split-KV decode kernel (one wave per SIMD),
    # a Gemma-shaped group of 4 query heads per KV head
    "bf16_d256_decode": GI.WORKLOADS["gemma_h640_d256"].with_(batch=3, seq=1, cache_len=1500),
    # MQA with 2 new tokens: 32 heads x 2 rows pass one wave's 32, so the
    # prefill kernel runs over the cache (bottom-right causal alignment)
    "mqa_two_tokens": GI.WORKLOADS["decode_h2560_mqa"].with_(batch=2, seq=2, cache_len=900),
    # the QKV projection's own norm/RoPE epilogue for head_dim 64 and 256
    # (more than 256 tokens): 256 with and without a cache to continue,
    # 64 with rotary 32 and with an odd head count (the last wave of
    # features holds one head)
    "bf16_d256_fused": GI.WORKLOADS["prefill_h1024"].with_(batch=2, seq=150, hq=4, hkv=2,
                                                           head_dim=256),
    "gemma_d256_chunk": GI.WORKLOADS["gemma_h640_d256"].with_(batch=2, seq=200, cache_len=100),
    "rot32_of_64_fused": GI.WORKLOADS["prefill_h1024"].with_(batch=2, seq=150, hq=8, hkv=2,
                                                             head_dim=64, rotary_dim=32),
    "bf16_d64_odd_heads": GI.WORKLOADS["prefill_h1024"].with_(batch=1, seq=300, hq=3, hkv=1,
                                                              head_dim=64),
    # partial rotary: 64 of 128 in the fused epilogue, 48 of 128 through the
    # separate norm/RoPE pass, 32 of 64 on the fallback path, 64 of 128 decode
    "rot64_of_128": GI.WORKLOADS["prefill_h1024"].with_(batch=2, seq=170, rotary_dim=64),
    "rot48_of_128": GI.WORKLOADS["prefill_h1024"].with_(batch=1, seq=140, rotary_dim=48),
    "rot32_of_64": GI.WORKLOADS["prefill_h1024"].with_(batch=1, seq=90, hq=8, hkv=2, head_dim=64,
                                                       rotary_dim=32),
    "rot64_decode": GI.WORKLOADS["decode_h2560_gqa"].with_(batch=2, cache_len=500, rotary_dim=64),
    # the fp16 carrier of the attention output on every attention kernel:
    # prefill, the decode merge (the decode workloads), the vector-unit path
    "o_fp16_d256": GI.WORKLOADS["prefill_h1024"].with_(batch=1, seq=130, hq=4, hkv=2,
                                                       head_dim=256, o_fp16=True),
    "o_fp16_d80": GI.WORKLOADS["quotient_h4096"].with_(batch=1, seq=90, hidden=640, hq=8, hkv=4),
    # the bf16 hi + lo carrier on the prefill path (o_proj reads W_o twice along K)
    "o_split_prefill": GI.WORKLOADS["wide_h5120"].with_(batch=1, seq=260, o_fp16=False,
                                                        o_split=True),
    # ... and on the decode path (few-token o_proj over [hi | lo]); the
    # decode workloads themselves carry o as fp16, with W_o rounded to fp16
    # inside the few-token product
    "o_split_decode": GI.WORKLOADS["decode_h2560_gqa"].with_(batch=3, cache_len=1000,
                                                             o_split=True, o_fp16=False),
    "o_split_mqa_decode": GI.WORKLOADS["decode_h2560_mqa"].with_(batch=2, cache_len=777,
                                                                 o_split=True, o_fp16=False),
}


def run_layer(w, h, cache=None, cache_len=None, out_f32=True):
    T = T_()
    d = GI.to_device(h, w)
    kw = {}
    if cache is not None:
        c = GI.to_device(cache, w)
        kw = dict(k_cache=c["k_cache"], v_cache=c["v_cache"],
                  cache_len=torch.tensor(cache_len, dtype=torch.int32, device="cuda"))
    out, kc, vc = T.gqa_layer_forward(cfg_of(w, out_f32), d["x"], d["w_qkv"], d["q_norm_w"],
                                      d["k_norm_w"], d["w_o"], **kw)
    torch.cuda.synchronize()
    return out, kc, vc


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_forward_parity(name):
    w = SMALL[name]
    announce(f"[layer] {name} B={w.batch} L={w.seq} cache={w.cache_len}")
    h = GI.host_layer_inputs(w)
    if w.cache_len:
        cache = GI.host_cache(w)
        cl = np.full(w.batch, w.cache_len, dtype=np.int64)
        out, kc, vc = run_layer(w, h, cache, cl)
        ref, rk, rv = oracle_layer(w, h, cache, cl)
        # the appended row of the cache
        n = w.cache_len
        assert_close(to_np(kc)[:, :, n:n + w.seq], rk[:, :, n:n + w.seq], w.dtype, "k append")
        assert_close(to_np(vc)[:, :, n:n + w.seq], rv[:, :, n:n + w.seq], w.dtype, "v append")
        # rows below are untouched
        assert np.array_equal(to_np(kc)[:, :, :n], cache["k_cache"][:, :, :n])
    else:
        out, kc, vc = run_layer(w, h)
        ref, _, _ = oracle_layer(w, h)
    assert_close(to_np(out), ref, w.dtype, "out")


@pytest.mark.parametrize("name", ["tiny_f32", "prefill_h1024", "quotient_h4096"])
def test_entry_points_parity(name):
    """qkv_proj_normrope, gqa_attn_core and gqa_o_proj separately."""
    T = T_()
    w = SMALL[name]
    announce(f"[entry points] {name}")
    res = resolved(w)
    h = GI.host_layer_inputs(w)
    d = GI.to_device(h, w)
    cfg = cfg_of(w)
    q, kc, vc = T.qkv_proj_normrope(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"])
    pos = np.tile(np.arange(w.seq), (w.batch, 1))
    rq, rk, rv = O.qkv_normrope(res, h["x"].astype(np.float64), h["w_qkv"].astype(np.float64),
                                h["q_norm_w"].astype(np.float64),
                                h["k_norm_w"].astype(np.float64), pos, w.rope_theta, w.rms_eps,
                                qk_norm=w.qk_norm)
    assert_close(to_np(q), rq, w.dtype, "q")
    assert_close(to_np(kc), rk, w.dtype, "k")
    assert_close(to_np(vc), rv, w.dtype, "v")
    # attention core on the oracle's own q, k, v (rounded to the storage type)
    qh = GI.round_bf16(rq.astype(np.float32)) if w.dtype == "bf16" else rq.astype(np.float32)
    kh = GI.round_bf16(rk.astype(np.float32)) if w.dtype == "bf16" else rk.astype(np.float32)
    vh = GI.round_bf16(rv.astype(np.float32)) if w.dtype == "bf16" else rv.astype(np.float32)
    dd = GI.to_device({"q": qh, "k": kh, "v": vh}, w)
    o = T.gqa_attn_core(cfg, dd["q"], dd["k"], dd["v"])
    ro = O.merge_heads(O.grouped_attention(qh.astype(np.float64), kh.astype(np.float64),
                                           vh.astype(np.float64), pos,
                                           np.full(w.batch, w.seq), res.scale, w.causal))
    assert_close(to_np(o), ro, w.dtype, "attention")
    # o_proj on an oracle-side activation
    oh = GI.round_bf16(ro.astype(np.float32)) if w.dtype == "bf16" else ro.astype(np.float32)
    out = T.gqa_o_proj(cfg, GI.to_device({"o": oh}, w)["o"], d["w_o"])
    assert_close(to_np(out), O.project(oh.astype(np.float64), h["w_o"].astype(np.float64)),
                 w.dtype, "o_proj")


@pytest.mark.parametrize("causal", [True, False])
def test_attention_rescales_in_later_tiles(causal):
    """Scores that grow by 0.3 log2 units per key (about 10 per 32-key
    tile) and one late key 40 units above the ramp: each row's running max
    passes the lazy-rescale threshold in most of its tiles, not only the
    first, and the spike forces one large rescale late in the row.  The
    attention core against the oracle on the same rounded q, k, v."""
    T = T_()
    w = GI.WORKLOADS["prefill_h1024"].with_(batch=2, seq=300, causal=causal)
    announce(f"[rescale ramp] causal={causal}")
    res = resolved(w)
    a = GI.host_ramp_attention(w)
    d = GI.to_device(a, w)
    o = T.gqa_attn_core(cfg_of(w), d["q"], d["k"], d["v"])
    pos = np.tile(np.arange(w.seq), (w.batch, 1))
    ro = O.merge_heads(O.grouped_attention(a["q"].astype(np.float64), a["k"].astype(np.float64),
                                           a["v"].astype(np.float64), pos,
                                           np.full(w.batch, w.seq), res.scale, causal))
    assert_close(to_np(o), ro, w.dtype, "attention")


@pytest.mark.parametrize("variant", [
    dict(hq=16, hkv=16),            # plain MHA (group 1)
    dict(hq=12, hkv=4),             # group 3
    dict(hq=16, hkv=2),             # group 8 -> two workgroups per KV group
    dict(hq=16, hkv=8, causal=False),
    dict(hq=8, hkv=8, qk_norm=False, seq=67),
])
def test_prefill_variants(variant):
    seq = variant.pop("seq", 150)
    w = GI.WORKLOADS["prefill_h1024"].with_(batch=2, seq=seq, **variant)
    announce(f"[variant] {variant} seq={seq}")
    h = GI.host_layer_inputs(w)
    out, _, _ = run_layer(w, h)
    ref, _, _ = oracle_layer(w, h)
    assert_close(to_np(out), ref, w.dtype, "out")


@pytest.mark.parametrize("tokens", [1, 17, 64, 65, 200, 256])
def test_few_token_projection_path(tokens):
    """Up to 256 tokens take the weight-streaming projections (K split over
    workgroups, 64-feature blocks streamed through LDS when K is a multiple
    of 64, else 32-feature tiles) and a separate norm + RoPE pass; ragged
    token and feature counts, with and without QK-norm and the hi+lo split
    (also with a 1024-wide o_proj)."""
    for base, kw in (("prefill_h1024", {}), ("wide_h5120", {"hq": 40, "hkv": 8}),
                     ("quotient_h4096", {}), ("prefill_h1024", {"o_split": True}),
                     ("quotient_h4096", {"o_fp16": False, "o_split": True})):
        w = GI.WORKLOADS[base].with_(batch=1, seq=tokens, **kw)
        announce(f"[few tokens] {base} {kw} T={tokens} o_split={w.o_split}")
        h = GI.host_layer_inputs(w)
        out, _, _ = run_layer(w, h)
        ref, _, _ = oracle_layer(w, h)
        assert_close(to_np(out), ref, w.dtype, "out")


def test_chunked_prefill_with_ragged_cache():
    """A chunk of new tokens appended to caches of different lengths per
    sequence (bottom-right causal alignment)."""
    w = GI.WORKLOADS["prefill_h1024"].with_(batch=3, seq=70, cache_len=300)
    announce("[chunked prefill] ragged cache lengths")
    h = GI.host_layer_inputs(w)
    cache = GI.host_cache(w)
    cl = np.array([300, 0, 123], dtype=np.int64)
    for b, n in enumerate(cl):
        cache["k_cache"][b, :, n:] = np.nan
        cache["v_cache"][b, :, n:] = np.nan
    out, kc, vc = run_layer(w, h, cache, cl)
    ref, rk, _ = oracle_layer(w, h, cache, cl)
    assert_close(to_np(out), ref, w.dtype, "out")


@pytest.mark.parametrize("seq,cache_lens", [
    (100, [300, 0, 123]),
    (17, [(37 * b) % 200 for b in range(20)]),
    (17, None),
])
def test_fused_epilogue_rows(seq, cache_lens):
    """More than 256 tokens take the persistent GEMM with the head_dim-128
    norm/RoPE/scatter epilogue, which stores 32-token chunks: with L >= 32 a
    chunk spans at most two sequences (two cache bases, whose offsets differ
    here), with L < 32 its rows are placed one by one; with and without
    caches to continue."""
    batch = 20 if cache_lens is None else len(cache_lens)
    cap = 0 if cache_lens is None else max(cache_lens)
    w = GI.WORKLOADS["prefill_h1024"].with_(batch=batch, seq=seq, cache_len=cap)
    announce(f"[fused epilogue rows] B={batch} L={seq} caches={cache_lens}")
    h = GI.host_layer_inputs(w)
    if cache_lens is None:
        out, _, _ = run_layer(w, h)
        ref, _, _ = oracle_layer(w, h)
    else:
        cache = GI.host_cache(w)
        cl = np.array(cache_lens, dtype=np.int64)
        for b, n in enumerate(cl):
            cache["k_cache"][b, :, n:] = np.nan
            cache["v_cache"][b, :, n:] = np.nan
        out, kc, vc = run_layer(w, h, cache, cl)
        ref, rk, rv = oracle_layer(w, h, cache, cl)
        kc, vc = to_np(kc), to_np(vc)
        for b, n in enumerate(cl):
            assert_close(kc[b, :, n:n + seq], rk[b, :, n:n + seq], w.dtype, f"k append {b}")
            assert_close(vc[b, :, n:n + seq], rv[b, :, n:n + seq], w.dtype, f"v append {b}")
            assert np.array_equal(kc[b, :, :n], cache["k_cache"][b, :, :n])
    assert_close(to_np(out), ref, w.dtype, "out")


@pytest.mark.parametrize("q_len", [2, 4, 8])
def test_multi_token_decode(q_len):
    """A few new tokens per sequence (group * q_len <= 32 takes the split-KV
    kernel)."""
    w = GI.WORKLOADS["decode_h2560_gqa"].with_(batch=2, seq=q_len, cache_len=531)
    announce(f"[multi-token decode] q_len={q_len}")
    h = GI.host_layer_inputs(w)
    cache = GI.host_cache(w)
    cl = np.array([531, 200], dtype=np.int64)
    cache["k_cache"][1, :, 200:] = np.nan
    cache["v_cache"][1, :, 200:] = np.nan
    out, _, _ = run_layer(w, h, cache, cl)
    ref, _, _ = oracle_layer(w, h, cache, cl)
    assert_close(to_np(out), ref, w.dtype, "out")


def test_future_tokens_do_not_leak():
    """Changing x at t' leaves rows t < t' bitwise unchanged on the GPU
    (distinguishable heads, nontrivial length)."""
    w = GI.WORKLOADS["prefill_h1024"].with_(batch=1, seq=190)
    announce("[causality] future-token perturbation")
    h = GI.host_layer_inputs(w)
    base, _, _ = run_layer(w, h)
    for tp in (64, 131, 189):
        h2 = dict(h)
        x2 = h["x"].copy()
        x2[:, tp] += 3.0
        h2["x"] = GI.round_bf16(x2)
        pert, _, _ = run_layer(w, h2)
        a, b = to_np(base), to_np(pert)
        assert np.array_equal(a[:, :tp], b[:, :tp]), tp
        assert not np.array_equal(a[:, tp], b[:, tp])


@pytest.mark.parametrize("name", ["prefill_h1024", "decode_h2560_gqa"])
def test_bf16_output_is_rounded_fp32_output(name):
    """With out_f32 off the o_proj output is the fp32 accumulator rounded to
    bf16 (nearest even), bit for bit."""
    w = SMALL[name]
    h = GI.host_layer_inputs(w)
    cache, cl = None, None
    if w.cache_len:
        cache = GI.host_cache(w)
        cl = np.full(w.batch, w.cache_len, dtype=np.int64)
    a, _, _ = run_layer(w, h, cache, cl, out_f32=True)
    b, _, _ = run_layer(w, h, cache, cl, out_f32=False)
    assert b.dtype == torch.bfloat16 and a.dtype == torch.float32
    assert torch.equal(a.to(torch.bfloat16), b)


def test_deterministic():
    w = SMALL["prefill_h1024"]
    h = GI.host_layer_inputs(w)
    a, _, _ = run_layer(w, h)
    b, _, _ = run_layer(w, h)
    assert torch.equal(a, b)


def test_quotient_equals_explicit_head_dim():
    """head_dim unset resolves to hidden/Hq and gives bitwise the same
    output as that head_dim set explicitly."""
    w0 = SMALL["quotient_h4096"]
    w1 = w0.with_(head_dim=128)
    h = GI.host_layer_inputs(w0)
    a, _, _ = run_layer(w0, h)
    b, _, _ = run_layer(w1, h)
    assert torch.equal(a, b)


def test_prefill_then_decode_matches_prefill():
    """Prefill of L-1 tokens into a cache, then one decoded token, equals the
    last row of a prefill over L tokens."""
    w = GI.WORKLOADS["prefill_h1024"].with_(batch=2, seq=97)
    h = GI.host_layer_inputs(w)
    full, _, _ = run_layer(w, h)
    T = T_()
    d = GI.to_device(h, w)
    cfg = cfg_of(w)
    kc = torch.zeros((2, w.hkv, 97, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    T.gqa_layer_forward(cfg, d["x"][:, :96].contiguous(), d["w_qkv"], d["q_norm_w"],
                        d["k_norm_w"], d["w_o"], k_cache=kc, v_cache=vc,
                        cache_len=torch.zeros(2, dtype=torch.int32, device="cuda"))
    last, _, _ = T.gqa_layer_forward(cfg, d["x"][:, 96:].contiguous(), d["w_qkv"],
                                     d["q_norm_w"], d["k_norm_w"], d["w_o"], k_cache=kc,
                                     v_cache=vc,
                                     cache_len=torch.full((2,), 96, dtype=torch.int32,
                                                          device="cuda"))
    assert_close(to_np(last)[:, 0], to_np(full)[:, 96], "bf16", "decode vs prefill")


def test_empty_calls_are_noops():
    T = T_()
    w = SMALL["prefill_h1024"]
    cfg = cfg_of(w)
    x = torch.zeros((0, 5, w.hidden), dtype=torch.bfloat16, device="cuda")
    h = GI.to_device(GI.host_layer_inputs(w.with_(batch=1, seq=1)), w)
    out, _, _ = T.gqa_layer_forward(cfg, x, h["w_qkv"], h["q_norm_w"], h["k_norm_w"], h["w_o"])
    assert out.shape == (0, 5, w.hidden)
