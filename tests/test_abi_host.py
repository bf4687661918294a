"""The C-ABI library without a GPU: it loads, exports every declared entry
point, resolves configurations by the pages' rules and rejects bad calls on
the host before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

T = pytest.importorskip("transformer_attention_layer_amd")


def _lib_or_skip():
    if not os.path.exists(T.LIB_PATH):
        pytest.skip("libgqa.so not built (run __graft_entry__.build())")
    return T.lib()


def _declared_functions(header="gqa.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_declares_entry_points():
    names = _declared_functions()
    for n in ["gqa_resolve", "gqa_workspace_bytes", "qkv_proj_normrope", "gqa_attn_core",
              "gqa_o_proj", "gqa_layer_forward", "gqa_layer_forward_train",
              "gqa_layer_backward", "gqa_status_string", "gqa_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib_or_skip()
    for n in _declared_functions():
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_every_header_has_its_library():
    """Each header under include/ belongs to one built library."""
    assert sorted(f for f in os.listdir(os.path.join(ROOT, "include"))
                  if f.endswith(".h")) == ["gqa.h", "gqa_peaks.h"]


def test_peaks_library_exports_and_checks_arguments():
    """The measurement microkernels' library exports what include/gqa_peaks.h
    declares, and rejects bad arguments on the host (nothing launched)."""
    from transformer_attention_layer_amd import peaks as P
    if not os.path.exists(P.PEAKS_LIB_PATH):
        pytest.skip("libgqa_peaks.so not built")
    L = P.lib()
    names = _declared_functions("gqa_peaks.h")
    assert names == ["gqa_peak_mfma_bf16", "gqa_peak_stream_read"]
    for n in names:
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value
    assert L.gqa_peak_mfma_bf16(0, 10, 16, None) == 1          # no workgroups
    assert L.gqa_peak_mfma_bf16(4, 10, None, None) == 1        # no sink
    assert L.gqa_peak_stream_read(None, 32768, 4, 16, None) == 1
    assert L.gqa_peak_stream_read(256, 1000, 4, 16, None) == 1  # size not a multiple of 32768
    assert L.gqa_peak_stream_read(8, 32768, 4, 16, None) == 1   # misaligned


def cfg(**kw):
    base = dict(hidden_size=1024, num_heads=16, num_kv_heads=8, head_dim=128)
    base.update(kw)
    return T.GQAConfig(**base)


def test_resolve_explicit_and_quotient():
    _lib_or_skip()
    # Qwen3-0.6B geometry: explicit 128 although 1024 / 16 = 64
    r = T.gqa_resolve(cfg())
    assert (r["head_dim"], r["num_kv_heads"]) == (128, 8)
    # quotient fallback (Qwen3-8B-like): 4096 / 32 = 128
    r = T.gqa_resolve(cfg(hidden_size=4096, num_heads=32, head_dim=None))
    assert r["head_dim"] == 128
    # Hkv unset means plain multi-head attention
    assert T.gqa_resolve(cfg(num_kv_heads=None))["num_kv_heads"] == 16
    # explicit head_dim needs no divisibility (1000 % 16 != 0)
    assert T.gqa_resolve(cfg(hidden_size=1000, dtype="f32"))["head_dim"] == 128
    # bf16 takes any even head_dim up to 256 (128 on the matrix-core path)
    for d in (64, 80, 256):
        assert T.gqa_resolve(cfg(head_dim=d))["head_dim"] == d
    # rotary_dim 0 / None means the whole head
    assert T.gqa_resolve(cfg())["rotary_dim"] == 128
    assert T.gqa_resolve(cfg(rotary_dim=32))["rotary_dim"] == 32


@pytest.mark.parametrize("kw,name", [
    (dict(hidden_size=1000, head_dim=None), "GQA_ERR_HEAD_DIM_INDIVISIBLE"),
    (dict(num_kv_heads=5), "GQA_ERR_GROUP_INDIVISIBLE"),
    (dict(head_dim=127, dtype="f32"), "GQA_ERR_ODD_HEAD_DIM"),
    (dict(head_dim=258), "GQA_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(head_dim=258, dtype="f32"), "GQA_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(hidden_size=1004), "GQA_ERR_UNSUPPORTED_SHAPE"),
    # bf16 rows move in 16-byte pieces: Hq*d = 3*6 = 18 is not a multiple of 8
    (dict(num_heads=3, num_kv_heads=3, head_dim=6), "GQA_ERR_UNSUPPORTED_SHAPE"),
    # the hi | lo split reads W_o twice in 32-wide K stages: 3*88 % 32 != 0
    (dict(num_heads=3, num_kv_heads=3, head_dim=88, o_split=True), "GQA_ERR_UNSUPPORTED_SHAPE"),
    (dict(hidden_size=0), "GQA_ERR_INVALID_ARG"),
    # two carriers of the attention output at once
    (dict(o_split=True, o_fp16=True), "GQA_ERR_INVALID_ARG"),
    (dict(rotary_dim=63), "GQA_ERR_INVALID_ARG"),
    (dict(rotary_dim=130), "GQA_ERR_INVALID_ARG"),
    (dict(rope_theta=0.0), "GQA_ERR_INVALID_ARG"),
    (dict(rms_eps=-1.0), "GQA_ERR_INVALID_ARG"),
    # FP8 caches: bf16 only, head_dim 64 or 128, positive finite scales
    (dict(kv_fp8=True, dtype="f32"), "GQA_ERR_UNSUPPORTED_DTYPE"),
    (dict(kv_fp8=True, head_dim=256), "GQA_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(kv_fp8=True, head_dim=80), "GQA_ERR_UNSUPPORTED_HEAD_DIM"),
    (dict(kv_fp8=True, k_scale=-1.0), "GQA_ERR_INVALID_ARG"),
    (dict(kv_fp8=True, v_scale=float("inf")), "GQA_ERR_INVALID_ARG"),
])
def test_resolve_rejects(kw, name):
    _lib_or_skip()
    with pytest.raises(T.GQAError) as e:
        T.gqa_resolve(cfg(**kw))
    assert e.value.name == name
    assert T.lib().gqa_last_error().decode()


def test_resolve_fp8_cache_scales():
    _lib_or_skip()
    r = T.gqa_resolve(cfg(kv_fp8=True, k_scale=0.0, v_scale=0.0))
    assert (r["kv_fp8"], r["k_scale"], r["v_scale"]) == (1, 1.0, 1.0)   # 0 means 1
    r = T.gqa_resolve(cfg(kv_fp8=True, k_scale=0.25, v_scale=3.0, head_dim=64))
    assert (r["k_scale"], r["v_scale"], r["head_dim"]) == (0.25, 3.0, 64)
    cc = cfg().c()
    cc.kv_fp8 = 2
    out = T._CConfig()
    assert T.STATUS_NAMES[T.lib().gqa_resolve(ctypes.byref(cc), ctypes.byref(out))] == \
        "GQA_ERR_INVALID_ARG"


def test_fp8_cache_rejects_prefill_attention_before_launch():
    """An FP8 cache is read by the split-KV decode kernel only: attention
    calls whose group * q_len exceeds 32 are rejected on the host."""
    _lib_or_skip()
    L = T.lib()
    c = cfg(kv_fp8=True)  # group 2: q_len up to 16
    assert T.STATUS_NAMES[_raw_call_layer(c, 2, 17, 64)] == "GQA_ERR_UNSUPPORTED_SHAPE"
    cc = c.c()
    st = L.gqa_attn_core(ctypes.byref(cc), 2, 17, 1, 1, 1, None, 64, 1, 1, 1 << 40, None)
    assert T.STATUS_NAMES[st] == "GQA_ERR_UNSUPPORTED_SHAPE"
    assert "decode" in L.gqa_last_error().decode()


def test_unsupported_head_dim_message_names_the_dimension():
    _lib_or_skip()
    # the quotient 2560 / 32 = 80 is supported in bf16; 8192 / 16 = 512 is not
    assert T.gqa_resolve(cfg(hidden_size=2560, num_heads=32, head_dim=None))["head_dim"] == 80
    with pytest.raises(T.GQAError) as e:
        T.gqa_resolve(cfg(hidden_size=8192, num_heads=16, num_kv_heads=16, head_dim=None))
    assert "512" in str(e.value)


def test_workspace_sizes():
    _lib_or_skip()
    c = cfg()
    assert T.gqa_workspace_bytes(c, 8, 2048, 2048, T.WS_ATTN) == 0          # prefill: none
    assert T.gqa_workspace_bytes(c, 8, 2048, 2048, T.WS_QKV) >= 8 * 2048 * 64 * 8
    lay = T.gqa_workspace_bytes(c, 8, 2048, 2048, T.WS_LAYER)
    assert lay >= 2 * 8 * 2048 * 16 * 128 * 2
    dec = T.gqa_workspace_bytes(cfg(hidden_size=2560, num_heads=32), 64, 1, 32769, T.WS_ATTN)
    assert dec > 0
    assert T.gqa_workspace_bytes(cfg(num_kv_heads=5), 1, 1, 1, T.WS_LAYER) == 0


def test_workspace_sizes_of_empty_and_few_token_calls():
    """Sizing an empty call (no batch, or no new tokens) is host arithmetic
    only and must not divide by the zero token count; a few-token call's
    projection workspace holds at least its fp32 output."""
    _lib_or_skip()
    dec = cfg(hidden_size=2560, num_heads=32, num_kv_heads=1)
    for kind in (T.WS_QKV, T.WS_ATTN, T.WS_LAYER):
        for batch, q_len in ((0, 1), (4, 0), (0, 0)):
            assert T.gqa_workspace_bytes(dec, batch, q_len, 64, kind) >= 0
    n_qkv = (32 + 2) * 128
    for tokens in (1, 64, 256):
        assert T.gqa_workspace_bytes(dec, tokens, 1, 64, T.WS_QKV) >= tokens * n_qkv * 4


def _raw_call_layer(c, batch, q_len, cap, ptr=1, ws_bytes=1 << 40):
    L = T.lib()
    cc = c.c()
    p = ctypes.c_void_p(ptr) if ptr else None
    return L.gqa_layer_forward(ctypes.byref(cc), batch, q_len, p, p, p, p, p, p, p, cap, None, p,
                               p, ws_bytes, None)


def test_entry_points_validate_before_launch():
    """Every rejected call returns before touching the device (no GPU here)."""
    _lib_or_skip()
    L = T.lib()
    # empty batch / sequence: a no-op
    assert _raw_call_layer(cfg(), 0, 16, 16) == 0
    assert _raw_call_layer(cfg(), 2, 0, 16) == 0
    # null tensors
    assert T.STATUS_NAMES[_raw_call_layer(cfg(), 2, 16, 16, ptr=0)] == "GQA_ERR_INVALID_ARG"
    # capacity below q_len
    assert T.STATUS_NAMES[_raw_call_layer(cfg(), 2, 16, 8)] == "GQA_ERR_CAPACITY"
    # workspace too small
    assert T.STATUS_NAMES[_raw_call_layer(cfg(), 2, 16, 16, ws_bytes=16)] == \
        "GQA_ERR_WORKSPACE_TOO_SMALL"
    # bad config
    assert T.STATUS_NAMES[_raw_call_layer(cfg(num_kv_heads=3), 2, 16, 16)] == \
        "GQA_ERR_GROUP_INDIVISIBLE"
    cc = cfg(qk_norm=True).c()
    st = L.qkv_proj_normrope(ctypes.byref(cc), 1, 4, 1, 1, None, None, None, 1, 1, 1, 4, 1,
                             1 << 30, None)
    assert T.STATUS_NAMES[st] == "GQA_ERR_INVALID_ARG"   # qk_norm on, weights missing
    st = L.gqa_attn_core(ctypes.byref(cc), -1, 4, 1, 1, 1, None, 4, 1, None, 0, None)
    assert T.STATUS_NAMES[st] == "GQA_ERR_INVALID_ARG"
    st = L.gqa_o_proj(ctypes.byref(cc), 5, None, 1, 1, None)
    assert T.STATUS_NAMES[st] == "GQA_ERR_INVALID_ARG"
    assert L.gqa_status_string(5) == b"GQA_ERR_UNSUPPORTED_HEAD_DIM"


def test_product_path_has_no_oracle_dependency():
    """The package never imports the oracle or a CPU fallback."""
    pkg = os.path.join(ROOT, "transformer_attention_layer_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f


def test_missing_library_fails_loudly():
    """Without the built library the binding raises at its first call
    instead of falling back to anything else."""
    import subprocess
    import sys
    code = ("import transformer_attention_layer_amd as T\n"
            "try:\n"
            "    T.lib()\n"
            "except ImportError as e:\n"
            "    print('raised', 'missing' in str(e))\n"
            "else:\n"
            "    print('loaded')\n")
    env = dict(os.environ, GQA_LIB=os.path.join(ROOT, "no_such_dir", "libgqa.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "raised True", r.stdout


def _raw_train(c, batch, q_len, saved_ptr=1, ws_bytes=1 << 40, backward=False, null_saved=False):
    L = T.lib()
    cc = c.c()
    p = ctypes.c_void_p(1)
    sv = T._CSaved(*([0 if null_saved else saved_ptr] * 6))
    if not backward:
        return L.gqa_layer_forward_train(ctypes.byref(cc), batch, q_len, p, p, p, p, p,
                                         ctypes.byref(sv), p, p, ws_bytes, None)
    g = T._CGrads(1, 1, 1, 1, 1)
    return L.gqa_layer_backward(ctypes.byref(cc), batch, q_len, p, p, p, p, p, ctypes.byref(sv),
                                p, ctypes.byref(g), p, ws_bytes, None)


@pytest.mark.parametrize("backward", [False, True])
def test_training_entry_points_validate_before_launch(backward):
    """The training pair takes bf16, head_dim 64 or 128, no o_split and no FP8
    cache; bad calls are rejected on the host (no GPU here)."""
    _lib_or_skip()
    name = lambda st: T.STATUS_NAMES[st]  # noqa: E731
    assert _raw_train(cfg(), 0, 16, backward=backward) == 0
    assert _raw_train(cfg(), 2, 0, backward=backward) == 0
    assert name(_raw_train(cfg(dtype="f32"), 2, 16, backward=backward)) == \
        "GQA_ERR_UNSUPPORTED_DTYPE"
    for d in (80, 256):
        assert name(_raw_train(cfg(head_dim=d), 2, 16, backward=backward)) == \
            "GQA_ERR_UNSUPPORTED_HEAD_DIM"
    assert name(_raw_train(cfg(o_split=True), 2, 16, backward=backward)) == \
        "GQA_ERR_UNSUPPORTED_SHAPE"
    assert name(_raw_train(cfg(kv_fp8=True), 2, 16, backward=backward)) == \
        "GQA_ERR_UNSUPPORTED_SHAPE"
    assert name(_raw_train(cfg(), 2, 16, null_saved=True, backward=backward)) == \
        "GQA_ERR_INVALID_ARG"
    # the vectorised norm/RoPE passes turn 4 features per lane: rotary width % 8
    assert name(_raw_train(cfg(rotary_dim=36), 2, 16, backward=backward)) == \
        "GQA_ERR_UNSUPPORTED_SHAPE"
    assert name(_raw_train(cfg(), 2, 16, ws_bytes=64, backward=backward)) == \
        "GQA_ERR_WORKSPACE_TOO_SMALL"


def test_backward_workspace_covers_its_buffers():
    """The backward's workspace holds at least dO and dy (bf16), dq/dk/dv
    (fp32) and the chunked transposes of dout, o, dy and x."""
    _lib_or_skip()
    c = cfg()
    B, L, H, qw, nq, kvw = 8, 2048, 1024, 2048, 4096, 1024
    T_ = B * L
    n = T.gqa_workspace_bytes(c, B, L, L, T.WS_BACKWARD)
    floor = T_ * qw * 2 + T_ * nq * 2 + T_ * (qw + 2 * kvw) * 4 + T_ * (H + qw + nq + H) * 2
    assert n >= floor
    # the training forward's RoPE table: L rows of d/2 (cos, sin) pairs
    assert T.gqa_workspace_bytes(c, B, L, L, T.WS_TRAIN_FORWARD) == L * 64 * 8
    assert T.gqa_workspace_bytes(cfg(dtype="f32"), B, L, L, T.WS_BACKWARD) > 0  # sized, then rejected


def test_o_fp16_flag_and_workspace():
    """o_fp16 takes 0 or 1, and the layer workspace grows by W_o as fp16
    (hidden x Hq*d x 2 bytes, 256-byte aligned), except for few tokens,
    whose o_proj rounds W_o inside the product."""
    _lib_or_skip()
    cc = cfg().c()
    cc.o_fp16 = 2
    out = T._CConfig()
    assert T.STATUS_NAMES[T.lib().gqa_resolve(ctypes.byref(cc), ctypes.byref(out))] == \
        "GQA_ERR_INVALID_ARG"
    assert T.gqa_resolve(cfg(o_fp16=True))["o_fp16"] == 1
    a = T.gqa_workspace_bytes(cfg(), 2, 300, 300, T.WS_LAYER)
    b = T.gqa_workspace_bytes(cfg(o_fp16=True), 2, 300, 300, T.WS_LAYER)
    assert b - a == 1024 * 16 * 128 * 2
    a = T.gqa_workspace_bytes(cfg(), 64, 1, 300, T.WS_LAYER)
    b = T.gqa_workspace_bytes(cfg(o_fp16=True), 64, 1, 300, T.WS_LAYER)
    assert b == a
