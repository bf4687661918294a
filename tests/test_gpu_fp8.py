"""GPU parity of the FP8 (E4M3) K/V cache ("Head Dimension" article, section
5.2; the format and scales are the oracle's reading 10): the split-KV decode
attention over FP8 caches, the FP8 append of the norm/RoPE pass and the whole
decode layer, against the CPU oracle on the same seeded inputs."""
import dataclasses
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gqa_inputs as GI  # noqa: E402
from gpu_util import announce, assert_close, cfg_of, resolved, to_np  # noqa: E402
from oracle import gqa_oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAN_CODE = 0x7F  # E4M3 NaN: marks cache rows the kernels must not read


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


def _codes_dev(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).cuda()


def check_codes(got, want, x_scaled, what):
    """Appended codes: equal to the oracle's, except where the exact value
    x / scale (the oracle's, float64) sits at the midpoint of two
    neighbouring codes to within the GPU's float32 rounding; there either
    code is the nearest.  Such ties must stay rare."""
    got = np.asarray(got, dtype=np.uint8)
    want = np.asarray(want, dtype=np.uint8)
    mism = got != want
    frac = float(mism.mean()) if mism.size else 0.0
    print(f"  {what}: {int(mism.sum())} of {mism.size} codes differ", flush=True)
    if not mism.any():
        return
    vg = O.e4m3_value(got[mism])
    vw = O.e4m3_value(want[mism])
    x = np.clip(np.asarray(x_scaled, dtype=np.float64)[mism], -448.0, 448.0)
    step = np.abs(vg - vw)
    assert np.all(np.isfinite(vg)), f"{what}: NaN code written"
    assert np.all(step > 0), f"{what}: codes differ in sign only"
    assert np.all(np.abs(x - 0.5 * (vg + vw)) <= 0.01 * step), \
        f"{what}: a code differs away from a rounding tie"
    assert frac < 1e-3, f"{what}: {frac:.2e} of the codes differ"


@pytest.mark.parametrize("d,hq,hkv,q_len,ks,vs", [
    (128, 32, 8, 1, 1.0, 1.0),
    (128, 32, 8, 2, 0.25, 2.0),
    (128, 32, 1, 1, 0.7, 1.3),    # MQA: 32 query heads on one KV head
    (64, 8, 4, 1, 0.5, 0.5),
    (64, 16, 2, 4, 1.0, 3.0),     # group 8 x 4 new tokens = 32 rows
])
def test_fp8_decode_attention(d, hq, hkv, q_len, ks, vs):
    """gqa_attn_core over FP8 caches whose codes the oracle's quantizer
    made: both sides attend over exactly the same values.  Three sequences
    of different lengths over several key splits; rows past each length
    hold NaN codes."""
    T = T_()
    announce(f"[fp8 decode attention] d={d} Hq={hq} Hkv={hkv} q_len={q_len} scales={ks},{vs}")
    rng = np.random.default_rng(1000 + d + hq + q_len)
    B, cap = 3, 2600
    kv_len = np.array([2600, 1500, 37], dtype=np.int64)
    q = GI.round_bf16(rng.standard_normal((B, hq, q_len, d)).astype(np.float32))
    kraw = rng.standard_normal((B, hkv, cap, d)) * np.exp2(rng.integers(-2, 3, (B, hkv, cap, d)))
    vraw = rng.standard_normal((B, hkv, cap, d))
    kc = O.quantize_e4m3(kraw / ks)
    vc = O.quantize_e4m3(vraw / vs)
    for b in range(B):
        kc[b, :, kv_len[b]:] = NAN_CODE
        vc[b, :, kv_len[b]:] = NAN_CODE
    cfg = T.GQAConfig(hidden_size=1024, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                      kv_fp8=True, k_scale=ks, v_scale=vs)
    qd = torch.from_numpy(q).cuda().to(torch.bfloat16)
    o = T.gqa_attn_core(cfg, qd, _codes_dev(kc), _codes_dev(vc),
                        kv_len=torch.from_numpy(kv_len.astype(np.int32)).cuda())
    kvals = np.zeros((B, hkv, cap, d))
    vvals = np.zeros((B, hkv, cap, d))
    for b in range(B):
        n = kv_len[b]
        kvals[b, :, :n] = O.e4m3_value(kc[b, :, :n]) * ks
        vvals[b, :, :n] = O.e4m3_value(vc[b, :, :n]) * vs
    pos = kv_len[:, None] - q_len + np.arange(q_len)[None, :]
    ref = O.merge_heads(O.grouped_attention(q.astype(np.float64), kvals, vvals, pos, kv_len,
                                            1.0 / np.sqrt(d), True))
    assert_close(to_np(o), ref, "bf16", "attention")


def _fp8_workload(q_len=1):
    return GI.WORKLOADS["decode_h2560_gqa"].with_(batch=3, seq=q_len, cache_len=1000)


@pytest.mark.parametrize("q_len", [1, 2])
def test_fp8_decode_layer(q_len):
    """The decode layer with FP8 caches of different lengths per sequence:
    the appended codes and the output against the oracle's kv_fp8 layer."""
    T = T_()
    w = _fp8_workload(q_len)
    ks, vs = 0.5, 2.0
    announce(f"[fp8 decode layer] B={w.batch} q_len={q_len} cache up to {w.cache_len}")
    h = GI.host_layer_inputs(w)
    cache = GI.host_cache(w)
    cl = np.array([1000, 400, 777], dtype=np.int64)
    kc = O.quantize_e4m3(np.nan_to_num(cache["k_cache"]) / ks)
    vc = O.quantize_e4m3(np.nan_to_num(cache["v_cache"]) / vs)
    for b in range(w.batch):
        kc[b, :, cl[b]:] = NAN_CODE
        vc[b, :, cl[b]:] = NAN_CODE
    cfg = dataclasses.replace(cfg_of(w), kv_fp8=True, k_scale=ks, v_scale=vs)
    d = GI.to_device(h, w)
    kdev, vdev = _codes_dev(kc), _codes_dev(vc)
    out, kdev, vdev = T.gqa_layer_forward(
        cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"], d["w_o"], k_cache=kdev,
        v_cache=vdev, cache_len=torch.from_numpy(cl.astype(np.int32)).cuda())
    res = resolved(w)
    ref, rk, rv = O.layer_forward(res, h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"],
                                  h["w_o"], rope_theta=w.rope_theta, rms_eps=w.rms_eps,
                                  k_cache=kc, v_cache=vc, cache_len=cl, kv_fp8=True,
                                  k_scale=ks, v_scale=vs)
    gk, gv = kdev.cpu().numpy(), vdev.cpu().numpy()
    pos = cl[:, None] + np.arange(q_len)[None, :]
    _, k64, v64 = O.qkv_normrope(res, h["x"].astype(np.float64), h["w_qkv"].astype(np.float64),
                                 h["q_norm_w"].astype(np.float64),
                                 h["k_norm_w"].astype(np.float64), pos, w.rope_theta, w.rms_eps)
    for b in range(w.batch):
        s0 = int(cl[b])
        check_codes(gk[b, :, s0:s0 + q_len], rk[b, :, s0:s0 + q_len], k64[b] / ks, f"k append {b}")
        check_codes(gv[b, :, s0:s0 + q_len], rv[b, :, s0:s0 + q_len], v64[b] / vs, f"v append {b}")
        assert np.array_equal(gk[b, :, :s0], kc[b, :, :s0]), "rows below the append changed"
    assert_close(to_np(out), ref, "bf16", "out")


@pytest.mark.parametrize("B,L", [(2, 40), (2, 200)])
def test_fp8_qkv_append(B, L):
    """qkv_proj_normrope into FP8 caches (few tokens: the weight-streaming
    projection; 400 tokens: the tiled GEMM), then the norm/RoPE pass writes
    the codes."""
    T = T_()
    w = GI.WORKLOADS["decode_h2560_gqa"].with_(batch=B, seq=L, cache_len=0)
    ks, vs = 0.25, 1.5
    announce(f"[fp8 qkv append] B={B} L={L}")
    res = resolved(w)
    h = GI.host_layer_inputs(w)
    d = GI.to_device(h, w)
    cfg = dataclasses.replace(cfg_of(w), kv_fp8=True, k_scale=ks, v_scale=vs)
    cap = L + 5
    kdev = torch.full((B, res.hkv, cap, res.d), NAN_CODE, dtype=torch.uint8, device="cuda")
    vdev = torch.full_like(kdev, NAN_CODE)
    q, kdev, vdev = T.qkv_proj_normrope(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"],
                                        k_cache=kdev, v_cache=vdev)
    pos = np.tile(np.arange(L), (B, 1))
    rq, rk, rv = O.qkv_normrope(res, h["x"].astype(np.float64), h["w_qkv"].astype(np.float64),
                                h["q_norm_w"].astype(np.float64),
                                h["k_norm_w"].astype(np.float64), pos, w.rope_theta, w.rms_eps)
    assert_close(to_np(q), rq, "bf16", "q")
    gk, gv = kdev.cpu().numpy(), vdev.cpu().numpy()
    check_codes(gk[:, :, :L], O.quantize_e4m3(rk / ks), rk / ks, "k codes")
    check_codes(gv[:, :, :L], O.quantize_e4m3(rv / vs), rv / vs, "v codes")
    assert np.all(gk[:, :, L:] == NAN_CODE) and np.all(gv[:, :, L:] == NAN_CODE)
