"""GPU parity of the layer's training path: gqa_layer_forward_train (the
output and the saved log-sum-exp) and gqa_layer_backward (the gradients of x,
the fused QKV weight, both QK-norm weights and W_o) against the oracle's
float64 forward and chain-rule backward on the same seeded inputs.

Gradients are compared relative to their own scale: max|err| / max|ref|
and sum|err| / sum|ref|.  The bounds follow from the arithmetic: the saved
q, k, v, o, the upstream gradient and every intermediate gradient that
feeds a matrix product (dO, P, dS, dy) are rounded to bf16 (relative
2^-9 each), and a gradient passes through up to five such roundings, with
fp32 accumulation in between."""
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

GRAD_TOL = (2e-2, 1e-2)  # (max|err| / max|ref|, sum|err| / sum|ref|)


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


def check_grad(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    diff = np.abs(got - ref)
    scale = float(np.abs(ref).max())
    max_rel = float(diff.max()) / scale if scale > 0 else float(diff.max())
    mean_rel = float(diff.sum() / np.abs(ref).sum()) if scale > 0 else float(diff.sum())
    print(f"  {what}: max_err/max_ref={max_rel:.3e} mean_rel={mean_rel:.3e}", flush=True)
    assert max_rel <= GRAD_TOL[0] and mean_rel <= GRAD_TOL[1], \
        f"{what}: {max_rel:.3e} (tol {GRAD_TOL[0]}), {mean_rel:.3e} (tol {GRAD_TOL[1]})"


BASE = GI.WORKLOADS["prefill_h1024"]

# (name, workload): several key/query tiles with ragged tails, GQA groups 2,
# 3 and 4, MQA, head_dim 64 and 128, no mask, no QK-norm, partial rotary.
CASES = [
    ("h1024_gqa2_L300", BASE.with_(batch=2, seq=300)),
    ("h1024_gqa2_L1", BASE.with_(batch=3, seq=1)),
    ("h640_gqa4_d128_rot64_L129", BASE.with_(hidden=640, hq=8, hkv=2, seq=129, batch=2,
                                             rotary_dim=64, seed=11)),
    ("h512_mqa_d64_noncausal_L200", BASE.with_(hidden=512, hq=8, hkv=1, head_dim=64, seq=200,
                                               batch=1, causal=False, seed=12)),
    ("h512_d64_nonorm_rot32_L97", BASE.with_(hidden=512, hq=4, hkv=4, head_dim=64, seq=97,
                                             batch=2, qk_norm=False, rotary_dim=32, seed=13)),
    # an odd group (3 query heads per KV head: one head per wave in dQ)
    ("h768_gqa3_d64_L190", BASE.with_(hidden=768, hq=12, hkv=4, head_dim=64, seq=190,
                                      batch=2, seed=14)),
]


def _run(w):
    T = T_()
    cfg = cfg_of(w)
    h = GI.host_layer_inputs(w)
    dout = GI.host_upstream_grad(w)
    d = GI.to_device(h, w)
    dd = torch.from_numpy(dout).cuda().to(torch.bfloat16)
    out, saved = T.gqa_layer_forward_train(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"],
                                           d["w_o"])
    grads = T.gqa_layer_backward(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"], d["w_o"],
                                 saved, dd)
    torch.cuda.synchronize()
    return h, dout, out, saved, grads


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(name, w):
    announce(f"[backward] {name}: B={w.batch} L={w.seq} H={w.hidden} {w.hq}/{w.hkv}/{w.d} "
             f"causal={w.causal} qk_norm={w.qk_norm} rot={w.rotary_dim}")
    res = resolved(w)
    h, dout, out, saved, grads = _run(w)
    ref_out, _, _ = O.layer_forward(res, h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"],
                                    h["w_o"], rope_theta=w.rope_theta, rms_eps=w.rms_eps,
                                    qk_norm=w.qk_norm, causal=w.causal, rotary_dim=w.rotary_dim)
    assert_close(to_np(out), ref_out, "bf16", "forward out")
    g = O.layer_backward(res, h["x"], h["w_qkv"], h["q_norm_w"] if w.qk_norm else None,
                         h["k_norm_w"] if w.qk_norm else None, h["w_o"], dout,
                         rope_theta=w.rope_theta, rms_eps=w.rms_eps, qk_norm=w.qk_norm,
                         causal=w.causal, rotary_dim=w.rotary_dim)
    check_grad(to_np(grads["dw_o"]), g["dw_o"], "dW_o")
    check_grad(to_np(grads["dw_qkv"]), g["dw_qkv"], "dW_qkv")
    check_grad(to_np(grads["dx"]), g["dx"], "dx")
    if w.qk_norm:
        check_grad(to_np(grads["dq_norm_w"]), g["dq_norm_w"], "dq_norm_w")
        check_grad(to_np(grads["dk_norm_w"]), g["dk_norm_w"], "dk_norm_w")


def test_saved_lse_is_the_row_log_sum_exp():
    """The forward's saved lse against log sum_j exp(q.k_j / sqrt(d)) over
    the visible keys, computed in float64 from the saved (bf16) q and k."""
    w = CASES[0][1]
    announce("[backward] saved lse")
    _, _, _, saved, _ = _run(w)
    q = to_np(saved.q).astype(np.float64)
    k = to_np(saved.k).astype(np.float64)
    lse = to_np(saved.lse)
    res = resolved(w)
    grp = res.hq // res.hkv
    L = w.seq
    mask = np.tril(np.ones((L, L), dtype=bool))
    worst = 0.0
    for b in range(w.batch):
        for hq in range(res.hq):
            s = q[b, hq] @ k[b, hq // grp].T * res.scale
            s = np.where(mask, s, -np.inf)
            m = s.max(-1)
            ref = m + np.log(np.exp(s - m[:, None]).sum(-1))
            worst = max(worst, float(np.abs(lse[b, hq] - ref).max()))
    print(f"  lse max abs err {worst:.3e}", flush=True)
    assert worst < 1e-2


def test_backward_is_deterministic():
    """Two backward calls on the same inputs give bit-identical gradients
    (no atomics)."""
    w = CASES[2][1]
    announce("[backward] determinism")
    T = T_()
    cfg = cfg_of(w)
    h = GI.host_layer_inputs(w)
    d = GI.to_device(h, w)
    dd = torch.from_numpy(GI.host_upstream_grad(w)).cuda().to(torch.bfloat16)
    _, saved = T.gqa_layer_forward_train(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"],
                                         d["w_o"])
    g1 = T.gqa_layer_backward(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"], d["w_o"],
                              saved, dd)
    g1 = {k: None if v is None else v.clone() for k, v in g1.items()}
    g2 = T.gqa_layer_backward(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"], d["w_o"],
                              saved, dd)
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k


def test_fullsize_directional_derivatives():
    """At the bench's size and launch configuration (8 x 2048, 1024-wide,
    16/8/128), where the float64 oracle is too slow: for each gradient g of a
    parameter p, the central difference f(p + v) - f(p - v) of
    f = sum(dout * forward) equals <g, (p + v) - (p - v)> to first order,
    with v along g itself (a wrong scale, sign or pattern of g breaks it).
    Step sizes: 0.5% of the parameter's RMS (2% for the 128-entry norm
    weights, whose bf16 steps are coarse); the bounds cover the O(step^2)
    truncation and the bf16 rounding noise of two forwards (measured 4e-8 to
    1.1e-3, and 6e-3 / 1e-2 for the norm weights)."""
    T = T_()
    w = GI.WORKLOADS["prefill_h1024"]
    announce(f"[backward] full size directional derivatives B={w.batch} L={w.seq}")
    cfg = cfg_of(w)
    h = GI.device_layer_inputs(w)
    dout = GI.device_upstream_grad(w)
    saved = T.TrainSaved(cfg, w.batch, w.seq)
    out = torch.empty((w.batch, w.seq, w.hidden), dtype=torch.float32, device="cuda")

    def f(p):
        T.gqa_layer_forward_train(cfg, p["x"], p["w_qkv"], p["q_norm_w"], p["k_norm_w"], p["w_o"],
                                  saved=saved, out=out)
        return float((out.double() * dout.double()).sum())

    f(h)
    g = T.gqa_layer_backward(cfg, h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"], h["w_o"],
                             saved, dout)
    g = {k: v.clone() for k, v in g.items()}
    for name, key, eps, tol in (("x", "dx", 0.005, 1e-2), ("w_qkv", "dw_qkv", 0.005, 1e-2),
                                ("w_o", "dw_o", 0.005, 1e-2), ("q_norm_w", "dq_norm_w", 0.02, 5e-2),
                                ("k_norm_w", "dk_norm_w", 0.02, 5e-2)):
        p0 = h[name]
        gr = g[key].double()
        assert torch.isfinite(gr).all(), key
        v = gr / gr.pow(2).mean().sqrt() * p0.double().pow(2).mean().sqrt() * eps
        pp, pm = dict(h), dict(h)
        pp[name] = (p0.double() + v).to(p0.dtype)
        pm[name] = (p0.double() - v).to(p0.dtype)
        pred = float((gr * (pp[name].double() - pm[name].double())).sum())
        est = f(pp) - f(pm)
        rel = abs(est - pred) / abs(pred)
        print(f"  {key}: difference {est:.6e} vs <g, step> {pred:.6e}: rel {rel:.2e}", flush=True)
        assert rel <= tol, (key, est, pred, rel)


def test_backward_persistent_gemm_shapes():
    """A shape whose backward GEMMs walk more than one 256 x 256 tile per
    workgroup (dx 4096 x 5120: 320 tiles; dO 4096 x 4096; dW_qkv 6144 x
    5120 over 4096 tokens: 480 tiles, one token chunk; dW_o 5120 x 4096: 320
    tiles), element by element against the oracle's chain rule in float32;
    a second backward call is bitwise identical."""
    w = BASE.with_(batch=16, seq=256, hidden=5120, hq=32, hkv=8, seed=15)
    announce(f"[backward] persistent GEMM shapes B={w.batch} L={w.seq} H={w.hidden} "
             f"{w.hq}/{w.hkv}/{w.d}")
    T = T_()
    res = resolved(w)
    h, dout, out, saved, grads = _run(w)
    g2 = T.gqa_layer_backward(cfg_of(w), *[GI.to_device({k: h[k]}, w)[k] for k in
                                           ("x", "w_qkv", "q_norm_w", "k_norm_w", "w_o")],
                              saved, torch.from_numpy(dout).cuda().to(torch.bfloat16))
    torch.cuda.synchronize()
    for k in grads:
        if grads[k] is not None:
            assert torch.equal(grads[k], g2[k]), k
    g = O.layer_backward(res, h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"], h["w_o"], dout,
                         rope_theta=w.rope_theta, rms_eps=w.rms_eps, qk_norm=w.qk_norm,
                         causal=w.causal, dtype=np.float32)
    check_grad(to_np(grads["dw_o"]), g["dw_o"], "dW_o")
    check_grad(to_np(grads["dw_qkv"]), g["dw_qkv"], "dW_qkv")
    check_grad(to_np(grads["dx"]), g["dx"], "dx")
    check_grad(to_np(grads["dq_norm_w"]), g["dq_norm_w"], "dq_norm_w")
    check_grad(to_np(grads["dk_norm_w"]), g["dk_norm_w"], "dk_norm_w")
