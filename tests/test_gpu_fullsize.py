"""GPU parity at the workloads' full sizes, in the launch configuration the
bench times.

- The 8 x 2048 prefill (hidden 1024) is compared element by element: the
  whole layer output, and q, k, v of the fused projection, whose persistent
  GEMM takes four 256 x 256 tiles per workgroup at this size.
- The 4096- and 5120-wide prefills are compared on 256 rows of every
  sequence (its first 64 tokens, its last, and an even stride between),
  from the oracle's row mode: row t needs only x[b, :t+1].
- The projection GEMMs at those sizes (20 and 16 tiles per workgroup) are
  compared element by element on sampled tokens that fall in every tile of
  the token axis (every feature is compared), and o_proj on the whole
  4096-wide output.
- Decode is compared on sampled sequences of the 32768-token caches.
- Every full-size call is also run twice and must give bitwise the same
  output.

The oracle runs in float32 here, the precision the tutorial's attention step
names, to keep the host work to seconds."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gqa_inputs as GI  # noqa: E402
from gpu_util import announce, assert_close, cfg_of, errors, resolved, to_np  # noqa: E402
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
    torch.cuda.empty_cache()


def T_():
    import transformer_attention_layer_amd as T
    return T


def sampled_rows(L: int, n: int = 256, head: int = 64):
    """The first `head` positions, the last, and an even stride between:
    `n` distinct positions in all (or every position if L <= n)."""
    if L <= n:
        return list(range(L))
    rest = np.linspace(head, L - 1, n - head).round().astype(int)
    rows = sorted(set(range(head)) | set(int(t) for t in rest))
    t = head + 1
    while len(rows) < n:  # rounding collisions: fill with unused positions
        if t not in rows:
            rows.append(t)
        t += 1
    return sorted(rows)


def tile_tokens(T: int, tile: int = 256):
    """One token in every `tile`-token block of the token axis (at a varying
    offset inside the block), plus the last token."""
    toks = [min(T - 1, j * tile + (37 * j + 11) % tile) for j in range((T + tile - 1) // tile)]
    return sorted(set(toks) | {T - 1})


def layer(w, d, **kw):
    T = T_()
    ws = T.LayerWorkspace(cfg_of(w), w.batch, w.seq, w.kv_capacity)
    return T.gqa_layer_forward(cfg_of(w), d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"],
                               d["w_o"], workspace=ws, **kw)


def test_prefill_h1024_whole_layer_elementwise():
    """Every output element of the 8 x 2048 prefill, and the appended k, v
    rows, against the oracle's whole layer; then the same call again must
    be bitwise identical."""
    w = GI.WORKLOADS["prefill_h1024"]
    announce(f"[full size] {w.name} whole layer B={w.batch} L={w.seq}")
    h = GI.host_layer_inputs(w)
    d = GI.to_device(h, w)
    out, kc, vc = layer(w, d)
    out2, _, _ = layer(w, d)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "repeat call differs"
    got, got_k, got_v = to_np(out), to_np(kc), to_np(vc)
    del out, out2, kc, vc, d
    torch.cuda.empty_cache()
    res = resolved(w)
    ref, rk, rv = O.layer_forward(res, h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"],
                                  h["w_o"], rope_theta=w.rope_theta, rms_eps=w.rms_eps,
                                  qk_norm=w.qk_norm, causal=w.causal,
                                  k_cache=np.zeros((w.batch, w.hkv, w.seq, w.d), np.float32),
                                  v_cache=np.zeros((w.batch, w.hkv, w.seq, w.d), np.float32),
                                  cache_len=np.zeros(w.batch, np.int64), dtype=np.float32)
    assert_close(got_k, rk, w.dtype, "k cache (all rows)")
    assert_close(got_v, rv, w.dtype, "v cache (all rows)")
    assert_close(got, ref, w.dtype, "out (every element)")
    # per-sequence view, so a wrong tile in one sequence cannot hide in the mean
    for b in range(w.batch):
        ma, mr = errors(got[b], ref[b])
        assert ma <= 2e-2 and mr <= 5e-3, (b, ma, mr)


def test_prefill_h1024_qkv_elementwise():
    """q, k, v of qkv_proj_normrope at 8 x 2048: 1024 tiles of 256 x 256 on
    the persistent GEMM (four per workgroup), every element."""
    T = T_()
    w = GI.WORKLOADS["prefill_h1024"]
    announce(f"[full size] {w.name} qkv_proj_normrope every element")
    h = GI.host_layer_inputs(w)
    d = GI.to_device(h, w)
    q, kc, vc = T.qkv_proj_normrope(cfg_of(w), d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"])
    torch.cuda.synchronize()
    gq, gk, gv = to_np(q), to_np(kc), to_np(vc)
    del q, kc, vc, d
    pos = np.tile(np.arange(w.seq), (w.batch, 1))
    rq, rk, rv = O.qkv_normrope(resolved(w), h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"],
                                pos, w.rope_theta, w.rms_eps, qk_norm=w.qk_norm)
    assert_close(gq, rq, w.dtype, "q")
    assert_close(gk, rk, w.dtype, "k")
    assert_close(gv, rv, w.dtype, "v")


@pytest.mark.parametrize("name", ["quotient_h4096", "wide_h5120"])
def test_prefill_rows_every_sequence(name):
    """256 rows of every sequence (first 64, last, stride between) of the
    whole layer at full size, in the bench's launch configuration; the
    repeat call is bitwise identical."""
    w = GI.WORKLOADS[name]
    trows = sampled_rows(w.seq)
    rows = [(b, t) for b in range(w.batch) for t in trows]
    announce(f"[full size] {name} B={w.batch} L={w.seq} {len(rows)} rows "
             f"(every sequence: t=0..63, t={w.seq - 1}, stride)")
    h = GI.host_layer_inputs(w)
    d = GI.to_device(h, w)
    out, _, _ = layer(w, d)
    out2, _, _ = layer(w, d)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "repeat call differs"
    del out2, d
    idx_b = torch.tensor([b for b, _ in rows], device="cuda")
    idx_t = torch.tensor([t for _, t in rows], device="cuda")
    got = to_np(out[idx_b, idx_t])
    del out
    torch.cuda.empty_cache()
    ref = O.layer_forward_rows(resolved(w), h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"],
                               h["w_o"], rows, rope_theta=w.rope_theta, rms_eps=w.rms_eps,
                               qk_norm=w.qk_norm, rotary_dim=w.rotary_dim, dtype=np.float32)
    for b in range(w.batch):
        sel = [i for i, (bb, _) in enumerate(rows) if bb == b]
        ma, mr = errors(got[sel], ref[sel])
        worst = rows[sel[int(np.abs(got[sel] - ref[sel]).max(axis=1).argmax())]][1]
        print(f"  sequence {b}: max_abs={ma:.3e} (row t={worst}) mean_rel={mr:.3e}", flush=True)
    assert_close(got, ref, w.dtype, f"{len(rows)} sampled rows")


@pytest.mark.parametrize("name", ["quotient_h4096", "wide_h5120"])
def test_qkv_projection_every_tile(name):
    """q, k, v of qkv_proj_normrope at full size (the persistent GEMM walks
    several tiles per workgroup) for one token in every 256-token tile and
    every feature, against the oracle's steps 1-4 at those tokens' positions."""
    T = T_()
    w = GI.WORKLOADS[name]
    toks = tile_tokens(w.batch * w.seq)
    announce(f"[full size] {name} qkv_proj_normrope, {len(toks)} tokens over every tile")
    h = GI.host_layer_inputs(w)
    d = GI.to_device(h, w)
    q, kc, vc = T.qkv_proj_normrope(cfg_of(w), d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"])
    q2, _, _ = T.qkv_proj_normrope(cfg_of(w), d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"])
    torch.cuda.synchronize()
    assert torch.equal(q, q2), "repeat call differs"
    del q2
    bi = torch.tensor([t // w.seq for t in toks], device="cuda")
    ti = torch.tensor([t % w.seq for t in toks], device="cuda")
    gq = to_np(q[bi, :, ti])     # [n, Hq, d]
    gk = to_np(kc[bi, :, ti])
    gv = to_np(vc[bi, :, ti])
    del q, kc, vc, d
    torch.cuda.empty_cache()
    xs = np.stack([h["x"][t // w.seq, t % w.seq] for t in toks])[None]  # [1, n, H]
    pos = np.array([[t % w.seq for t in toks]])
    rq, rk, rv = O.qkv_normrope(resolved(w), xs, h["w_qkv"], h["q_norm_w"], h["k_norm_w"], pos,
                                w.rope_theta, w.rms_eps, qk_norm=w.qk_norm)
    assert_close(gq, rq[0].transpose(1, 0, 2), w.dtype, "q")
    assert_close(gk, rk[0].transpose(1, 0, 2), w.dtype, "k")
    assert_close(gv, rv[0].transpose(1, 0, 2), w.dtype, "v")


def test_o_proj_h4096_every_element():
    """gqa_o_proj at the 4096-wide size: [32768, 4096] x [4096, 4096]^T, 2048
    tiles (eight per workgroup), every element, on a seeded bf16 activation."""
    T = T_()
    w = GI.WORKLOADS["quotient_h4096"]
    announce("[full size] o_proj 32768 x 4096 x 4096 every element")
    rng = np.random.default_rng(77)
    o = GI.round_bf16(rng.standard_normal((w.batch * w.seq, w.hq * w.d), dtype=np.float32))
    wo = GI.host_layer_inputs(w.with_(batch=1, seq=1))["w_o"]
    d = GI.to_device({"o": o, "w_o": wo}, w)
    out = T.gqa_o_proj(cfg_of(w), d["o"], d["w_o"])
    out2 = T.gqa_o_proj(cfg_of(w), d["o"], d["w_o"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "repeat call differs"
    got = to_np(out)
    del out, out2, d
    torch.cuda.empty_cache()
    assert_close(got, O.project(o, wo), w.dtype, "o_proj")


@pytest.mark.parametrize("name", ["decode_h2560_gqa", "decode_h2560_mqa"])
def test_decode_full_size(name):
    """Full-size decode (64 sequences against 32768-token caches) in the
    bench's launch configuration on 4 sampled sequences, plus the appended
    k, v rows; a second identical step must be bitwise identical (the
    append rewrites the same row)."""
    w = GI.WORKLOADS[name]
    seqs = [0, 21, 37, 63]
    announce(f"[full size] {name} B={w.batch} cache={w.cache_len} sequences={seqs}")
    h = GI.host_layer_inputs(w)
    d = GI.to_device(h, w)
    cache = GI.device_cache(w)
    # host copies of the sampled sequences' caches, taken before the call
    kc_h = cache["k_cache"][seqs].float().cpu().numpy()
    vc_h = cache["v_cache"][seqs].float().cpu().numpy()
    cl = torch.full((w.batch,), w.cache_len, dtype=torch.int32, device="cuda")
    out, kc, vc = layer(w, d, k_cache=cache["k_cache"], v_cache=cache["v_cache"], cache_len=cl)
    out2, _, _ = layer(w, d, k_cache=cache["k_cache"], v_cache=cache["v_cache"], cache_len=cl)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "repeat decode step differs"
    got = to_np(out[seqs])
    new_k = to_np(kc[seqs][:, :, w.cache_len])
    new_v = to_np(vc[seqs][:, :, w.cache_len])
    del cache, kc, vc, out, out2
    torch.cuda.empty_cache()
    ref, rk, rv = O.layer_forward(resolved(w), h["x"][seqs], h["w_qkv"], h["q_norm_w"],
                                  h["k_norm_w"], h["w_o"], rope_theta=w.rope_theta,
                                  rms_eps=w.rms_eps, qk_norm=w.qk_norm, k_cache=kc_h,
                                  v_cache=vc_h, cache_len=np.full(len(seqs), w.cache_len),
                                  dtype=np.float32)
    assert_close(new_k, rk[:, :, w.cache_len], w.dtype, "appended k")
    assert_close(new_v, rv[:, :, w.cache_len], w.dtype, "appended v")
    assert_close(got, ref, w.dtype, "sampled sequences")


def test_gemma_d256_rows():
    """The head_dim-256 prefill (separate norm/RoPE pass) on 256 rows of
    every sequence."""
    w = GI.WORKLOADS["gemma_h640_d256"]
    trows = sampled_rows(w.seq)
    rows = [(b, t) for b in range(w.batch) for t in trows]
    announce(f"[full size] {w.name} {len(rows)} rows")
    h = GI.host_layer_inputs(w)
    d = GI.to_device(h, w)
    out, _, _ = layer(w, d)
    torch.cuda.synchronize()
    idx_b = torch.tensor([b for b, _ in rows], device="cuda")
    idx_t = torch.tensor([t for _, t in rows], device="cuda")
    got = to_np(out[idx_b, idx_t])
    ref = O.layer_forward_rows(resolved(w), h["x"], h["w_qkv"], h["q_norm_w"], h["k_norm_w"],
                               h["w_o"], rows, rope_theta=w.rope_theta, rms_eps=w.rms_eps,
                               qk_norm=w.qk_norm, rotary_dim=w.rotary_dim, dtype=np.float32)
    assert_close(got, ref, w.dtype, "sampled rows")


def test_sampling_helpers():
    """The row and tile samplers cover what they claim."""
    r = sampled_rows(16384)
    assert len(r) == 256 and r[:64] == list(range(64)) and r[-1] == 16383
    assert len(set(r)) == 256
    toks = tile_tokens(32768)
    assert {t // 256 for t in toks} == set(range(128)) and toks[-1] == 32767
