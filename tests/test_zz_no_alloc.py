"""gqa_layer_forward_noalloc (the layer forward whose workspace is the
library's static device scratch) against gqa_layer_forward with a caller
workspace: the same kernels, so the outputs and the appended cache rows
must be bitwise identical.  Two calls in a row, the second smaller, so the
second runs on scratch that still holds the first call's data; and a call
that needs more scratch than the library holds is rejected on the host."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gqa_inputs as GI  # noqa: E402
from gpu_util import announce, assert_close, cfg_of, oracle_layer, to_np  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_attention_layer_amd as T
    T.lib()
    yield


def _both(w, cache_len):
    """Run the layer on identical inputs through both entry points, each on
    its own copy of the caches; returns (noalloc results, workspace results,
    host inputs, host caches)."""
    import transformer_attention_layer_amd as T
    h = GI.host_layer_inputs(w)
    d = GI.to_device(h, w)
    cache = GI.host_cache(w, fill_unused=0.0)
    cfg = cfg_of(w)
    cl = torch.tensor(cache_len, dtype=torch.int32, device="cuda")
    res = []
    for noalloc in (True, False):
        c = GI.to_device(cache, w)
        f = T.gqa_layer_forward_noalloc if noalloc else T.gqa_layer_forward
        out, kc, vc = f(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"], d["w_o"],
                        k_cache=c["k_cache"], v_cache=c["v_cache"], cache_len=cl)
        torch.cuda.synchronize()
        res.append((out, kc, vc))
    return res[0], res[1], h, cache


def test_noalloc_matches_workspace_entry_point_twice():
    big = GI.WORKLOADS["decode_h2560_gqa"].with_(batch=16, cache_len=9000)
    small = GI.WORKLOADS["decode_h2560_mqa"].with_(batch=3, seq=2, cache_len=700, seed=9)
    for i, (w, cl) in enumerate(((big, [9000] * 16), (small, [700, 0, 311]))):
        announce(f"[noalloc] call {i + 1}: {w.name} B={w.batch} L={w.seq} cache={cl}")
        (a, ka, va), (b, kb, vb), h, cache = _both(w, cl)
        assert torch.equal(a, b), f"call {i + 1}: output differs from gqa_layer_forward"
        assert torch.equal(ka, kb) and torch.equal(va, vb), f"call {i + 1}: cache differs"
        ref, _, _ = oracle_layer(w, h, cache, np.array(cl))
        assert_close(to_np(a), ref, w.dtype, f"call {i + 1} vs oracle")


def test_noalloc_prefill_chunk_then_decode():
    """A short prefill into the caches, then one decode step, both without a
    workspace, against the same two calls with one."""
    import transformer_attention_layer_amd as T
    w = GI.WORKLOADS["prefill_h1024"].with_(batch=2, seq=300)
    announce("[noalloc] prefill 2x300 then decode")
    h = GI.host_layer_inputs(w)
    d = GI.to_device(h, w)
    cfg = cfg_of(w)
    outs = []
    for f in (T.gqa_layer_forward_noalloc, T.gqa_layer_forward):
        kc = torch.zeros((2, w.hkv, 301, 128), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        z = torch.zeros(2, dtype=torch.int32, device="cuda")
        o1, _, _ = f(cfg, d["x"], d["w_qkv"], d["q_norm_w"], d["k_norm_w"], d["w_o"],
                     k_cache=kc, v_cache=vc, cache_len=z)
        o2, _, _ = f(cfg, d["x"][:, :1].contiguous(), d["w_qkv"], d["q_norm_w"], d["k_norm_w"],
                     d["w_o"], k_cache=kc, v_cache=vc, cache_len=z + 300)
        torch.cuda.synchronize()
        outs.append((o1.clone(), o2.clone(), kc.clone()))
    for x, y in zip(outs[0], outs[1]):
        assert torch.equal(x, y)


def test_noalloc_rejects_calls_beyond_its_scratch():
    import transformer_attention_layer_amd as T
    w = GI.WORKLOADS["prefill_h1024"].with_(batch=8, seq=2048)
    announce("[noalloc] a call beyond the static scratch is rejected")
    cfg = cfg_of(w)
    need = T.gqa_workspace_bytes(cfg, w.batch, w.seq, w.seq, T.WS_LAYER)
    assert need > (32 << 20)
    x = torch.zeros((w.batch, w.seq, w.hidden), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros(((w.hq + 2 * w.hkv) * 128, w.hidden), dtype=torch.bfloat16, device="cuda")
    nw = torch.ones(128, dtype=torch.bfloat16, device="cuda")
    wo = torch.zeros((w.hidden, w.hq * 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((w.batch, w.hkv, w.seq, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    with pytest.raises(T.GQAError, match="GQA_ERR_WORKSPACE_TOO_SMALL"):
        T.gqa_layer_forward_noalloc(cfg, x, wq, nw, nw, wo, k_cache=kc, v_cache=vc)
