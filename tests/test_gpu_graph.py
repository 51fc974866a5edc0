"""The norm + rotary pass and the attention can be captured in a HIP graph once
the tile plan for the packing is cached: every launch goes to the caller's
stream, nothing is allocated or copied at call time.  Each replay must give the
eager bytes, also after the inputs are overwritten between replays (the graph
reads the buffers' current contents) and with unrelated eager work and
synchronisation in between."""
from __future__ import annotations

import numpy as np
import pytest

from synth import configs, rng
from tests.gpu_util import log, require_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()


@pytest.mark.parametrize("mode", ["bf16", "fp8", "i8", "i8pv"])
def test_capture_and_replay(mode):
    import torch

    import packed_varlen_attention_head_amd as h3a

    w = configs.BF16["two_seg_bf16"]
    S, H, D = w.tokens, w.heads, w.head_dim
    log(f"[graph] {w.name} {mode}")
    tab = torch.empty((2, S, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    cu = h3a.build_rope_table(w.segments, w.rot_dims, w.base, tab)
    gq = torch.from_numpy((1.0 + 0.1 * rng.normal(71, rng.TAG_GAMMA_Q, D)).astype(np.float32)).cuda()
    gk = torch.from_numpy((1.0 + 0.1 * rng.normal(71, rng.TAG_GAMMA_K, D)).astype(np.float32)).cuda()
    inputs = [tuple(to_device(rng.normal_tensor(71 + i, tag, (S, H, D), "bf16"), "bf16")
                    for tag in (rng.TAG_Q, rng.TAG_K, rng.TAG_V)) for i in range(2)]
    q, k, v = (torch.empty_like(x) for x in inputs[0])
    qo, ko, o = torch.empty_like(q), torch.empty_like(k), torch.empty_like(q)
    cols = h3a.vt_e4m3_columns(cu)
    q8 = (torch.empty(q.shape, dtype=torch.uint8, device="cuda"),
          torch.empty((H, S, D // 32), dtype=torch.uint8, device="cuda"))
    k8 = tuple(torch.empty_like(x) for x in q8)
    vt8 = (torch.empty((H, D, cols), dtype=torch.uint8, device="cuda"),
           torch.empty((H, cols // 64, 2, 32, D // 32), dtype=torch.uint8, device="cuda"))
    nb = h3a.i8_key_blocks(cu)
    qi8 = (torch.empty(q.shape, dtype=torch.int8, device="cuda"), torch.empty((H, S), dtype=torch.float32, device="cuda"))
    ki8 = (torch.empty(k.shape, dtype=torch.int8, device="cuda"), torch.empty((H, nb), dtype=torch.float32, device="cuda"))
    scale = w.scale

    def step(stream=None):
        if mode in ("i8", "i8pv"):
            h3a.qk_rmsnorm_rope_i8q(q, k, gq, gk, w.eps, tab, w.rot_dim, q8=qi8[0], q_scale=qi8[1], k_out=ko,
                                    stream=stream)
            h3a.quantize_i8_keys(ko, cu, out=ki8[0], scale_out=ki8[1], stream=stream)
            if mode == "i8":
                h3a.varlen_attn_fwd_i8qk(qi8, ki8, v, cu, scale, out=o, stream=stream)
            else:
                h3a.prepare_vt_e4m3(v, cu, out=vt8[0], scale_out=vt8[1], stream=stream)
                h3a.varlen_attn_fwd_i8qk_fp8pv(qi8, ki8, vt8, cu, scale, out=o, stream=stream)
        elif mode == "fp8":
            h3a.qk_rmsnorm_rope_e4m3(q, k, gq, gk, w.eps, tab, w.rot_dim, q8=q8[0], k8=k8[0], q_scale=q8[1],
                                     k_scale=k8[1], stream=stream)
            h3a.prepare_vt_e4m3(v, cu, out=vt8[0], scale_out=vt8[1], stream=stream)
            h3a.varlen_attn_fwd_fp8(q8, k8, vt8, cu, scale, out=o, stream=stream)
        else:
            h3a.qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim, q_out=qo, k_out=ko, stream=stream)
            h3a.varlen_attn_fwd(qo, ko, v, cu, scale, out=o, stream=stream)

    def load(i):
        for dst, src in zip((q, k, v), inputs[i]):
            dst.copy_(src)

    eager = []
    for i in range(2):
        load(i)
        step()
        torch.cuda.synchronize()
        eager.append(o.clone())
    assert not torch.equal(eager[0], eager[1])

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream: the plan is cached before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep, i in enumerate((0, 1, 1, 0)):
        load(i)
        o.fill_(float("nan"))  # eager work between replays; the replay must overwrite it
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(o, eager[i])
        log(f"  replay {rep} (inputs {i}): equal to eager = {same}")
        assert same


def test_captured_plan_survives_eviction():
    """A graph keeps the device address of the tile plan its attention launch
    read.  That plan must outlive cache evictions: capture, then run more distinct
    packings than the cache holds (256, each evicting the oldest unpinned plan),
    then replay -- still the eager bytes.  A call whose plan is not cached fails
    on a capturing stream (building one would allocate and synchronise) and
    leaves the capture usable."""
    import torch

    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()
    S, H, D = 1000, 2, 128
    cu = np.array([0, 300, 1000])
    q, k, v = (to_device(rng.normal_tensor(91, tag, (S, H, D), "bf16"), "bf16")
               for tag in (rng.TAG_Q, rng.TAG_K, rng.TAG_V))
    scale = 1.0 / np.sqrt(D)
    o = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        h3a.varlen_attn_fwd(q, k, v, cu, scale, out=o)  # caches the plan
    torch.cuda.synchronize()
    eager = o.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h3a.varlen_attn_fwd(q, k, v, cu, scale, out=o)
        with pytest.raises(RuntimeError, match="not cached"):
            h3a.varlen_attn_fwd(q, k, v, np.array([0, 301, 1000]), scale, out=o)
    torch.cuda.synchronize()

    # 300 other packings: every one a new plan, evicting the oldest unpinned ones
    tmp = torch.empty_like(q)
    for i in range(300):
        h3a.varlen_attn_fwd(q, k, v, np.array([0, 2 + i, 1000]), scale, out=tmp)
    torch.cuda.synchronize()
    log("[graph] 300 packings after capture; replaying")
    for rep in range(3):
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(o, eager)
        log(f"  replay {rep}: equal to eager = {same}")
        assert same
    del g
    torch.cuda.synchronize()
    h3a.release_caches()
