"""GPU parity of split plans: attention items whose keys are cut into ranges of
whole 64-key tiles, each range storing partial rows that a merge kernel
combines.  With the split policy forced on, every item of four or more key
tiles is cut into about three ranges (some of one tile, some crossing the
steady loop), so edge packings, grouped K/V, D = 64 and 128, the fused Q norm
and both FP8 kernels all run through the split path and are compared with the
oracle; determinism, streams, concurrent calls sharing one plan's workspace
and graph capture (which must use the plan's unsplit items) are checked too."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import configs, rng
from tests.gpu_util import compare, log, require_gpu, sample_rows, to_device, to_f64

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 63, 64, 65, 127, 128, 129, 0, 255, 256, 257, 700, 3000]


def h3a():
    import packed_varlen_attention_head_amd as m

    return m


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    h3a().release_caches()
    h3a().set_split_policy(h3a().H3A_SPLIT_ALWAYS)
    yield
    h3a().set_split_policy(h3a().H3A_SPLIT_AUTO)
    h3a().release_caches()


def inputs(seed, lens, Hq, Hkv, D):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S = int(cu[-1])
    q = rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), "bf16")
    k = rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), "bf16")
    v = rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), "bf16")
    return cu, q, k, v


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (6, 2)])
def test_split_bf16_vs_oracle(D, Hq, Hkv):
    cu, q, k, v = inputs(900 + D + Hq, EDGE_LENS, Hq, Hkv, D)
    log(f"[split bf16] D={D} Hq={Hq} Hkv={Hkv} S={int(cu[-1])}")
    scale = 1.0 / np.sqrt(D)
    o = h3a().varlen_attn_fwd_ex(*(to_device(x, "bf16") for x in (q, k, v)), cu, scale)
    ref = oracle.varlen_attention_gqa(*(rng.as_f64(x, "bf16") for x in (q, k, v)), cu, scale)
    compare(to_f64(o), ref, "bf16", "o (split plan)")


def test_split_determinism_streams_and_concurrent_calls():
    """Bitwise equal across runs and streams; two streams issuing calls with the
    same packing back to back (sharing the plan's partial workspace) both stay
    correct."""
    import torch

    lens = [3000, 700, 257]
    cu, q, k, v = inputs(911, lens, 4, 4, 128)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    a = h3a().varlen_attn_fwd(qd, kd, vd, cu, 0.088)
    b = h3a().varlen_attn_fwd(qd, kd, vd, cu, 0.088)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    q2 = to_device(rng.normal_tensor(912, rng.TAG_Q, q.shape, "bf16"), "bf16")
    torch.cuda.synchronize()
    outs = []
    for i in range(6):  # interleaved, no host synchronisation in between
        s = s1 if i % 2 == 0 else s2
        with torch.cuda.stream(s):
            outs.append(h3a().varlen_attn_fwd(qd if i % 2 == 0 else q2, kd, vd, cu, 0.088, stream=s))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    for i, o in enumerate(outs):
        assert torch.equal(o, a if i % 2 == 0 else outs[1]), i
    ref2 = oracle.varlen_attention(*(rng.as_f64(x, "bf16") for x in (rng.normal_tensor(912, rng.TAG_Q, q.shape,
                                                                                          "bf16"), k, v)), cu, 0.088)
    compare(to_f64(outs[1]), ref2, "bf16", "o, second stream's input")
    compare(to_f64(a), oracle.varlen_attention(*(rng.as_f64(x, "bf16") for x in (q, k, v)), cu, 0.088), "bf16",
            "o, first stream's input")


def test_split_fused_q_norm():
    import torch

    D, H, R = 128, 2, 96
    lens = [3000, 129, 700]
    cu, q, k, v = inputs(921, lens, H, H, D)
    S = int(cu[-1])
    log(f"[split fused q] S={S}")
    segs = [(1, 1, L, L) for L in lens]
    tab = torch.empty((2, S, R // 2), dtype=torch.float32, device="cuda")
    h3a().build_rope_table(segs, (32, 32, 32), 10000.0, tab)
    g = (1.0 + 0.1 * rng.normal(921, rng.TAG_GAMMA_Q, D)).astype(np.float32)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o = to_f64(h3a().varlen_attn_fwd_qnorm(qd, kd, vd, cu, 1.0 / np.sqrt(D), torch.from_numpy(g).cuda(), 1e-6, tab, R))
    ocu, cos, sin = oracle.rope_table(segs, (32, 32, 32), 10000.0)
    qn = oracle.rope_rotate(oracle.rms_norm(rng.as_f64(q, "bf16"), g, 1e-6), cos, sin, R)
    # the kernel rounds the normalised q to bf16 before the product, as the unfused pass stores it
    ref = oracle.varlen_attention(oracle.bf16_round(qn), rng.as_f64(k, "bf16"), rng.as_f64(v, "bf16"), ocu,
                                  1.0 / np.sqrt(D))
    compare(o, ref, "bf16", "o (split, fused q norm)")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode", ["fp8qk", "fp8"])
def test_split_fp8(mode, D):
    from tests.test_gpu_fp8 import TOL_FP8PV_MEANREL, check, gpu_fp8, gpu_fp8qk, mx_operands, weight_rounding_bound

    cu, q, k, v = inputs(931 + D, EDGE_LENS, 4, 2, D)
    log(f"[split {mode}] D={D} S={int(cu[-1])}")
    scale = 1.0 / np.sqrt(D)
    if mode == "fp8qk":
        o = to_f64(gpu_fp8qk(q, k, v, cu, scale))
        qf, kf, vf = (rng.as_f64(x, "bf16") for x in (q, k, v))
        compare(o, oracle.varlen_attention_mx_qk(qf, kf, vf, cu, scale), "bf16", "o (split, fp8 scores)")
        return
    o = to_f64(gpu_fp8(q, k, v, cu, scale))
    bound, ref = weight_rounding_bound(*mx_operands(q, k, v, cu), cu, scale)
    check(o, ref, "o (split, fp8 both)", bound, TOL_FP8PV_MEANREL)


def test_split_plan_not_used_under_capture():
    """A captured call uses the cached plan's unsplit items: its replays equal an
    eager call under the never-split policy bit for bit, and equal the oracle."""
    import torch

    lens = [3000, 700]
    cu, q, k, v = inputs(941, lens, 2, 2, 128)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o = torch.empty_like(qd)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        h3a().varlen_attn_fwd(qd, kd, vd, cu, 0.1, out=o, stream=side)  # caches the (split) plan
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    split_eager = o.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h3a().varlen_attn_fwd(qd, kd, vd, cu, 0.1, out=o)
    h3a().set_split_policy(h3a().H3A_SPLIT_NEVER)
    try:
        plain = h3a().varlen_attn_fwd(qd, kd, vd, cu, 0.1)
    finally:
        h3a().set_split_policy(h3a().H3A_SPLIT_ALWAYS)
    for i in range(3):
        o.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, plain), i
        h3a().varlen_attn_fwd(qd, kd, vd, cu, 0.1)  # eager split calls between replays
    del g
    ref = oracle.varlen_attention(*(rng.as_f64(x, "bf16") for x in (q, k, v)), cu, 0.1)
    compare(to_f64(plain), ref, "bf16", "o (unsplit items)")
    compare(to_f64(split_eager), ref, "bf16", "o (split items)")


def test_split_causal_is_unsplit_and_correct():
    """Causal plans are never split (their items already cost what their rows see)."""
    cu, q, k, v = inputs(951, [700, 3000, 65], 4, 2, 128)
    o = h3a().varlen_attn_fwd_ex(*(to_device(x, "bf16") for x in (q, k, v)), cu, 0.088, causal=True)
    ref = oracle.varlen_attention_gqa(*(rng.as_f64(x, "bf16") for x in (q, k, v)), cu, 0.088, causal=True)
    compare(to_f64(o), ref, "bf16", "o (causal)")


def test_auto_split_headline_share():
    """The automatic policy on the S = 20,423 packing with three heads (one GPU's
    share of 24 heads over eight): the 16,200-token segment's items are split
    (see the planner test); sampled rows against the oracle."""
    h3a().set_split_policy(h3a().H3A_SPLIT_AUTO)
    try:
        w = configs.ALL["h3_s20423_bf16"].replace(heads=3)
        T = configs.make_tensors(w)
        log(f"[auto split] {w.name} heads=3 S={w.tokens}")
        cu = oracle.cu_seqlens(w.segments)
        q, k, v = (to_device(x, "bf16") for x in (T.q, T.k, T.v))
        o = to_f64(h3a().varlen_attn_fwd(q, k, v, cu, w.scale))
        rows = sample_rows(cu, every=53)
        ref = oracle.varlen_attention_rows(*(rng.as_f64(x, "bf16") for x in (T.q, T.k, T.v)), cu, w.scale, rows)
        compare(o[rows], ref, "bf16", f"o ({len(rows)} rows)")
    finally:
        h3a().set_split_policy(h3a().H3A_SPLIT_ALWAYS)
