"""GPU parity of the encoder towers' attention workloads against the fp64 oracle:
causal grouped-query attention (text tower) through the whole chain on two
workloads, edge lengths around the tile sizes, GPU-side invariants (prefix
isolation, grouped heads equal to repeated K/V), and per-frame ragged ViT
attention (vision tower)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import configs, rng
from tests.gpu_util import compare, log, require_gpu, sample_rows, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()


def h3a():
    import packed_varlen_attention_head_amd as m

    return m


@pytest.mark.parametrize("name", sorted(configs.CAUSAL_WORKLOADS))
def test_causal_gqa_chain(name):
    import torch

    w = configs.CAUSAL_WORKLOADS[name]
    T = configs.make_tensors(w)
    log(f"[causal gqa chain] {name} S={w.tokens} Hq={w.heads} Hkv={w.kv} D={w.head_dim} {w.dtype}")
    q, k, v = (to_device(x, w.dtype) for x in (T.q, T.k, T.v))
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    cu = h3a().build_rope_table_ex(w.segments, w.rope_mode, w.rot_dims, w.base, tab)
    h3a().qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim)
    o = h3a().varlen_attn_fwd_ex(q, k, v, cu, w.scale, causal=True)
    torch.cuda.synchronize()
    qn_g, kn_g, og = to_f64(q), to_f64(k), to_f64(o)

    qf, kf, vf = (rng.as_f64(x, w.dtype) for x in (T.q, T.k, T.v))
    ocu, cos, sin = oracle.rope_table_mode(w.segments, w.rope_mode, w.rot_dims, w.base)
    assert np.array_equal(cu, ocu)
    qn, kn = oracle.qk_rmsnorm_rope(qf, kf, T.gamma_q, T.gamma_k, w.eps, cos, sin, w.rot_dim)
    compare(qn_g, qn, w.dtype, "q'")
    compare(kn_g, kn, w.dtype, "k'")
    if w.tokens <= 512:
        compare(og, oracle.varlen_attention_gqa(qn_g, kn_g, vf, ocu, w.scale, causal=True), w.dtype,
                "o (from the GPU's q', k')")
        compare(og, oracle.varlen_attention_gqa(qn, kn, vf, ocu, w.scale, causal=True), w.dtype, "o end to end")
    else:
        rows = sample_rows(ocu, every=11)
        ref = oracle.varlen_attention_gqa_rows(qn_g, kn_g, vf, ocu, w.scale, rows, causal=True)
        compare(og[rows], ref, w.dtype, f"o from the GPU's q', k' ({len(rows)} rows)")
        ref = oracle.varlen_attention_gqa_rows(qn, kn, vf, ocu, w.scale, rows, causal=True)
        compare(og[rows], ref, w.dtype, f"o end to end ({len(rows)} rows)")


EDGE_LENS = [1, 63, 64, 65, 127, 128, 129, 0, 255, 256, 257, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (6, 3), (2, 2)])
@pytest.mark.parametrize("causal", [True, False])
def test_gqa_edges(dtype, D, Hq, Hkv, causal):
    import torch

    cu = np.concatenate([[0], np.cumsum(EDGE_LENS)]).astype(np.int64)
    S = int(cu[-1])
    seed = 100 + D + 10 * Hq + Hkv + (1 if causal else 0)
    log(f"[gqa edges] dtype={dtype} D={D} Hq={Hq} Hkv={Hkv} causal={causal} S={S} seed={seed}")
    qb = rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), dtype)
    kb = rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), dtype, 0.0, 0.5)
    vb = rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), dtype)
    q, k, v = (to_device(x, dtype) for x in (qb, kb, vb))
    scale = 1.0 / np.sqrt(D)
    o = to_f64(h3a().varlen_attn_fwd_ex(q, k, v, cu, scale, causal=causal))
    ref = oracle.varlen_attention_gqa(*(rng.as_f64(x, dtype) for x in (qb, kb, vb)), cu, scale, causal=causal)
    compare(o, ref, dtype, "o")


def test_causal_prefix_isolation_and_repeated_kv():
    """On the GPU: perturbing token i leaves every earlier output row bit-identical, and
    non-causal grouped heads equal plain multi-head attention on repeated K/V bit for bit."""
    import torch

    lens = [700, 300]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S, Hq, Hkv, D = 1000, 8, 2, 128
    qb = rng.normal_tensor(7, rng.TAG_Q, (S, Hq, D), "bf16")
    kb = rng.normal_tensor(7, rng.TAG_K, (S, Hkv, D), "bf16")
    vb = rng.normal_tensor(7, rng.TAG_V, (S, Hkv, D), "bf16")
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    o = h3a().varlen_attn_fwd_ex(q, k, v, cu, 0.088, causal=True)
    for t in (k, v):
        t2 = t.clone()
        t2[400] += 1.0
        args = (q, t2, v) if t is k else (q, k, t2)
        o2 = h3a().varlen_attn_fwd_ex(*args, cu, 0.088, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o2[:400], o[:400])
        assert torch.equal(o2[700:], o[700:])
        assert not torch.equal(o2[400:700], o[400:700])
    g = Hq // Hkv
    kr = k.repeat_interleave(g, dim=1).contiguous()
    vr = v.repeat_interleave(g, dim=1).contiguous()
    for causal in (False, True):
        a = h3a().varlen_attn_fwd_ex(q, k, v, cu, 0.088, causal=causal)
        b = h3a().varlen_attn_fwd_ex(q, kr, vr, cu, 0.088, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(a, b), causal
    # the bidirectional grouped call with Hkv == Hq is the plain entry point
    a = h3a().varlen_attn_fwd_ex(q, kr, vr, cu, 0.088, causal=False)
    b = h3a().varlen_attn_fwd(q, kr, vr, cu, 0.088)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_per_frame_ragged_vit_attention():
    """Per-frame cu_seqlens over a ragged two-image batch, 2-D rotary table, bidirectional."""
    import torch

    w = configs.VISION_FRAMES
    T = configs.make_tensors(w)
    log(f"[vision frames] S={w.tokens} H={w.heads} D={w.head_dim} segments={w.lengths}")
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    cu = h3a().build_rope_table(w.segments, w.rot_dims, w.base, tab)
    q, k, v = (to_device(x, w.dtype) for x in (T.q, T.k, T.v))
    o = to_f64(h3a().varlen_attn_fwd(q, k, v, cu, w.scale))
    ocu, cos, sin = oracle.rope_table(w.segments, w.rot_dims, w.base)
    g = to_f64(tab)
    assert max(np.abs(g[0] - cos).max(), np.abs(g[1] - sin).max()) <= 1.2e-7
    qf, kf, vf = (rng.as_f64(x, w.dtype) for x in (T.q, T.k, T.v))
    compare(o, oracle.varlen_attention(qf, kf, vf, ocu, w.scale), w.dtype, "o")
