"""GPU checks of the fused-Q path and of wider head counts: attention that
normalises and rotates raw Q in its prologue must equal the separate norm +
rotary pass followed by attention bit for bit, and both must match the fp64
oracle; H = 56 heads through the whole chain."""
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


def unfused_and_fused(w, T, kv_heads=None):
    """(o unfused, o fused, k' unfused, k' single-tensor pass, table, cu) for workload w."""
    import torch

    q, k, v = (to_device(x, w.dtype) for x in (T.q, T.k, T.v))
    q0 = q.clone()
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, w.tokens, max(w.rot_dim // 2, 1)), dtype=torch.float32, device="cuda")
    cu = h3a().build_rope_table_ex(w.segments, w.rope_mode, w.rot_dims, w.base, tab)
    qn, kn = torch.empty_like(q), torch.empty_like(k)
    h3a().qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim, q_out=qn, k_out=kn)
    o_ref = h3a().varlen_attn_fwd_ex(qn, kn, v, cu, w.scale)
    kn2 = h3a().rmsnorm_rope(k, gk, w.eps, tab, w.rot_dim, x_out=torch.empty_like(k))
    o_fused = h3a().varlen_attn_fwd_qnorm(q, kn2, v, cu, w.scale, gq, w.eps, tab, w.rot_dim)
    torch.cuda.synchronize()
    assert torch.equal(q, q0), "the fused path modified q"
    return o_ref, o_fused, kn, kn2, qn, cu


CASES = {
    # name: (workload, kv heads)
    "h3_s20423": (configs.H3_S20423, 24),
    "two_seg_gqa": (configs.TWO_SEG, 8),
    "vit3d_d64_r48_as_r64": (configs.VIT3D_TILES.replace(rot_dims=(32, 16, 16)), 32),
    "d64_r32": (configs.TINY_F32.replace(dtype="bf16", rot_dims=(16, 8, 8)), 2),
    "d128_r128": (configs.TWO_SEG.replace(rot_dims=(64, 32, 32), segments=((2, 16, 16, 512), (1, 9, 13, 117))), 24),
    "d128_r0": (configs.TWO_SEG.replace(rot_dims=(0, 0, 0), segments=((1, 300, 1, 300),)), 24),
    "d128_r32": (configs.TWO_SEG.replace(rot_dims=(0, 16, 16), segments=((1, 20, 30, 600), (1, 1, 1, 1))), 24),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_q_equals_unfused_bitwise(name):
    import torch

    w, hkv = CASES[name]
    w = w.replace(kv_heads=hkv)
    T = configs.make_tensors(w)
    log(f"[fused q] {name} S={w.tokens} Hq={w.heads} Hkv={w.kv} D={w.head_dim} R={w.rot_dim}")
    o_ref, o_fused, kn, kn2, qn, cu = unfused_and_fused(w, T)
    assert torch.equal(kn, kn2), "single-tensor norm + rotary differs from the k half of the fused pair"
    diff = (o_ref.float() - o_fused.float()).abs().max().item()
    log(f"  max |fused - unfused| = {diff:.3e}")
    assert torch.equal(o_ref, o_fused)
    # and the fused output against the oracle (from the GPU's own q', k')
    og = to_f64(o_fused)
    rows = sample_rows(cu, every=211)
    args = (to_f64(qn), to_f64(kn), rng.as_f64(T.v, w.dtype), cu, w.scale, rows)
    ref = oracle.varlen_attention_rows(*args) if w.kv == w.heads else oracle.varlen_attention_gqa_rows(*args)
    compare(og[rows], ref, w.dtype, f"o fused vs oracle ({len(rows)} rows)")


def test_56_heads_chain():
    """56 heads (the shipped DiT's head count) through table -> norm + rotary -> attention."""
    import torch

    w = configs.TWO_SEG.replace(heads=56, name="two_seg_h56")
    T = configs.make_tensors(w)
    log(f"[56 heads] S={w.tokens} H={w.heads}")
    o_ref, o_fused, kn, _, qn, cu = unfused_and_fused(w, T)
    assert torch.equal(o_ref, o_fused)
    qf, kf, vf = (rng.as_f64(x, w.dtype) for x in (T.q, T.k, T.v))
    ocu, cos, sin = oracle.rope_table(w.segments, w.rot_dims, w.base)
    qn_o, kn_o = oracle.qk_rmsnorm_rope(qf, kf, T.gamma_q, T.gamma_k, w.eps, cos, sin, w.rot_dim)
    compare(to_f64(qn), qn_o, w.dtype, "q'")
    compare(to_f64(kn), kn_o, w.dtype, "k'")
    rows = sample_rows(ocu, every=97)
    compare(to_f64(o_ref)[rows], oracle.varlen_attention_rows(qn_o, kn_o, vf, ocu, w.scale, rows), w.dtype,
            f"o end to end ({len(rows)} rows)")


def test_fused_qkv_buffer_views_in_place():
    """q, k, v as views of one [S, 3, H, D] buffer (the fused qkv GEMM output): in-place norm +
    rotary on the q and k views, attention on the views; the v view and the guard columns of
    a padded row stay untouched."""
    import torch

    w = configs.TWO_SEG
    T = configs.make_tensors(w)
    S, H, D = w.tokens, w.heads, w.head_dim
    buf = torch.full((S, 3 * H * D + 64), -1024.0, dtype=torch.bfloat16, device="cuda")
    qv = buf[:, :H * D].view(S, H, D)
    kv = buf[:, H * D:2 * H * D].view(S, H, D)
    vv = buf[:, 2 * H * D:3 * H * D].view(S, H, D)
    for view, x in ((qv, T.q), (kv, T.k), (vv, T.v)):
        view.copy_(to_device(x, "bf16"))
    v_before = vv.clone()
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, S, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    cu = h3a().build_rope_table(w.segments, w.rot_dims, w.base, tab)
    h3a().qk_rmsnorm_rope(qv, kv, gq, gk, w.eps, tab, w.rot_dim)
    o = h3a().varlen_attn_fwd(qv, kv, vv, cu, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(vv, v_before)
    assert torch.all(buf[:, 3 * H * D:] == -1024.0)
    # the same chain on separate contiguous tensors gives the same bits
    q, k, v = (to_device(x, "bf16") for x in (T.q, T.k, T.v))
    h3a().qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim)
    o2 = h3a().varlen_attn_fwd(q, k, v, cu, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(qv, q) and torch.equal(kv, k) and torch.equal(o, o2)
