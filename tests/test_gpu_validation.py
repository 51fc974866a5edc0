"""The binding refuses, by name and before anything is launched, tensors whose
shape, dtype or device would make a kernel read or write outside them: the
gains, the rotary table, caller-provided outputs, E4M3 codes and the
transposed V layout.  Each refused call leaves its destination untouched."""
from __future__ import annotations

import numpy as np
import pytest

from tests.gpu_util import log, require_gpu

pytestmark = pytest.mark.gpu

LENS = [100, 37]
H, D, R = 2, 128, 96


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()


def setup():
    import torch

    import packed_varlen_attention_head_amd as h3a

    S = sum(LENS)
    g = torch.Generator(device="cpu").manual_seed(0)
    q, k, v = (torch.randn(S, H, D, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    tab = torch.empty((2, S, R // 2), dtype=torch.float32, device="cuda")
    cu = h3a.build_rope_table([(1, 1, L, L) for L in LENS], (32, 32, 32), 10000.0, tab)
    gam = torch.ones(D, dtype=torch.float32, device="cuda")
    return h3a, q, k, v, tab, cu, gam


def refused(fn, status, *untouched):
    import torch

    import packed_varlen_attention_head_amd as h3a

    before = [t.clone() for t in untouched]
    with pytest.raises(h3a.H3AError) as e:
        fn()
    torch.cuda.synchronize()
    log(f"  refused: {e.value}")
    assert e.value.status == status
    for t, b in zip(untouched, before):
        assert torch.equal(t, b)


def test_gains_and_table():
    import torch

    h3a, q, k, v, tab, cu, gam = setup()
    qo, ko = torch.zeros_like(q), torch.zeros_like(k)
    run = lambda gq, gk, t: h3a.qk_rmsnorm_rope(q, k, gq, gk, 1e-6, t, R, q_out=qo, k_out=ko)  # noqa: E731
    refused(lambda: run(gam[:64], gam, tab), h3a.H3A_ESHAPE, qo, ko)
    refused(lambda: run(gam, gam.to(torch.bfloat16), tab), h3a.H3A_EDTYPE, qo, ko)
    refused(lambda: run(gam.cpu(), gam, tab), h3a.H3A_EINVAL, qo, ko)
    refused(lambda: run(gam, gam, tab[:, :-1]), h3a.H3A_ESHAPE, qo, ko)
    refused(lambda: run(gam, gam, tab[:, :, :32]), h3a.H3A_ESHAPE, qo, ko)
    refused(lambda: run(gam, gam, tab.double()), h3a.H3A_EDTYPE, qo, ko)
    refused(lambda: h3a.rmsnorm_rope(q, gam[:-1], 1e-6, tab, R, x_out=qo), h3a.H3A_ESHAPE, qo)
    refused(lambda: h3a.varlen_attn_fwd_qnorm(q, k, v, cu, 0.1, gam, 1e-6, tab[:, :, :16], R), h3a.H3A_ESHAPE)
    bad = torch.zeros((2, sum(LENS) + 1, R // 2), dtype=torch.float32, device="cuda")
    refused(lambda: h3a.build_rope_table([(1, 1, L, L) for L in LENS], (32, 32, 32), 1e4, bad), h3a.H3A_ESHAPE, bad)
    # the valid call still runs
    run(gam, gam, tab)
    torch.cuda.synchronize()
    assert torch.isfinite(qo.float()).all()


def test_attention_outputs():
    import torch

    h3a, q, k, v, tab, cu, gam = setup()
    S = q.shape[0]
    small = torch.zeros((S - 1, H, D), dtype=torch.bfloat16, device="cuda")
    refused(lambda: h3a.varlen_attn_fwd(q, k, v, cu, 0.1, out=small), h3a.H3A_ESHAPE, small)
    f32 = torch.zeros((S, H, D), dtype=torch.float32, device="cuda")
    refused(lambda: h3a.varlen_attn_fwd(q, k, v, cu, 0.1, out=f32), h3a.H3A_ESHAPE, f32)
    refused(lambda: h3a.varlen_attn_fwd_ex(q, k, v, cu, 0.1, causal=True, out=small), h3a.H3A_ESHAPE, small)
    o = h3a.varlen_attn_fwd(q, k, v, cu, 0.1)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()


def test_fp8_operands():
    import torch

    h3a, q, k, v, tab, cu, gam = setup()
    S = q.shape[0]
    q8, k8 = h3a.quantize_e4m3(q), h3a.quantize_e4m3(k)
    cols = h3a.vt_e4m3_columns(cu)
    assert cols == sum(-(-L // 64) * 64 for L in LENS)
    wide = torch.zeros((H, D, cols + 64), dtype=torch.uint8, device="cuda")
    refused(lambda: h3a.prepare_vt_e4m3(v, cu, out=wide), h3a.H3A_ESHAPE, wide)
    refused(lambda: h3a.prepare_vt_e4m3(v.float(), cu), h3a.H3A_EDTYPE)
    vt8 = h3a.prepare_vt_e4m3(v, cu)
    out = torch.zeros((S, H, D), dtype=torch.bfloat16, device="cuda")
    refused(lambda: h3a.varlen_attn_fwd_fp8(q8, k8, (vt8[0][:, :, :-64].contiguous(), vt8[1]), cu, 0.1, out=out),
            h3a.H3A_ESHAPE, out)
    refused(lambda: h3a.varlen_attn_fwd_fp8(q8, k8, vt8, cu, 0.1, out=out[:-1]), h3a.H3A_ESHAPE, out)
    refused(lambda: h3a.varlen_attn_fwd_fp8((q.view(torch.uint8)[:, :, :D].contiguous().view(torch.int8), q8[1]), k8,
                                            vt8, cu, 0.1, out=out), h3a.H3A_EDTYPE, out)
    refused(lambda: h3a.varlen_attn_fwd_fp8qk(q8, k8, v, cu, 0.1, out=out[:, :1]), h3a.H3A_ESHAPE, out)
    q8o = torch.zeros((S - 1, H, D), dtype=torch.uint8, device="cuda")
    refused(lambda: h3a.qk_rmsnorm_rope_e4m3(q, k, gam, gam, 1e-6, tab, R, q8=q8o), h3a.H3A_ESHAPE, q8o)
    # scale arrays: exact packed shapes, uint8, contiguous; operands as (codes, scales) pairs
    qs_short = torch.zeros((H, S, D // 32 - 1), dtype=torch.uint8, device="cuda")
    refused(lambda: h3a.varlen_attn_fwd_fp8qk((q8[0], qs_short), k8, v, cu, 0.1, out=out), h3a.H3A_ESHAPE, out)
    refused(lambda: h3a.varlen_attn_fwd_fp8qk((q8[0], q8[1].view(torch.int8)), k8, v, cu, 0.1, out=out),
            h3a.H3A_EDTYPE, out)
    vs_strided = torch.zeros(vt8[1].shape[:-1] + (2 * (D // 32),), dtype=torch.uint8, device="cuda")[..., ::2]
    refused(lambda: h3a.varlen_attn_fwd_fp8(q8, k8, (vt8[0], vs_strided), cu, 0.1, out=out), h3a.H3A_ESHAPE, out)
    refused(lambda: h3a.varlen_attn_fwd_fp8(q8[0], k8, vt8, cu, 0.1, out=out), h3a.H3A_EINVAL, out)
    refused(lambda: h3a.quantize_e4m3(q, scale_out=qs_short), h3a.H3A_ESHAPE)
    refused(lambda: h3a.prepare_vt_e4m3(v, cu, scale_out=vt8[1][:, :-1].contiguous()), h3a.H3A_ESHAPE)
    o = h3a.varlen_attn_fwd_fp8(q8, k8, vt8, cu, 0.1, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    assert np.isfinite(o.float().cpu().numpy()).all()


def test_int8_operands():
    import torch

    h3a, q, k, v, tab, cu, gam = setup()
    S = q.shape[0]
    nb = h3a.i8_key_blocks(cu)
    assert nb == sum(-(-L // 64) for L in LENS)
    qi8, ki8 = h3a.quantize_i8_rows(q), h3a.quantize_i8_keys(k, cu)
    out = torch.zeros((S, H, D), dtype=torch.bfloat16, device="cuda")
    refused(lambda: h3a.quantize_i8_rows(q.float()), h3a.H3A_EDTYPE)
    refused(lambda: h3a.quantize_i8_rows(q, scale_out=torch.zeros((H, S - 1), device="cuda")), h3a.H3A_ESHAPE)
    refused(lambda: h3a.quantize_i8_keys(k, cu, scale_out=torch.zeros((H, nb + 1), device="cuda")), h3a.H3A_ESHAPE)
    u8 = torch.zeros((S, H, D), dtype=torch.uint8, device="cuda")
    refused(lambda: h3a.quantize_i8_rows(q, out=u8), h3a.H3A_ESHAPE, u8)
    # E4M3 codes are not INT8 codes, and scale arrays must be fp32 of the exact shape
    q8, k8 = h3a.quantize_e4m3(q), h3a.quantize_e4m3(k)
    refused(lambda: h3a.varlen_attn_fwd_i8qk(q8, ki8, v, cu, 0.1, out=out), h3a.H3A_EDTYPE, out)
    refused(lambda: h3a.varlen_attn_fwd_i8qk(qi8, (ki8[0], ki8[1][:, :-1].contiguous()), v, cu, 0.1, out=out),
            h3a.H3A_ESHAPE, out)
    refused(lambda: h3a.varlen_attn_fwd_i8qk((qi8[0], qi8[1].half()), ki8, v, cu, 0.1, out=out), h3a.H3A_EDTYPE, out)
    vt8 = h3a.prepare_vt_e4m3(v, cu)
    refused(lambda: h3a.varlen_attn_fwd_i8qk_fp8pv(qi8, ki8, (vt8[0][:, :, :-64].contiguous(), vt8[1]), cu, 0.1,
                                                   out=out), h3a.H3A_ESHAPE, out)
    refused(lambda: h3a.varlen_attn_fwd_i8qk_fp8pv(q8, k8, vt8, cu, 0.1, out=out), h3a.H3A_EDTYPE, out)
    qi8o = torch.zeros((S - 1, H, D), dtype=torch.int8, device="cuda")
    refused(lambda: h3a.qk_rmsnorm_rope_i8q(q, k, gam, gam, 1e-6, tab, R, q8=qi8o), h3a.H3A_ESHAPE, qi8o)
    refused(lambda: h3a.qk_rmsnorm_rope_i8q(q.float(), k.float(), gam, gam, 1e-6, tab, R), h3a.H3A_EDTYPE)
    # centred keys: means and their workspace fp32 of the exact shapes
    nseg = len(LENS)
    refused(lambda: h3a.segment_key_means(k.float(), cu), h3a.H3A_EDTYPE)
    refused(lambda: h3a.segment_key_means(k, cu, workspace=torch.zeros((1, H, D), device="cuda")), h3a.H3A_ESHAPE)
    mu_bad = torch.zeros((nseg, H, D - 1), device="cuda")
    refused(lambda: h3a.segment_key_means(k, cu, out=mu_bad), h3a.H3A_ESHAPE, mu_bad)
    refused(lambda: h3a.quantize_i8_keys(k, cu, mu=mu_bad), h3a.H3A_ESHAPE)
    refused(lambda: h3a.quantize_i8_keys(k, cu, mu=torch.zeros((nseg, H, D), device="cuda").half()), h3a.H3A_EDTYPE)
    mu = h3a.segment_key_means(k, cu)
    ki8 = h3a.quantize_i8_keys(k, cu, mu=mu)
    o = h3a.varlen_attn_fwd_i8qk(qi8, ki8, v, cu, 0.1, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    o = h3a.varlen_attn_fwd_i8qk_fp8pv(qi8, ki8, vt8, cu, 0.1, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()


def test_all_empty_packing_is_a_no_op():
    """Every call accepts a packing whose segments are all empty (S = 0, zero-size
    tensors whose data pointers may be null) and returns empty results."""
    import torch

    import packed_varlen_attention_head_amd as h3a

    segs = [(1, 1, 1, 0), (2, 3, 4, 0)]  # valid grids, no tokens
    tab = torch.empty((2, 0, R // 2), dtype=torch.float32, device="cuda")
    cu = h3a.build_rope_table(segs, (32, 32, 32), 10000.0, tab)
    assert list(cu) == [0, 0, 0]
    q, k, v = (torch.empty((0, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    gam = torch.ones(D, dtype=torch.float32, device="cuda")
    h3a.qk_rmsnorm_rope(q, k, gam, gam, 1e-6, tab, R)
    assert h3a.varlen_attn_fwd(q, k, v, cu, 0.1).shape == (0, H, D)
    assert h3a.varlen_attn_fwd_ex(q, k, v, cu, 0.1, causal=True).shape == (0, H, D)
    assert h3a.varlen_attn_fwd_qnorm(q, k, v, cu, 0.1, gam, 1e-6, tab, R).shape == (0, H, D)
    q8, k8 = h3a.qk_rmsnorm_rope_e4m3(q, k, gam, gam, 1e-6, tab, R)
    assert h3a.vt_e4m3_columns(cu) == 0
    vt8 = h3a.prepare_vt_e4m3(v, cu)
    assert h3a.varlen_attn_fwd_fp8qk(q8, k8, v, cu, 0.1).shape == (0, H, D)
    assert h3a.varlen_attn_fwd_fp8(q8, k8, vt8, cu, 0.1).shape == (0, H, D)
    assert h3a.i8_key_blocks(cu) == 0
    qi8, kn = h3a.qk_rmsnorm_rope_i8q(q, k, gam, gam, 1e-6, tab, R)
    ki8 = h3a.quantize_i8_keys(kn, cu)
    assert h3a.quantize_i8_rows(q)[0].shape == (0, H, D)
    assert h3a.varlen_attn_fwd_i8qk(qi8, ki8, v, cu, 0.1).shape == (0, H, D)
    assert h3a.varlen_attn_fwd_i8qk_fp8pv(qi8, ki8, vt8, cu, 0.1).shape == (0, H, D)
    assert h3a.i8_key_mean_chunks(cu) == 0
    mu = h3a.segment_key_means(k, cu)
    torch.cuda.synchronize()
    assert mu.shape == (2, H, D) and not mu.any()  # every segment empty: mean 0
    assert h3a.quantize_i8_keys(kn, cu, mu=mu)[0].shape == (0, H, D)
    torch.cuda.synchronize()
