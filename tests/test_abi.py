"""The C ABI on the CPU: the library loads, exports what include/h3a.h declares,
and rejects invalid requests with a status and a message naming the argument
before any HIP call (so no GPU is needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import packed_varlen_attention_head_amd as h3a

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(h3a.LIB_PATH), reason="libh3a.so not built")

P = 0x7F0000000000  # a 16-byte aligned address that is never dereferenced


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "h3a.h")).read()
    return sorted(set(re.findall(r"\b(h3a_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = h3a.lib()
    names = declared_symbols()
    assert set(names) == set(h3a.EXPORTS)
    for name in names:
        assert hasattr(L, name), name
    assert h3a.version() >= 100


def i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def rope(segments, dims=(32, 32, 32), base=10000.0, table=P, S=None, cu_out=None):
    segs, sp = i32(np.asarray(segments).reshape(-1)) if segments is not None else (None, None)
    d, dp = i32(dims) if dims is not None else (None, None)
    n = len(segments) if segments is not None else 0
    if S is None:
        S = int(sum(s[3] for s in segments)) if segments is not None else 0
    cp = cu_out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if cu_out is not None else None
    return h3a.lib().h3a_build_rope_table(sp, n, dp, base, table, S, cp, None)


@pytest.mark.parametrize("kw,status,word", [
    (dict(segments=None), h3a.H3A_EINVAL, "segments"),
    (dict(segments=[]), h3a.H3A_EINVAL, "nseg"),
    (dict(segments=[(1, 2, 2, 4)], dims=None), h3a.H3A_EINVAL, "axis_dims"),
    (dict(segments=[(1, 2, 2, 4)], dims=(32, 31, 32)), h3a.H3A_EINVAL, "axis_dims[1]"),
    (dict(segments=[(1, 2, 2, 4)], dims=(64, 64, 64)), h3a.H3A_EUNSUPPORTED, "rotated dims"),
    (dict(segments=[(1, 2, 2, 5)]), h3a.H3A_EINVAL, "length"),
    (dict(segments=[(0, 2, 2, 0)]), h3a.H3A_EINVAL, "grid"),
    (dict(segments=[(1, 2, 2, -1)]), h3a.H3A_EINVAL, "length"),
    (dict(segments=[(1, 2, 2, 4)], S=5), h3a.H3A_ESHAPE, "S = 5"),
    (dict(segments=[(1, 2, 2, 4)], base=0.0), h3a.H3A_EINVAL, "base"),
    (dict(segments=[(1, 2, 2, 4)], base=float("nan")), h3a.H3A_EINVAL, "base"),
    (dict(segments=[(1, 2, 2, 4)], table=None), h3a.H3A_EINVAL, "cos_sin"),
    (dict(segments=[(1, 2, 2, 4)], table=P + 4), h3a.H3A_EUNSUPPORTED, "cos_sin"),
])
def test_rope_table_rejects(kw, status, word):
    cu = np.full(8, -7, dtype=np.int32)
    assert rope(cu_out=cu, **kw) == status
    assert word in h3a.last_error()
    assert np.all(cu == -7), "an invalid call wrote cu_seqlens_out"


def rope_ex(segments, mode=h3a.H3A_ROPE_GRID, dims=(32, 32, 32), base=10000.0, start=(0, 0, 0), stop=(1, 1, 1),
            table=P, spec=True):
    segs, sp = i32(np.asarray(segments).reshape(-1))
    S = int(sum(s[3] for s in segments))
    sp_ = ctypes.byref(h3a.rope_spec(mode, dims, base, start, stop)) if spec else None
    return h3a.lib().h3a_build_rope_table_ex(sp, len(segments), sp_, table, S, None, None)


@pytest.mark.parametrize("kw,status,word", [
    (dict(spec=False), h3a.H3A_EINVAL, "spec"),
    (dict(mode=4), h3a.H3A_EINVAL, "mode"),
    (dict(mode=-1), h3a.H3A_EINVAL, "mode"),
    (dict(mode=h3a.H3A_ROPE_LINSPACE, stop=(1, float("inf"), 1)), h3a.H3A_EINVAL, "linspace"),
    (dict(mode=h3a.H3A_ROPE_INTERLEAVED, dims=(4, 8, 4)), h3a.H3A_EINVAL, "interleaved"),
    (dict(mode=h3a.H3A_ROPE_INTERLEAVED, dims=(8, 4, 4), base=-1.0), h3a.H3A_EINVAL, "base"),
    (dict(mode=h3a.H3A_ROPE_LINSPACE, segments=[(1, 2, 2, 5)]), h3a.H3A_EINVAL, "length"),
    (dict(mode=h3a.H3A_ROPE_INTERLEAVED, dims=(8, 4, 4), segments=[(1, 2, 2, 5)]), h3a.H3A_EINVAL, "length"),
    (dict(mode=h3a.H3A_ROPE_NORMALIZED, segments=[(1, 2, 2, -1)]), h3a.H3A_EINVAL, "negative"),
    (dict(mode=h3a.H3A_ROPE_NORMALIZED, segments=[(2000, 2000, 2000, 5)]), h3a.H3A_EINVAL, "INT32_MAX"),
    (dict(mode=h3a.H3A_ROPE_NORMALIZED, segments=[(1, 2, 2, 6)], table=None), h3a.H3A_EINVAL, "cos_sin"),
])
def test_rope_table_ex_rejects(kw, status, word):
    kw.setdefault("segments", [(1, 2, 2, 4)])
    assert rope_ex(**kw) == status
    assert word in h3a.last_error(), h3a.last_error()


def qk(dtype=h3a.H3A_BF16, S=16, H=2, D=128, sq=None, sk=None, sqo=None, sko=None, q=P, k=P + (1 << 24),
       qo=None, ko=None, gq=P + (2 << 24), gk=P + (3 << 24), eps=1e-6, cs=P + (4 << 24), rot=96):
    hd = H * D
    qo = q if qo is None else qo
    ko = k if ko is None else ko
    return h3a.lib().h3a_qk_rmsnorm_rope(q, k, qo, ko, dtype, S, H, D, sq or hd, sk or hd, sqo or hd, sko or hd,
                                         gq, gk, eps, cs, rot, None)


@pytest.mark.parametrize("kw,status,word", [
    (dict(dtype=7), h3a.H3A_EDTYPE, "dtype"),
    (dict(D=96, rot=48), h3a.H3A_EUNSUPPORTED, "head_dim"),
    (dict(rot=95), h3a.H3A_EINVAL, "rot_dim"),
    (dict(rot=130), h3a.H3A_EINVAL, "rot_dim"),
    (dict(rot=40), h3a.H3A_EUNSUPPORTED, "rot_dim / 2"),
    (dict(dtype=h3a.H3A_F32, rot=36), h3a.H3A_EUNSUPPORTED, "rot_dim / 2"),
    (dict(H=0), h3a.H3A_EINVAL, "H ="),
    (dict(S=-1), h3a.H3A_EINVAL, "S ="),
    (dict(sq=100), h3a.H3A_ESHAPE, "q: token stride"),
    (dict(sko=255), h3a.H3A_ESHAPE, "k_out"),
    (dict(sq=260), h3a.H3A_EUNSUPPORTED, "multiple of 16 bytes"),
    (dict(q=None), h3a.H3A_EINVAL, "q is NULL"),
    (dict(k=P + 2), h3a.H3A_EUNSUPPORTED, "k is not 16-byte aligned"),
    (dict(gq=None), h3a.H3A_EINVAL, "gamma_q"),
    (dict(cs=None), h3a.H3A_EINVAL, "cos_sin"),
    (dict(eps=-1.0), h3a.H3A_EINVAL, "eps"),
    (dict(qo=P + 256), h3a.H3A_EINVAL, "q_out overlaps q"),
    (dict(qo=P + (1 << 24)), h3a.H3A_EINVAL, "q_out overlaps k"),
    (dict(qo=P + (5 << 24), ko=P + (5 << 24) + 64), h3a.H3A_EINVAL, "q_out overlaps k_out"),
])
def test_qk_rmsnorm_rope_rejects(kw, status, word):
    assert qk(**kw) == status
    assert word in h3a.last_error(), h3a.last_error()


def test_qk_rmsnorm_rope_empty_is_a_no_op():
    assert qk(S=0) == h3a.H3A_OK


def attn(dtype=h3a.H3A_BF16, S=300, H=2, D=128, cu=(0, 100, 300), strides=None, q=P, k=P + (1 << 24),
         v=P + (2 << 24), o=P + (3 << 24), scale=0.088):
    hd = H * D
    s = strides or (hd, hd, hd, hd)
    c, cp = i32(cu) if cu is not None else (None, None)
    n = len(cu) - 1 if cu is not None else 1
    return h3a.lib().h3a_varlen_attn_fwd(q, k, v, o, dtype, S, H, D, *s, cp, n, scale, None)


@pytest.mark.parametrize("kw,status,word", [
    (dict(dtype=3), h3a.H3A_EDTYPE, "dtype"),
    (dict(D=256), h3a.H3A_EUNSUPPORTED, "head_dim"),
    (dict(cu=None), h3a.H3A_EINVAL, "cu_seqlens"),
    (dict(cu=(0,)), h3a.H3A_EINVAL, "nseg"),
    (dict(cu=(1, 100, 300)), h3a.H3A_EINVAL, "cu_seqlens[0]"),
    (dict(cu=(0, 200, 100, 300)), h3a.H3A_EINVAL, "decreases at index 2"),
    (dict(cu=(0, 100, 299)), h3a.H3A_ESHAPE, "cu_seqlens[nseg]"),
    (dict(scale=0.0), h3a.H3A_EINVAL, "scale"),
    (dict(scale=float("inf")), h3a.H3A_EINVAL, "scale"),
    (dict(strides=(256, 128, 256, 256)), h3a.H3A_ESHAPE, "k: token stride"),
    (dict(strides=(256, 256, 256, 260)), h3a.H3A_EUNSUPPORTED, "o: token stride"),
    (dict(v=None), h3a.H3A_EINVAL, "v is NULL"),
    (dict(o=P + 8), h3a.H3A_EUNSUPPORTED, "o is not 16-byte aligned"),
    (dict(o=P + 512), h3a.H3A_EINVAL, "o overlaps q"),
    (dict(o=P + (2 << 24) - 256), h3a.H3A_EINVAL, "o overlaps v"),
    (dict(H=0), h3a.H3A_EINVAL, "H ="),
    (dict(strides=(256, 256, 1 << 24, 256)), h3a.H3A_EUNSUPPORTED, "v: token stride"),
])
def test_varlen_attn_rejects(kw, status, word):
    assert attn(**kw) == status
    assert word in h3a.last_error(), h3a.last_error()


def attn_ex(dtype=h3a.H3A_BF16, S=300, Hq=8, Hkv=2, D=128, cu=(0, 100, 300), strides=None, q=P,
            k=P + (1 << 24), v=P + (2 << 24), o=P + (3 << 24), scale=0.088, causal=1):
    s = strides or (Hq * D, Hkv * D, Hkv * D, Hq * D)
    c, cp = i32(cu)
    return h3a.lib().h3a_varlen_attn_fwd_ex(q, k, v, o, dtype, S, Hq, Hkv, D, *s, cp, len(cu) - 1, scale, causal,
                                            None)


@pytest.mark.parametrize("kw,status,word", [
    (dict(Hkv=3), h3a.H3A_ESHAPE, "does not divide"),
    (dict(Hkv=0), h3a.H3A_EINVAL, "Hkv ="),
    (dict(Hq=0), h3a.H3A_EINVAL, "H ="),
    (dict(causal=2), h3a.H3A_EINVAL, "causal"),
    (dict(causal=-1), h3a.H3A_EINVAL, "causal"),
    (dict(strides=(1024, 128, 256, 1024)), h3a.H3A_ESHAPE, "k: token stride"),
    (dict(strides=(1024, 256, 256, 512)), h3a.H3A_ESHAPE, "o: token stride"),
    (dict(dtype=9), h3a.H3A_EDTYPE, "dtype"),
    (dict(D=96), h3a.H3A_EUNSUPPORTED, "head_dim"),
    (dict(o=P + (1 << 24) + 512), h3a.H3A_EINVAL, "o overlaps k"),
])
def test_varlen_attn_ex_rejects(kw, status, word):
    assert attn_ex(**kw) == status
    assert word in h3a.last_error(), h3a.last_error()


def _device_visible():
    import torch

    return torch.cuda.device_count() > 0


@pytest.mark.skipif(_device_visible(), reason="a valid call would launch on the visible GPU")
def test_grouped_tensors_side_by_side_pass_validation():
    """A narrow K/V tensor right below a wider output: no false overlap.  Without a GPU the
    call gets past validation and stops at the device query (EHIP)."""
    S = 300
    st = attn_ex(dtype=h3a.H3A_F32, S=S, Hq=4, Hkv=1, strides=(512, 128, 128, 512), q=P + (1 << 26),
                 k=P + (1 << 27), v=P, o=P + S * 128 * 4)
    assert st == h3a.H3A_EHIP and "hipGetDevice" in h3a.last_error(), h3a.last_error()
    # q, k, v as column slices of one fused [S, (Hq + 2 Hkv) D] bf16 buffer
    Hq, Hkv, D = 8, 2, 128
    row = (Hq + 2 * Hkv) * D
    st = attn_ex(S=S, strides=(row, row, row, Hq * D), q=P, k=P + Hq * D * 2, v=P + (Hq + Hkv) * D * 2,
                 o=P + (1 << 27))
    assert st == h3a.H3A_EHIP, h3a.last_error()
    # and a real overlap inside the fused row is still caught
    st = attn_ex(S=S, strides=(row, row, row, row), q=P, k=P + Hq * D * 2, v=P + (Hq + Hkv) * D * 2,
                 o=P + (Hq + Hkv) * D * 2 + 256)
    assert st == h3a.H3A_EINVAL and "o overlaps" in h3a.last_error(), h3a.last_error()


def attn_qn(dtype=h3a.H3A_BF16, S=300, Hq=8, Hkv=2, D=128, rot=96, g=P + (5 << 24), cs=P + (6 << 24), eps=1e-6,
            o=P + (3 << 24), scale=0.088):
    c, cp = i32((0, 100, 300))
    return h3a.lib().h3a_varlen_attn_fwd_qnorm(P, P + (1 << 24), P + (2 << 24), o, dtype, S, Hq, Hkv, D, Hq * D,
                                               Hkv * D, Hkv * D, Hq * D, cp, 2, scale, g, eps, cs, rot, None)


@pytest.mark.parametrize("kw,status,word", [
    (dict(dtype=h3a.H3A_F32), h3a.H3A_EUNSUPPORTED, "bf16 only"),
    (dict(dtype=5), h3a.H3A_EDTYPE, "dtype"),
    (dict(rot=48), h3a.H3A_EUNSUPPORTED, "multiple of 32"),
    (dict(rot=160), h3a.H3A_EINVAL, "rot_dim"),
    (dict(rot=96, D=64), h3a.H3A_EINVAL, "rot_dim"),
    (dict(g=None), h3a.H3A_EINVAL, "gamma_q"),
    (dict(g=P + 4), h3a.H3A_EUNSUPPORTED, "gamma_q is not 16-byte aligned"),
    (dict(cs=None), h3a.H3A_EINVAL, "cos_sin"),
    (dict(eps=float("nan")), h3a.H3A_EINVAL, "eps"),
    (dict(Hkv=3), h3a.H3A_ESHAPE, "does not divide"),
    (dict(o=P + 256), h3a.H3A_EINVAL, "o overlaps q"),
    (dict(scale=-1.0), h3a.H3A_EINVAL, "scale"),
])
def test_varlen_attn_fwd_qnorm_rejects(kw, status, word):
    assert attn_qn(**kw) == status
    assert word in h3a.last_error(), h3a.last_error()


@pytest.mark.parametrize("kw,status,word", [
    (dict(H=0), h3a.H3A_EINVAL, "H ="),
    (dict(rot=40), h3a.H3A_EUNSUPPORTED, "rot_dim / 2"),
    (dict(xo=P + 256), h3a.H3A_EINVAL, "x_out overlaps x"),
    (dict(g=None), h3a.H3A_EINVAL, "gamma"),
    (dict(sx=100), h3a.H3A_ESHAPE, "x: token stride"),
])
def test_rmsnorm_rope_rejects(kw, status, word):
    H = kw.get("H", 2)
    sx = kw.get("sx", max(H, 1) * 128)
    st = h3a.lib().h3a_rmsnorm_rope(P, kw.get("xo", P), h3a.H3A_BF16, 16, H, 128, sx, sx, kw.get("g", P + (2 << 24)),
                                    1e-6, P + (4 << 24), kw.get("rot", 96), None)
    assert st == status
    assert word in h3a.last_error(), h3a.last_error()


@pytest.mark.parametrize("kw,status,word", [
    (dict(H=0), h3a.H3A_EINVAL, "H ="),
    (dict(D=96), h3a.H3A_EUNSUPPORTED, "head_dim"),
    (dict(sy=120), h3a.H3A_ESHAPE, "y: token stride"),
    (dict(sy=264), h3a.H3A_EUNSUPPORTED, "multiple of 16 bytes"),
    (dict(y=P + 256), h3a.H3A_EINVAL, "y overlaps x"),
    (dict(y=None), h3a.H3A_EINVAL, "y is NULL"),
    (dict(ys=None), h3a.H3A_EINVAL, "y_scale is NULL"),
    (dict(ys=P + (1 << 24) + 4000), h3a.H3A_EINVAL, "y_scale overlaps"),
])
def test_quantize_e4m3_rejects(kw, status, word):
    H, D = kw.get("H", 2), kw.get("D", 128)
    st = h3a.lib().h3a_quantize_e4m3(P, kw.get("y", P + (1 << 24)), kw.get("ys", P + (2 << 24)), 16, H, D,
                                     max(H, 1) * D, kw.get("sy", max(H, 1) * D), None)
    assert st == status
    assert word in h3a.last_error(), h3a.last_error()


@pytest.mark.parametrize("kw,status,word", [
    (dict(Hkv=3), h3a.H3A_ESHAPE, "does not divide"),
    (dict(causal=5), h3a.H3A_EINVAL, "causal"),
    (dict(sq=1032), h3a.H3A_EUNSUPPORTED, "q: token stride"),
    (dict(sk=64), h3a.H3A_ESHAPE, "k: token stride"),
    (dict(o=P + 512), h3a.H3A_EINVAL, "o overlaps q"),
    (dict(D=80), h3a.H3A_EUNSUPPORTED, "head_dim"),
    (dict(qs=None), h3a.H3A_EINVAL, "q_scale is NULL"),
    (dict(ks=P + (5 << 24) + 2), h3a.H3A_EUNSUPPORTED, "k_scale is not 4-byte aligned"),
    (dict(qs=P + (3 << 24) + 64), h3a.H3A_EINVAL, "o overlaps q_scale"),
])
def test_varlen_attn_fwd_fp8qk_rejects(kw, status, word):
    Hq, Hkv, D = 8, kw.get("Hkv", 2), kw.get("D", 128)
    c, cp = i32((0, 100, 300))
    st = h3a.lib().h3a_varlen_attn_fwd_fp8qk(P, P + (1 << 24), kw.get("qs", P + (4 << 24)), kw.get("ks", P + (5 << 24)),
                                             P + (2 << 24), kw.get("o", P + (3 << 24)), 300, Hq, Hkv,
                                             D, kw.get("sq", Hq * D), kw.get("sk", Hkv * D), Hkv * D, Hq * D, cp, 2,
                                             0.088, kw.get("causal", 0), None)
    assert st == status
    assert word in h3a.last_error(), h3a.last_error()


@pytest.mark.parametrize("kw,status,word", [
    (dict(Hk=0), h3a.H3A_EINVAL, "Hk ="),
    (dict(rot=40), h3a.H3A_EUNSUPPORTED, "rot_dim / 2"),
    (dict(sq8=100), h3a.H3A_ESHAPE, "q8: token stride"),
    (dict(q8=P + 512), h3a.H3A_EINVAL, "q8 overlaps"),
    (dict(cs=None), h3a.H3A_EINVAL, "cos_sin"),
    (dict(ks=None), h3a.H3A_EINVAL, "k_scale is NULL"),
    (dict(qs=P + (2 << 24) + 8), h3a.H3A_EINVAL, "q_scale or k_scale overlaps"),
    (dict(ks=P + (7 << 24) + 100), h3a.H3A_EINVAL, "q_scale overlaps k_scale"),
])
def test_qk_rmsnorm_rope_e4m3_rejects(kw, status, word):
    Hq, Hk, D = 8, kw.get("Hk", 2), 128
    st = h3a.lib().h3a_qk_rmsnorm_rope_e4m3(P, P + (1 << 24), kw.get("q8", P + (2 << 24)), P + (3 << 24),
                                            kw.get("qs", P + (7 << 24)), kw.get("ks", P + (8 << 24)), 16, Hq, Hk,
                                            D, Hq * D, max(Hk, 1) * D, kw.get("sq8", Hq * D), max(Hk, 1) * D,
                                            P + (4 << 24), P + (5 << 24), 1e-6, kw.get("cs", P + (6 << 24)),
                                            kw.get("rot", 96), None)
    assert st == status
    assert word in h3a.last_error(), h3a.last_error()


@pytest.mark.parametrize("kw,status,word", [
    (dict(Hk=0), h3a.H3A_EINVAL, "Hk ="),
    (dict(rot=40), h3a.H3A_EUNSUPPORTED, "rot_dim / 2"),
    (dict(sq8=100), h3a.H3A_ESHAPE, "q8: token stride"),
    (dict(q8=P + 512), h3a.H3A_EINVAL, "q8 overlaps"),
    (dict(q8=P + (3 << 24) + 256), h3a.H3A_EINVAL, "q8 overlaps"),
    (dict(cs=None), h3a.H3A_EINVAL, "cos_sin"),
    (dict(qs=None), h3a.H3A_EINVAL, "q_scale is NULL"),
    (dict(qs=P + (7 << 24) + 2), h3a.H3A_EUNSUPPORTED, "q_scale is not 4-byte aligned"),
    (dict(qs=P + (1 << 24) + 64), h3a.H3A_EINVAL, "q_scale overlaps"),
    (dict(qs=P + (2 << 24) + 64), h3a.H3A_EINVAL, "q_scale overlaps q8"),
    (dict(ko=P + (1 << 24) + 256), h3a.H3A_EINVAL, "k_out overlaps k without"),
    (dict(ko=P + 256), h3a.H3A_EINVAL, "k_out overlaps q"),
])
def test_qk_rmsnorm_rope_i8q_rejects(kw, status, word):
    Hq, Hk, D = 8, kw.get("Hk", 2), 128
    st = h3a.lib().h3a_qk_rmsnorm_rope_i8q(P, P + (1 << 24), kw.get("q8", P + (2 << 24)), kw.get("ko", P + (3 << 24)),
                                           kw.get("qs", P + (7 << 24)), 16, Hq, Hk, D, Hq * D, max(Hk, 1) * D,
                                           kw.get("sq8", Hq * D), max(Hk, 1) * D, P + (4 << 24), P + (5 << 24), 1e-6,
                                           kw.get("cs", P + (6 << 24)), kw.get("rot", 96), None)
    assert st == status
    assert word in h3a.last_error(), h3a.last_error()


def test_qk_rmsnorm_rope_i8q_accepts_k_in_place_and_empty():
    """k_out = k with the same stride is accepted (validation only: S = 0 launches nothing)."""
    st = h3a.lib().h3a_qk_rmsnorm_rope_i8q(P, P + (1 << 24), P + (2 << 24), P + (1 << 24), P + (7 << 24), 0, 8, 2,
                                           128, 8 * 128, 2 * 128, 8 * 128, 2 * 128, P + (4 << 24), P + (5 << 24),
                                           1e-6, P + (6 << 24), 96, None)
    assert st == h3a.H3A_OK, h3a.last_error()


@pytest.mark.parametrize("kw,status,word", [
    (dict(cols=320), h3a.H3A_ESHAPE, "vt_cols = 320"),
    (dict(vt=P + (1 << 24) + 8), h3a.H3A_EUNSUPPORTED, "vt8 is not 16-byte aligned"),
    (dict(vs=None), h3a.H3A_EINVAL, "vt_scale is NULL"),
    (dict(vs=P + (2 << 24) + 1), h3a.H3A_EUNSUPPORTED, "vt_scale is not 4-byte aligned"),
    (dict(vs=P + (1 << 24) + 4096), h3a.H3A_EINVAL, "vt_scale overlaps v or vt8"),
])
def test_prepare_vt_e4m3_rejects(kw, status, word):
    Hkv, D = 2, 128
    c, cp = i32((0, 100, 300))  # 128 + 256 padded columns
    st = h3a.lib().h3a_prepare_vt_e4m3(P, kw.get("vt", P + (1 << 24)), kw.get("vs", P + (2 << 24)), 300, Hkv, D,
                                       Hkv * D, kw.get("cols", 384), cp, 2, None)
    assert st == status
    assert word in h3a.last_error(), h3a.last_error()


@pytest.mark.parametrize("kw,status,word", [
    (dict(cols=448), h3a.H3A_ESHAPE, "vt_cols = 448"),
    (dict(vs=None), h3a.H3A_EINVAL, "vt_scale is NULL"),
    (dict(qs=P + (4 << 24) + 1), h3a.H3A_EUNSUPPORTED, "q_scale is not 4-byte aligned"),
    (dict(vs=P + (3 << 24) + 256), h3a.H3A_EINVAL, "o overlaps a scale array"),
    (dict(vt=None), h3a.H3A_EINVAL, "vt8 is NULL"),
])
def test_varlen_attn_fwd_fp8_rejects(kw, status, word):
    Hq, Hkv, D = 8, 2, 128
    c, cp = i32((0, 100, 300))
    st = h3a.lib().h3a_varlen_attn_fwd_fp8(P, P + (1 << 24), kw.get("vt", P + (2 << 24)), kw.get("qs", P + (4 << 24)),
                                           P + (5 << 24), kw.get("vs", P + (6 << 24)), P + (3 << 24), 300, Hq, Hkv, D,
                                           Hq * D, Hkv * D, kw.get("cols", 384), Hq * D, cp, 2, 0.088, 0, None)
    assert st == status
    assert word in h3a.last_error(), h3a.last_error()


@pytest.mark.parametrize("kw,status,word", [
    (dict(H=0), h3a.H3A_EINVAL, "H ="),
    (dict(D=96), h3a.H3A_EUNSUPPORTED, "head_dim"),
    (dict(sy=120), h3a.H3A_ESHAPE, "y: token stride"),
    (dict(y=P + 256), h3a.H3A_EINVAL, "y overlaps x"),
    (dict(ys=None), h3a.H3A_EINVAL, "y_scale is NULL"),
    (dict(ys=P + (2 << 24) + 2), h3a.H3A_EUNSUPPORTED, "y_scale is not 4-byte aligned"),
    (dict(ys=P + (1 << 24) + 4000), h3a.H3A_EINVAL, "y_scale overlaps"),
])
def test_quantize_i8_rows_rejects(kw, status, word):
    H, D = kw.get("H", 2), kw.get("D", 128)
    st = h3a.lib().h3a_quantize_i8_rows(P, kw.get("y", P + (1 << 24)), kw.get("ys", P + (2 << 24)), 16, H, D,
                                        max(H, 1) * D, kw.get("sy", max(H, 1) * D), None)
    assert st == status
    assert word in h3a.last_error(), h3a.last_error()


@pytest.mark.parametrize("kw,status,word", [
    (dict(nb=5), h3a.H3A_ESHAPE, "n_blocks = 5"),
    (dict(cu=(0, 100, 90)), h3a.H3A_EINVAL, "decreases"),
    (dict(ys=None), h3a.H3A_EINVAL, "y_scale is NULL"),
    (dict(y=P + 256), h3a.H3A_EINVAL, "y overlaps x"),
    (dict(ys=P + (1 << 24) + 256), h3a.H3A_EINVAL, "y_scale overlaps"),
])
def test_quantize_i8_keys_rejects(kw, status, word):
    H, D = 2, 128
    c, cp = i32(kw.get("cu", (0, 100, 300)))  # 2 + 4 key blocks
    S = 300 if c[-1] == 300 else int(c[-1])
    st = h3a.lib().h3a_quantize_i8_keys(P, kw.get("y", P + (1 << 24)), kw.get("ys", P + (2 << 24)), S, H, D, H * D,
                                        H * D, kw.get("nb", 6), cp, 2, None)
    assert st == status
    assert word in h3a.last_error(), h3a.last_error()


def test_i8_key_blocks_counts_each_segment_from_its_start():
    n = ctypes.c_int64(-1)
    c, cp = i32((0, 65, 65, 66, 194))
    assert h3a.lib().h3a_i8_key_blocks(cp, 4, ctypes.byref(n)) == h3a.H3A_OK and n.value == 2 + 0 + 1 + 2
    assert h3a.i8_key_blocks([0, 64, 128, 129]) == 3
    assert h3a.lib().h3a_i8_key_blocks(cp, 4, None) == h3a.H3A_EINVAL


@pytest.mark.parametrize("kw,status,word", [
    (dict(Hkv=3), h3a.H3A_ESHAPE, "does not divide"),
    (dict(causal=2), h3a.H3A_EINVAL, "causal"),
    (dict(sk=64), h3a.H3A_ESHAPE, "k: token stride"),
    (dict(o=P + 512), h3a.H3A_EINVAL, "o overlaps q"),
    (dict(qs=None), h3a.H3A_EINVAL, "q_scale is NULL"),
    (dict(ks=P + (5 << 24) + 2), h3a.H3A_EUNSUPPORTED, "k_scale is not 4-byte aligned"),
    (dict(qs=P + (3 << 24) + 64), h3a.H3A_EINVAL, "o overlaps q_scale"),
    (dict(scale=0.0), h3a.H3A_EINVAL, "scale"),
])
def test_varlen_attn_fwd_i8qk_rejects(kw, status, word):
    Hq, Hkv, D = 8, kw.get("Hkv", 2), 128
    c, cp = i32((0, 100, 300))
    st = h3a.lib().h3a_varlen_attn_fwd_i8qk(P, P + (1 << 24), kw.get("qs", P + (4 << 24)), kw.get("ks", P + (5 << 24)),
                                            P + (2 << 24), kw.get("o", P + (3 << 24)), 300, Hq, Hkv, D, Hq * D,
                                            kw.get("sk", Hkv * D), Hkv * D, Hq * D, cp, 2, kw.get("scale", 0.088),
                                            kw.get("causal", 0), None)
    assert st == status
    assert word in h3a.last_error(), h3a.last_error()


def qk_ex(Hq=8, Hk=0, **kw):
    D, hd, hk = 128, Hq * 128, max(Hk, 1) * 128
    return h3a.lib().h3a_qk_rmsnorm_rope_ex(P, P + (1 << 24), P, P + (1 << 24), h3a.H3A_BF16, 16, Hq, Hk, D, hd, hk,
                                            hd, hk, P + (2 << 24), P + (3 << 24), 1e-6, P + (4 << 24), 96, None)


def test_qk_rmsnorm_rope_ex_rejects():
    assert qk_ex(Hk=0) == h3a.H3A_EINVAL and "Hk =" in h3a.last_error()
    assert qk_ex(Hq=0, Hk=2) == h3a.H3A_EINVAL and "H =" in h3a.last_error()


def test_varlen_attn_empty_is_a_no_op():
    assert attn(S=0, cu=(0, 0, 0)) == h3a.H3A_OK


def test_binding_reports_errors_by_exception():
    with pytest.raises(h3a.H3AError) as e:
        h3a.plan_tiles([0, 5, 3], heads=2, block_m=128, n_xcd=8)
    assert e.value.status == h3a.H3A_EINVAL and "decreases" in e.value.message


def attn_noalloc(cu, Hq=2, Hkv=2, D=128, dtype=h3a.H3A_BF16, causal=0):
    """h3a_varlen_attn_fwd_noalloc with never-dereferenced, disjoint operand addresses."""
    c, cp = i32(cu)
    S = int(c[-1])
    q, k, v, o = (P + i * (1 << 40) for i in range(4))
    return h3a.lib().h3a_varlen_attn_fwd_noalloc(q, k, v, o, dtype, S, Hq, Hkv, D, Hq * D, Hkv * D, Hkv * D,
                                                 Hq * D, cp, len(c) - 1, 0.088, causal, None)


@pytest.mark.parametrize("cu,H,word", [
    (np.arange(258) * 3, 2, "257"),                               # 257 non-empty segments
    (np.concatenate([[0], np.arange(1, 258) * 3, [800] * 40]), 2, "257"),  # empty ones do not help
    ([0, 1 << 20], 16, "131072 work items"),                      # 8,192 query tiles x 16 heads
    ([0, 60000, 120000], 70, "65,536"),                           # 65,660 items
])
def test_noalloc_limits_rejected_before_the_device(cu, H, word):
    """Past its fixed plan array the allocation-free entry point fails with
    EUNSUPPORTED before any HIP call, naming the limit."""
    assert attn_noalloc(cu, Hq=H, Hkv=H) == h3a.H3A_EUNSUPPORTED
    msg = h3a.last_error()
    assert ("256" in msg or "65536" in msg), msg
    assert word.replace(",", "") in msg.replace(",", "") or "non-empty segments" in msg, msg


def test_noalloc_validates_like_the_cached_entry():
    """Same argument checks as h3a_varlen_attn_fwd_ex (shared code): bad head
    counts, dtype, cu_seqlens and overlapping outputs fail the same way."""
    assert attn_noalloc([0, 10], Hq=3, Hkv=2) == h3a.H3A_ESHAPE
    assert attn_noalloc([0, 10], D=96) == h3a.H3A_EUNSUPPORTED
    assert attn_noalloc([0, 10], dtype=7) == h3a.H3A_EDTYPE
    assert attn_noalloc([0, 10, 9]) == h3a.H3A_EINVAL and "decreases" in h3a.last_error()
    assert attn_noalloc([0, 10], causal=2) == h3a.H3A_EINVAL


def test_set_split_policy():
    assert h3a.lib().h3a_set_split_policy(7) == h3a.H3A_EINVAL and "split policy" in h3a.last_error()
    assert h3a.lib().h3a_set_split_policy(-1) == h3a.H3A_EINVAL
    for p in (h3a.H3A_SPLIT_NEVER, h3a.H3A_SPLIT_ALWAYS, h3a.H3A_SPLIT_AUTO):
        assert h3a.lib().h3a_set_split_policy(p) == h3a.H3A_OK


@pytest.mark.parametrize("kw,status,word", [
    (dict(cols=448), h3a.H3A_ESHAPE, "vt_cols = 448"),
    (dict(vs=None), h3a.H3A_EINVAL, "vt_scale is NULL"),
    (dict(qs=P + (4 << 24) + 2), h3a.H3A_EUNSUPPORTED, "q_scale is not 4-byte aligned"),
    (dict(ks=None), h3a.H3A_EINVAL, "k_scale is NULL"),
    (dict(vs=P + (3 << 24) + 256), h3a.H3A_EINVAL, "o overlaps a scale array"),
    (dict(ks=P + (3 << 24) + 64), h3a.H3A_EINVAL, "o overlaps a scale array"),
    (dict(vt=None), h3a.H3A_EINVAL, "vt8 is NULL"),
    (dict(vt=P + (2 << 24) + 8), h3a.H3A_EUNSUPPORTED, "vt8 is not 16-byte aligned"),
    (dict(Hkv=3), h3a.H3A_ESHAPE, "does not divide"),
])
def test_varlen_attn_fwd_i8qk_fp8pv_rejects(kw, status, word):
    Hq, Hkv, D = 8, kw.get("Hkv", 2), 128
    c, cp = i32((0, 100, 300))  # 2 + 4 key blocks, 384 padded columns
    st = h3a.lib().h3a_varlen_attn_fwd_i8qk_fp8pv(P, P + (1 << 24), kw.get("vt", P + (2 << 24)),
                                                  kw.get("qs", P + (4 << 24)), kw.get("ks", P + (5 << 24)),
                                                  kw.get("vs", P + (6 << 24)), P + (3 << 24), 300, Hq, Hkv, D, Hq * D,
                                                  Hkv * D, kw.get("cols", 384), Hq * D, cp, 2, 0.088, 0, None)
    assert st == status
    assert word in h3a.last_error(), h3a.last_error()


def test_i8_key_mean_chunks_counts_each_segment_from_its_start():
    n = ctypes.c_int64(-1)
    c, cp = i32((0, 257, 257, 258, 770))
    assert h3a.lib().h3a_i8_key_mean_chunks(cp, 4, ctypes.byref(n)) == h3a.H3A_OK and n.value == 2 + 0 + 1 + 2
    assert h3a.i8_key_mean_chunks([0, 256, 512, 513]) == 3
    assert h3a.lib().h3a_i8_key_mean_chunks(cp, 4, None) == h3a.H3A_EINVAL


@pytest.mark.parametrize("kw,status,word", [
    (dict(nc=3), h3a.H3A_ESHAPE, "n_chunks = 3"),
    (dict(part=None), h3a.H3A_EINVAL, "partial is NULL"),
    (dict(mu=None), h3a.H3A_EINVAL, "mu is NULL"),
    (dict(mu=P + (2 << 24) + 2), h3a.H3A_EUNSUPPORTED, "mu is not 4-byte aligned"),
    (dict(mu=P + (1 << 24) + 64), h3a.H3A_EINVAL, "partial overlaps mu"),
    (dict(part=P + 4096), h3a.H3A_EINVAL, "partial or mu overlaps k"),
])
def test_segment_key_means_rejects(kw, status, word):
    H, D = 2, 128
    c, cp = i32((0, 100, 300))  # 1 + 1 chunks of 256 keys
    st = h3a.lib().h3a_segment_key_means(P, kw.get("part", P + (1 << 24)), kw.get("mu", P + (2 << 24)), 300, H, D,
                                         H * D, kw.get("nc", 2), cp, 2, None)
    assert st == status
    assert word in h3a.last_error(), h3a.last_error()


@pytest.mark.parametrize("kw,status,word", [
    (dict(mu=None), h3a.H3A_EINVAL, "mu is NULL"),
    (dict(mu=P + (3 << 24) + 4), h3a.H3A_EUNSUPPORTED, "mu is not 16-byte aligned"),
    (dict(mu=P + (1 << 24) + 256), h3a.H3A_EINVAL, "mu overlaps y or y_scale"),
    (dict(nb=5), h3a.H3A_ESHAPE, "n_blocks = 5"),
])
def test_quantize_i8_keys_centered_rejects(kw, status, word):
    H, D = 2, 128
    c, cp = i32((0, 100, 300))  # 2 + 4 key blocks
    st = h3a.lib().h3a_quantize_i8_keys_centered(P, kw.get("mu", P + (3 << 24)), P + (1 << 24), P + (2 << 24), 300, H,
                                                 D, H * D, H * D, kw.get("nb", 6), cp, 2, None)
    assert st == status
    assert word in h3a.last_error(), h3a.last_error()
