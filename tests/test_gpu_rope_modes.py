"""GPU parity of the other rotary table modes (linspace, length-normalised ids,
interleaved M-RoPE) against the fp64 oracle, at table level and through the
whole chain (table -> RMSNorm + rotary -> per-segment attention)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import configs, rng
from tests.gpu_util import compare, log, require_gpu, sample_rows, to_device, to_f64

pytestmark = pytest.mark.gpu

GRID, LINSPACE, NORMALIZED, INTERLEAVED = (oracle.ROPE_GRID, oracle.ROPE_LINSPACE, oracle.ROPE_NORMALIZED,
                                           oracle.ROPE_INTERLEAVED)
TABLE_TOL = 1.2e-7  # fp64 angle rounded once to fp32, plus one libm last bit


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()


def h3a():
    import packed_varlen_attention_head_amd as m

    return m


def device_table(segments, mode, dims, base, start=(0.0, 0.0, 0.0), stop=(0.0, 0.0, 0.0)):
    import torch

    S = int(sum(s[3] for s in segments))
    t = torch.full((2, S, sum(dims) // 2), -5.0, dtype=torch.float32, device="cuda")
    cu = h3a().build_rope_table_ex(segments, mode, dims, base, t, start=start, stop=stop)
    torch.cuda.synchronize()
    return t, cu


H3 = configs.H3_S20423.segments
TABLE_CASES = {
    # name: (segments, mode, dims, base, start, stop)
    "linspace_h3": (H3, LINSPACE, (32, 32, 32), 10000.0, (0.5, -1.0, 0.0), (12.0, 1.0, 3.0)),
    "linspace_ragged": (configs.RAGGED64.segments, LINSPACE, (32, 32, 32), 10000.0, (0.0, 0.0, -4.0),
                        (1.0, 7.0, 4.0)),
    "normalized_vit3d": (configs.VIT3D_TILES.segments, NORMALIZED, (16, 16, 16), 100.0, None, None),
    "normalized_h3_suffix": (((10, 30, 54, 16200 + 7),) + H3[1:], NORMALIZED, (32, 32, 32), 10000.0, None, None),
    "interleaved_qwen": (configs.MROPE_PACKED.segments, INTERLEAVED, (48, 40, 40), 1000000.0, None, None),
    "interleaved_equal": (H3, INTERLEAVED, (32, 32, 32), 10000.0, None, None),
    "interleaved_tiny": (((2, 3, 4, 24), (5, 1, 1, 3)), INTERLEAVED, (8, 4, 4), 64.0, None, None),
}


@pytest.mark.parametrize("case", sorted(TABLE_CASES))
def test_rope_mode_table(case):
    segs, mode, dims, base, start, stop = TABLE_CASES[case]
    kw = dict(start=start, stop=stop) if mode == LINSPACE else {}
    log(f"[rope mode table] {case} mode={mode} S={sum(s[3] for s in segs)}")
    t, cu = device_table(segs, mode, dims, base, **kw)
    ocu, ocos, osin = oracle.rope_table_mode(segs, mode, dims, base, **kw)
    assert np.array_equal(cu, ocu)
    g = to_f64(t)
    err = max(np.abs(g[0] - ocos).max(), np.abs(g[1] - osin).max())
    log(f"  max |table - oracle| = {err:.3e}")
    assert err <= TABLE_TOL


def test_linspace_over_the_extent_is_the_grid():
    """start 0, stop = the extent: the GPU's linspace table equals its grid table bit for bit."""
    import torch

    seg = [(10, 30, 54, 16200)]
    g, _ = device_table(seg, GRID, (32, 32, 32), 10000.0)
    l, _ = device_table(seg, LINSPACE, (32, 32, 32), 10000.0, start=(0, 0, 0), stop=(10, 30, 54))
    assert torch.equal(g, l)
    g2 = torch.empty_like(g)
    h3a().build_rope_table(seg, (32, 32, 32), 10000.0, g2)
    torch.cuda.synchronize()
    assert torch.equal(g, g2)


def test_normalized_suffix_is_identity():
    seg = [(4, 16, 16, 1024 + 5), (1, 1, 1, 3)]
    t, _ = device_table(seg, NORMALIZED, (16, 16, 16), 100.0)
    g = to_f64(t)
    for rows in (slice(1024, 1029), slice(1029, 1032)):
        assert np.all(g[0, rows] == 1.0) and np.all(g[1, rows] == 0.0)


def run_chain(w, T):
    import torch

    q, k, v = (to_device(x, w.dtype) for x in (T.q, T.k, T.v))
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    cu = h3a().build_rope_table_ex(w.segments, w.rope_mode, w.rot_dims, w.base, tab, start=w.lin_start,
                                   stop=w.lin_stop)
    h3a().qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim)
    o = h3a().varlen_attn_fwd(q, k, v, cu, w.scale)
    torch.cuda.synchronize()
    return to_f64(q), to_f64(k), to_f64(o), cu


@pytest.mark.parametrize("name", sorted(configs.MODE_WORKLOADS))
def test_mode_workload_chain(name):
    w = configs.MODE_WORKLOADS[name]
    T = configs.make_tensors(w)
    log(f"[mode chain] {name} S={w.tokens} H={w.heads} D={w.head_dim} R={w.rot_dim} mode={w.rope_mode}")
    qn_g, kn_g, o, cu = run_chain(w, T)
    qf, kf, vf = (rng.as_f64(x, w.dtype) for x in (T.q, T.k, T.v))
    ocu, cos, sin = oracle.rope_table_mode(w.segments, w.rope_mode, w.rot_dims, w.base, start=w.lin_start,
                                           stop=w.lin_stop)
    assert np.array_equal(cu, ocu)
    qn, kn = oracle.qk_rmsnorm_rope(qf, kf, T.gamma_q, T.gamma_k, w.eps, cos, sin, w.rot_dim)
    compare(qn_g, qn, w.dtype, "q'")
    compare(kn_g, kn, w.dtype, "k'")
    # attention on the GPU's own q', k' (widened exactly), then end to end
    compare(o, oracle.varlen_attention(qn_g, kn_g, vf, ocu, w.scale), w.dtype, "o (from the GPU's q', k')")
    rows = sample_rows(ocu, every=13)
    compare(o[rows], oracle.varlen_attention_rows(qn, kn, vf, ocu, w.scale, rows), w.dtype, "o end to end")
