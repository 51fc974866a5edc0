"""GPU parity of the low-precision path: the E4M3 quantiser bit for bit against
the oracle's codec, FP8-score attention against the oracle's attention on
E4M3-rounded q and k (the bf16 path's tolerance), and the whole chain against
exact attention at the stated looser tolerance."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import configs, rng
from tests.gpu_util import compare, log, require_gpu, sample_rows, to_device, to_f64

pytestmark = pytest.mark.gpu

# FP8-score attention against exact attention (three mantissa bits per q, k
# element): measured on the oracle at 3.9e-2 mean-rel and 1.6e-2 max abs on
# the S = 20,423 inputs.
TOL_FP8_ABS = 5e-2
TOL_FP8_MEANREL = 6e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()


def h3a():
    import packed_varlen_attention_head_amd as m

    return m


def bf16_specials() -> np.ndarray:
    """bf16 bit patterns: every finite E4M3 value and the midpoints between neighbours
    (both representable in bf16), one bf16 step either side of each midpoint, values past
    448, subnormal-range and tiny values, signed zeros."""
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = 0.5 * (pos[1:] + pos[:-1])
    vals = np.concatenate([pos, mids, [448.0, 449.0, 464.0, 480.0, 1e4, 3e38, 2.0 ** -10, 2.0 ** -12, 1e-30]])
    vals = np.concatenate([vals, -vals])
    bits = rng.f32_to_bf16_bits(vals.astype(np.float32))
    mid_bits = rng.f32_to_bf16_bits(np.concatenate([mids, -mids]).astype(np.float32))
    extra = np.concatenate([mid_bits + 1, mid_bits - 1, np.array([0x0000, 0x8000], dtype=np.uint16)])
    return np.concatenate([bits, extra.astype(np.uint16)])


def test_quantize_codes_bit_exact():
    import torch

    special = bf16_specials()
    scales = [1e-3, 0.05, 1.0, 7.0, 60.0, 300.0]
    rand = np.concatenate([rng.normal_tensor(11, rng.TAG_Q, (4096,), "bf16", 0.0, s) for s in scales])
    bits = np.concatenate([special, rand])
    D = 128
    S = -(-len(bits) // D)
    bits = np.concatenate([bits, np.zeros(S * D - len(bits), dtype=np.uint16)]).reshape(S, 1, D)
    x = to_device(bits, "bf16")
    # padded output rows: 128 code bytes + 128 guard bytes
    ybuf = torch.full((S, 2 * D), 0xA5, dtype=torch.uint8, device="cuda")
    y = ybuf[:, :D].view(S, 1, D)
    h3a().quantize_e4m3(x, out=y)
    torch.cuda.synchronize()
    got = y.cpu().numpy().reshape(-1)
    want = oracle.e4m3_encode(rng.bf16_bits_to_f32(bits).astype(np.float64)).reshape(-1)
    bad = np.nonzero(got != want)[0]
    log(f"[quantize] {got.size} codes, {len(bad)} mismatches")
    assert len(bad) == 0, (bad[:8], got[bad[:8]], want[bad[:8]])
    assert torch.all(ybuf[:, D:] == 0xA5)


def _gpu_fp8_attention(qb, kb, vb, cu, scale, causal):
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    q8, k8 = h3a().quantize_e4m3(q), h3a().quantize_e4m3(k)
    return h3a().varlen_attn_fwd_fp8qk(q8, k8, v, cu, scale, causal=causal)


EDGE_LENS = [1, 63, 64, 65, 127, 128, 129, 0, 255, 256, 257, 700]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8qk_vs_quantized_oracle(D, Hq, Hkv, causal):
    """Seeded bf16 q, k, v: the GPU quantises and attends; the oracle attends on the
    same operands rounded to E4M3 (its own codec), exactly."""
    cu = np.concatenate([[0], np.cumsum(EDGE_LENS)]).astype(np.int64)
    S = int(cu[-1])
    seed = 300 + D + Hq + (1 if causal else 0)
    log(f"[fp8qk] D={D} Hq={Hq} Hkv={Hkv} causal={causal} S={S} seed={seed}")
    qb = rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), "bf16")
    kb = rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), "bf16")
    vb = rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), "bf16")
    scale = 1.0 / np.sqrt(D)
    o = to_f64(_gpu_fp8_attention(qb, kb, vb, cu, scale, causal))
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    compare(o, oracle.varlen_attention_fp8qk(qf, kf, vf, cu, scale, causal=causal), "bf16", "o vs E4M3 oracle")


@pytest.mark.parametrize("name", ["two_seg_bf16", "h3_s20423_bf16"])
def test_fp8qk_chain(name):
    """table -> norm + rotary (bf16) -> E4M3 q', k' -> FP8-score attention, against the
    oracle's attention on its own q', k' stored in bf16 and rounded to E4M3 (the code
    decision in the kernel's precision; bf16 tolerance) and against exact attention (the
    looser FP8 tolerance)."""
    import torch

    w = configs.ALL[name]
    T = configs.make_tensors(w)
    log(f"[fp8 chain] {name} S={w.tokens}")
    q, k, v = (to_device(x, w.dtype) for x in (T.q, T.k, T.v))
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    cu = h3a().build_rope_table(w.segments, w.rot_dims, w.base, tab)
    h3a().qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim)
    q8, k8 = h3a().quantize_e4m3(q), h3a().quantize_e4m3(k)
    o = to_f64(h3a().varlen_attn_fwd_fp8qk(q8, k8, v, cu, w.scale))
    qf, kf, vf = (rng.as_f64(x, w.dtype) for x in (T.q, T.k, T.v))
    ocu, cos, sin = oracle.rope_table(w.segments, w.rot_dims, w.base)
    qn, kn = oracle.qk_rmsnorm_rope(qf, kf, T.gamma_q, T.gamma_k, w.eps, cos, sin, w.rot_dim)
    rows = sample_rows(ocu, every=97)
    # the codes are decided from q', k' stored in bf16, as on the GPU
    q8o, k8o = (oracle.e4m3_round(oracle.bf16_round(x)) for x in (qn, kn))
    ref_q = oracle.varlen_attention_rows(q8o, k8o, vf, ocu, w.scale, rows)
    compare(o[rows], ref_q, "bf16", f"o vs E4M3 oracle ({len(rows)} rows)")
    ref = oracle.varlen_attention_rows(qn, kn, vf, ocu, w.scale, rows)
    err = np.abs(o[rows] - ref)
    max_abs, mean_rel = float(err.max()), float(err.sum() / np.abs(ref).sum())
    log(f"  o vs exact attention: max_abs={max_abs:.3e} mean_rel={mean_rel:.3e}")
    assert max_abs <= TOL_FP8_ABS and mean_rel <= TOL_FP8_MEANREL


def test_fp8qk_segment_isolation_and_determinism():
    import torch

    lens = [900, 500]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S, H, D = 1400, 4, 128
    qb = rng.normal_tensor(5, rng.TAG_Q, (S, H, D), "bf16")
    kb = rng.normal_tensor(5, rng.TAG_K, (S, H, D), "bf16")
    vb = rng.normal_tensor(5, rng.TAG_V, (S, H, D), "bf16")
    a = _gpu_fp8_attention(qb, kb, vb, cu, 0.088, False)
    b = _gpu_fp8_attention(qb, kb, vb, cu, 0.088, False)
    kb2 = kb.copy()
    kb2[1000] ^= 0x0040
    c = _gpu_fp8_attention(qb, kb2, vb, cu, 0.088, False)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(a[:900], c[:900]) and not torch.equal(a[900:], c[900:])


@pytest.mark.parametrize("name,kv", [("h3_s20423_bf16", 24), ("two_seg_bf16", 8)])
def test_fused_norm_rope_e4m3_equals_two_passes(name, kv):
    """The norm + rotary pass that writes E4M3 codes gives the same bytes as the bf16 pass
    followed by the quantiser, and leaves q, k untouched."""
    import torch

    w = configs.ALL[name].replace(kv_heads=kv)
    T = configs.make_tensors(w)
    log(f"[fused e4m3] {name} Hq={w.heads} Hk={w.kv}")
    q, k = to_device(T.q, "bf16"), to_device(T.k, "bf16")
    q0, k0 = q.clone(), k.clone()
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    h3a().build_rope_table(w.segments, w.rot_dims, w.base, tab)
    q8, k8 = h3a().qk_rmsnorm_rope_e4m3(q, k, gq, gk, w.eps, tab, w.rot_dim)
    qn, kn = torch.empty_like(q), torch.empty_like(k)
    h3a().qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim, q_out=qn, k_out=kn)
    q8b, k8b = h3a().quantize_e4m3(qn), h3a().quantize_e4m3(kn)
    torch.cuda.synchronize()
    assert torch.equal(q, q0) and torch.equal(k, k0)
    assert torch.equal(q8, q8b) and torch.equal(k8, k8b)


# Both products in FP8: the probabilities are rounded to E4M3 as well, each by
# at most 2^-4 of itself (three mantissa bits, nearest even), so against
# attention on E4M3 q, k, v with exact weights an output element moves by at
# most 2^-4 sum_j p_j |v_j| / sum_j p_j -- attention on |v| -- plus the bf16
# path's own rounding (TOL_BF16_ABS).  On the oracle the weight rounding moves
# the S = 5,120 outputs by 2.6e-2 mean-rel; the whole FP8 path sits at 5.3e-2
# mean-rel from exact attention, with max abs 2.1e-2 (S = 5,120) and 4.8e-2
# (S = 20,423 sampled rows, whose short segments have the largest outputs).
P_ROUND = 2.0 ** -4
TOL_FP8PV_MEANREL = 4e-2
TOL_FP8_EXACT_ABS, TOL_FP8_EXACT_MEANREL = 1e-1, 8e-2


def expected_vt(vbits: np.ndarray, cu) -> np.ndarray:
    """The transposed, segment-padded E4M3 layout built from the oracle's codec."""
    S, H, D = vbits.shape
    codes = oracle.e4m3_encode(rng.bf16_bits_to_f32(vbits).astype(np.float64))
    lens = np.diff(np.asarray(cu))
    pad = (lens + 63) // 64 * 64
    out = np.zeros((H, D, int(pad.sum())), dtype=np.uint8)
    col = 0
    for s, L in enumerate(lens):
        a = int(cu[s])
        out[:, :, col:col + L] = codes[a:a + L].transpose(1, 2, 0)
        col += int(pad[s])
    return out


def check(g, r, what, tol_abs, tol_rel):
    """tol_abs: a number, or an elementwise bound of the same shape as r."""
    err = np.abs(g - r)
    max_abs, mean_rel = float(err.max()), float(err.sum() / np.abs(r).sum())
    worst = float(np.max(err - tol_abs))
    log(f"  {what}: max_abs={max_abs:.3e} mean_rel={mean_rel:.3e} max(err - bound)={worst:.3e} n={err.size}")
    assert np.all(np.isfinite(g))
    assert worst <= 0 and mean_rel <= tol_rel, (max_abs, mean_rel, worst)


def weight_rounding_bound(ref_abs_v):
    from tests.gpu_util import TOL_BF16_ABS

    return P_ROUND * ref_abs_v + TOL_BF16_ABS


@pytest.mark.parametrize("D", [64, 128])
def test_prepare_vt_layout_bit_exact(D):
    import torch

    lens = [1, 63, 64, 65, 0, 129, 700]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S, H = int(cu[-1]), 3
    vb = rng.normal_tensor(41 + D, rng.TAG_V, (S, H, D), "bf16", 0.0, 30.0)  # wide enough to saturate some
    vt = h3a().prepare_vt_e4m3(to_device(vb, "bf16"), cu)
    torch.cuda.synchronize()
    want = expected_vt(vb, cu)
    got = vt.cpu().numpy()
    log(f"[vt layout] D={D} columns={want.shape[2]} mismatches={int(np.sum(got != want))}")
    assert got.shape == want.shape and np.array_equal(got, want)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_vs_operand_oracle(D, Hq, Hkv, causal):
    cu = np.concatenate([[0], np.cumsum(EDGE_LENS)]).astype(np.int64)
    S = int(cu[-1])
    seed = 500 + D + Hq + (1 if causal else 0)
    log(f"[fp8 pv] D={D} Hq={Hq} Hkv={Hkv} causal={causal} S={S} seed={seed}")
    qb = rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), "bf16")
    kb = rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), "bf16")
    vb = rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), "bf16")
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    o = h3a().varlen_attn_fwd_fp8(h3a().quantize_e4m3(q), h3a().quantize_e4m3(k), h3a().prepare_vt_e4m3(v, cu), cu,
                                  1.0 / np.sqrt(D), causal=causal)
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    ref = oracle.varlen_attention_fp8(qf, kf, vf, cu, 1.0 / np.sqrt(D), causal=causal)
    ref_abs_v = oracle.varlen_attention_fp8(qf, kf, np.abs(vf), cu, 1.0 / np.sqrt(D), causal=causal)
    check(to_f64(o), ref, "o vs E4M3-operand oracle", weight_rounding_bound(ref_abs_v), TOL_FP8PV_MEANREL)


@pytest.mark.parametrize("name", ["two_seg_bf16", "h3_s20423_bf16"])
def test_fp8_chain(name):
    import torch

    w = configs.ALL[name]
    T = configs.make_tensors(w)
    log(f"[fp8 full chain] {name} S={w.tokens}")
    q, k, v = (to_device(x, w.dtype) for x in (T.q, T.k, T.v))
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    cu = h3a().build_rope_table(w.segments, w.rot_dims, w.base, tab)
    q8, k8 = h3a().qk_rmsnorm_rope_e4m3(q, k, gq, gk, w.eps, tab, w.rot_dim)
    o = to_f64(h3a().varlen_attn_fwd_fp8(q8, k8, h3a().prepare_vt_e4m3(v, cu), cu, w.scale))
    qf, kf, vf = (rng.as_f64(x, w.dtype) for x in (T.q, T.k, T.v))
    ocu, cos, sin = oracle.rope_table(w.segments, w.rot_dims, w.base)
    qn, kn = oracle.qk_rmsnorm_rope(qf, kf, T.gamma_q, T.gamma_k, w.eps, cos, sin, w.rot_dim)
    rows = sample_rows(ocu, every=97)
    q8o, k8o = (oracle.e4m3_round(oracle.bf16_round(x)) for x in (qn, kn))
    ref8 = oracle.varlen_attention_rows(q8o, k8o, oracle.e4m3_round(vf), ocu, w.scale, rows)
    ref8_abs = oracle.varlen_attention_rows(q8o, k8o, np.abs(oracle.e4m3_round(vf)), ocu, w.scale, rows)
    check(o[rows], ref8, f"o vs E4M3-operand oracle ({len(rows)} rows)", weight_rounding_bound(ref8_abs),
          TOL_FP8PV_MEANREL)
    ref = oracle.varlen_attention_rows(qn, kn, vf, ocu, w.scale, rows)
    check(o[rows], ref, "o vs exact attention", TOL_FP8_EXACT_ABS, TOL_FP8_EXACT_MEANREL)


def test_many_segments_fp8_layout_and_attention():
    """150 ragged segments (three launches of the V-layout pass), grouped K/V."""
    import torch

    lens = [int(x) for x in 1 + (rng.uniform(77, rng.TAG_LENS, 150) * 300).astype(np.int64)]
    lens[7] = 0
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S, Hq, Hkv, D = int(cu[-1]), 4, 2, 64
    log(f"[fp8 many segments] S={S} nseg={len(lens)}")
    qb = rng.normal_tensor(78, rng.TAG_Q, (S, Hq, D), "bf16")
    kb = rng.normal_tensor(78, rng.TAG_K, (S, Hkv, D), "bf16")
    vb = rng.normal_tensor(78, rng.TAG_V, (S, Hkv, D), "bf16")
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    vt = h3a().prepare_vt_e4m3(v, cu)
    torch.cuda.synchronize()
    assert np.array_equal(vt.cpu().numpy(), expected_vt(vb, cu))
    o = h3a().varlen_attn_fwd_fp8(h3a().quantize_e4m3(q), h3a().quantize_e4m3(k), vt, cu, 0.125)
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    ref = oracle.varlen_attention_fp8(qf, kf, vf, cu, 0.125)
    ref_abs = oracle.varlen_attention_fp8(qf, kf, np.abs(vf), cu, 0.125)
    check(to_f64(o), ref, "o vs E4M3-operand oracle", weight_rounding_bound(ref_abs), TOL_FP8PV_MEANREL)
