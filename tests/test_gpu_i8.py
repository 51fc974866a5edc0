"""GPU parity of the INT8 score product (per-token q scales, per-64-key-block k
scales of each segment) against the oracle's section 5e.

The quantisers are compared byte for byte (codes) and bit for bit (fp32
scales) with the oracle on N(0,1) rows, rows at magnitudes from 2^-60 to 2^60,
exact rounding ties, zero rows, bf16-subnormal rows and non-finite values;
the key quantiser on segments of every length class.  The attention is
compared with attention on the values the codes stand for at the bf16
tolerance (the int32 score sums are exact; the rest is the bf16 path), over
the edge packing x D 64/128 x grouped K/V x causal, with forced key-range
splits, at magnitudes far from one, and for NaN propagation; the chain
(table -> norm + rotary -> INT8 codes -> attention) against exact attention
within the oracle's own INT8 error plus the bf16 tolerance."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import configs, rng
from tests.gpu_util import TOL_BF16_MEANREL, compare, log, require_gpu, sample_rows, to_device, to_f64

pytestmark = pytest.mark.gpu

EDGE_LENS = [1, 63, 64, 65, 127, 128, 129, 0, 255, 256, 257, 700]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    h3a().release_caches()


def h3a():
    import packed_varlen_attention_head_amd as m

    return m


def _f32_bits_to_bf16(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp32 values that are bf16-representable."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _inputs(seed, lens, Hq, Hkv, D):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S = int(cu[-1])
    q = rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), "bf16")
    k = rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), "bf16")
    v = rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), "bf16")
    return cu, q, k, v


def special_rows(D: int) -> np.ndarray:
    """bf16 rows [n, D]: N(0,1) at magnitudes 2^-60..2^60, rows whose maximum is 127 with
    halves between integers (exact ties of x * 127 / amax), zero rows, bf16-subnormal rows,
    and rows holding a NaN, +inf or -inf."""
    r = np.random.default_rng(7)
    rows = []
    for e in range(-60, 61, 10):
        rows.append(r.normal(size=D) * 2.0 ** e)
    for _ in range(4):
        t = np.floor(r.uniform(-126, 126, size=D)) + 0.5  # x.5: ties to even under the unit scale
        t[r.integers(D)] = 127.0
        rows.append(t)
    rows.append(np.zeros(D))
    sub = r.integers(1, 127, size=D) * 2.0 ** -133  # bf16 subnormals (below 2^-126)
    rows.append(sub * np.where(r.random(D) < 0.5, -1.0, 1.0))
    for bad in (np.nan, np.inf, -np.inf):
        x = r.normal(size=D)
        x[3] = bad
        rows.append(x)
    x32 = np.asarray(rows, dtype=np.float32)
    fin = np.isfinite(x32)
    bits = np.zeros(x32.shape, dtype=np.uint16)
    bits[fin] = oracle_bf16_bits(x32[fin])
    bits[~fin] = _f32_bits_to_bf16(x32[~fin])
    return bits


def oracle_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp32 values rounded to nearest even (for building inputs)."""
    u = x32.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _codes_and_scales_equal(got_c, got_s, want_c, want_s, what):
    import torch

    gc = got_c.cpu().numpy()
    gs = got_s.cpu().numpy()
    assert np.array_equal(gc, want_c), f"{what}: {int((gc != want_c).sum())} codes differ"
    same = (gs.view(np.uint32) == want_s.view(np.uint32)) | (np.isnan(gs) & np.isnan(want_s))
    assert same.all(), f"{what}: scales differ at {np.argwhere(~same)[:5].tolist()}"
    assert torch.is_tensor(got_c)


@pytest.mark.parametrize("D", [64, 128])
def test_quantize_rows_bit_exact(D):
    rows = special_rows(D)
    n = rows.shape[0]
    H = 3
    x = np.zeros((n, H, D), dtype=np.uint16)
    x[:, 0] = rows
    x[:, 1] = rows[::-1]
    x[:, 2] = rng.normal_tensor(31, rng.TAG_Q, (n, D), "bf16")
    log(f"[i8 rows] D={D} rows={n}")
    c, s = h3a().quantize_i8_rows(to_device(x, "bf16"))
    wc, ws = oracle.i8_quantize_rows(rng.as_f64(x, "bf16"))
    _codes_and_scales_equal(c, s, wc, ws, "q rows")
    # and on a long random tensor with a token stride wider than a row
    S = 1000
    xb = rng.normal_tensor(32, rng.TAG_Q, (S, 4, D), "bf16")
    xd = to_device(xb, "bf16")
    c, s = h3a().quantize_i8_rows(xd)
    wc, ws = oracle.i8_quantize_rows(rng.as_f64(xb, "bf16"))
    _codes_and_scales_equal(c, s, wc, ws, "q rows, N(0,1)")


@pytest.mark.parametrize("D", [64, 128])
def test_quantize_key_blocks_bit_exact(D):
    import torch

    lens = EDGE_LENS + [1000, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S, H = int(cu[-1]), 2
    x = rng.normal_tensor(33, rng.TAG_K, (S, H, D), "bf16")
    # a segment at 2^40, one at 2^-40, specials inside blocks of the 700-key segment
    mags = np.repeat(2.0 ** np.array([0, 0, 40, 0, 0, 0, 0, 0, -40, 0, 0, 0, 0, 0], dtype=np.float64)[:len(lens)],
                     lens)
    xf = rng.as_f64(x, "bf16") * mags[:, None, None]
    x = oracle_bf16_bits(xf.astype(np.float32))
    a700 = int(cu[EDGE_LENS.index(700)])
    special = special_rows(D)
    x[a700 + 64: a700 + 64 + len(special), 1] = special  # one 64-key block gets them all
    x[a700 + 200, 0, 5] = _f32_bits_to_bf16(np.array([np.nan], np.float32))[0]
    log(f"[i8 keys] D={D} S={S} blocks={h3a().i8_key_blocks(cu)}")
    c, s = h3a().quantize_i8_keys(to_device(x, "bf16"), cu)
    wc, ws = oracle.i8_quantize_key_blocks(rng.as_f64(x, "bf16"), cu)
    _codes_and_scales_equal(c, s, wc, ws, "k blocks")
    assert torch.isnan(s[0, oracle.i8_key_blocks(cu)[EDGE_LENS.index(700)] + 3])


def gpu_i8qk(qb, kb, vb, cu, scale, causal=False):
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    return h3a().varlen_attn_fwd_i8qk(h3a().quantize_i8_rows(q), h3a().quantize_i8_keys(k, cu), v, cu, scale,
                                      causal=causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (6, 2)])
def test_i8qk_vs_oracle(D, Hq, Hkv, causal):
    cu, qb, kb, vb = _inputs(1300 + D + Hq + causal, EDGE_LENS, Hq, Hkv, D)
    log(f"[i8qk] D={D} Hq={Hq} Hkv={Hkv} causal={causal} S={int(cu[-1])}")
    scale = 1.0 / np.sqrt(D)
    o = to_f64(gpu_i8qk(qb, kb, vb, cu, scale, causal))
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    compare(o, oracle.varlen_attention_i8qk(qf, kf, vf, cu, scale, causal=causal), "bf16", "o vs INT8 oracle")


@pytest.mark.parametrize("qmag,kmag", [(1e-3, 1e3), (1e3, 1e-3), (1e-2, 1e-2)])
def test_i8qk_magnitudes_far_from_one(qmag, kmag):
    """The scales carry the range: q and k far from magnitude one, scores of order one."""
    lens = [700, 129, 1]
    cu, qb, kb, vb = _inputs(1311, lens, 4, 2, 128)
    qf = rng.as_f64(qb, "bf16") * qmag
    kf = rng.as_f64(kb, "bf16") * kmag
    qb, kb = oracle_bf16_bits(qf.astype(np.float32)), oracle_bf16_bits(kf.astype(np.float32))
    scale = 1.0 / np.sqrt(128) / (qmag * kmag)
    o = to_f64(gpu_i8qk(qb, kb, vb, cu, scale))
    ref = oracle.varlen_attention_i8qk(rng.as_f64(qb, "bf16"), rng.as_f64(kb, "bf16"), rng.as_f64(vb, "bf16"), cu,
                                       scale)
    compare(o, ref, "bf16", f"o, q at {qmag}, k at {kmag}")


def test_i8qk_split_plans_and_determinism():
    import torch

    cu, qb, kb, vb = _inputs(1321, EDGE_LENS + [3000], 4, 2, 128)
    scale = 0.088
    a = gpu_i8qk(qb, kb, vb, cu, scale)
    b = gpu_i8qk(qb, kb, vb, cu, scale)
    assert torch.equal(a, b)
    h3a().set_split_policy(h3a().H3A_SPLIT_ALWAYS)
    try:
        o = to_f64(gpu_i8qk(qb, kb, vb, cu, scale))
    finally:
        h3a().set_split_policy(h3a().H3A_SPLIT_AUTO)
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    compare(o, oracle.varlen_attention_i8qk(qf, kf, vf, cu, scale), "bf16", "o (split plan) vs INT8 oracle")


def test_i8qk_nan_propagation():
    """A NaN query element poisons its row's scale: that query row (every head dim) is NaN;
    a NaN key element poisons its 64-key block's scale: every row of its segment and head is
    NaN; every other element is finite.  Outside the 32-row wave of the NaN row nothing
    changes bit for bit; inside it the NaN lane sends the wave through the rare rescale
    path, whose other rows are then rounded against another reference (bf16 tolerance)."""
    import torch

    lens = [150, 77, 29]
    cu, qb, kb, vb = _inputs(1331, lens, 2, 2, 128)
    base = gpu_i8qk(qb, kb, vb, cu, 0.088)
    nan = _f32_bits_to_bf16(np.array([np.nan], np.float32))[0]
    q2, k2 = qb.copy(), kb.copy()
    q2[10, 1, 7] = nan          # segment 0, head 1, row 10
    k2[150 + 70, 0, 3] = nan    # segment 1 (keys 150..226), head 0, block 1
    o = gpu_i8qk(q2, k2, vb, cu, 0.088)
    bad = torch.zeros(o.shape, dtype=torch.bool, device=o.device)
    bad[10, 1] = True
    bad[150:227, 0] = True
    assert torch.isnan(o[bad]).all() and not torch.isnan(o[~bad]).any()
    wave = torch.zeros_like(bad)
    wave[0:32, 1] = True  # rows 0..31 of segment 0, head 1: the NaN row's wave
    keep = ~bad & ~wave
    assert torch.equal(o[keep], base[keep])
    near = ~bad & wave
    compare(to_f64(o[near]), to_f64(base[near]), "bf16", "the NaN row's wave mates")


@pytest.mark.parametrize("name,kv", [("h3_s20423_bf16", 24), ("two_seg_bf16", 8), ("vit3d_tiles_bf16", 8)])
def test_fused_norm_rope_i8q_equals_two_passes(name, kv):
    """The norm + rotary pass writing q as INT8 codes and per-token scales gives the same
    bytes as the bf16 pass followed by the row quantiser (and k_out the same bf16 values,
    also in place), on q holding a zero row, a NaN and an infinity; q is left untouched."""
    import torch

    w = configs.BF16[name].replace(kv_heads=kv)
    T = configs.make_tensors(w)
    log(f"[fused i8q] {name} Hq={w.heads} Hk={w.kv} D={w.head_dim}")
    qb = T.q.copy()
    qb[5, 0] = 0
    qb[17, 1, 9] = _f32_bits_to_bf16(np.array([np.nan], np.float32))[0]
    qb[w.tokens - 1, w.heads - 1, 0] = _f32_bits_to_bf16(np.array([np.inf], np.float32))[0]
    q, k = to_device(qb, "bf16"), to_device(T.k, "bf16")
    q0, k0 = q.clone(), k.clone()
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    h3a().build_rope_table_ex(w.segments, w.rope_mode, w.rot_dims, w.base, tab, start=w.lin_start, stop=w.lin_stop)
    (q8, qs), kn_f = h3a().qk_rmsnorm_rope_i8q(q, k, gq, gk, w.eps, tab, w.rot_dim)
    qn, kn = torch.empty_like(q), torch.empty_like(k)
    h3a().qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim, q_out=qn, k_out=kn)
    q8b, qsb = h3a().quantize_i8_rows(qn)
    torch.cuda.synchronize()
    # bit patterns: q holds a NaN
    assert torch.equal(q.view(torch.int16), q0.view(torch.int16)) and torch.equal(k, k0)
    assert torch.equal(kn_f, kn)
    _codes_and_scales_equal(q8, qs, q8b.cpu().numpy(), qsb.cpu().numpy(), "fused q rows")
    assert qs[0, 5] == 0 and torch.isnan(qs[1, 17]) and not torch.isfinite(qs[w.heads - 1, w.tokens - 1])
    # k in place, q8 written into a wider token stride
    wide = torch.zeros((w.tokens, w.heads + 1, w.head_dim), dtype=torch.int8, device="cuda")
    (q8w, qsw), kk = h3a().qk_rmsnorm_rope_i8q(q, k, gq, gk, w.eps, tab, w.rot_dim, q8=wide[:, :w.heads],
                                                k_out=k)
    torch.cuda.synchronize()
    assert kk is k and torch.equal(k, kn)
    assert torch.equal(q8w, q8) and torch.equal(wide[:, w.heads], torch.zeros_like(wide[:, w.heads]))
    _codes_and_scales_equal(q8w, qsw, q8.cpu().numpy(), qs.cpu().numpy(), "fused q rows, strided")


@pytest.mark.parametrize("name", ["two_seg_bf16", "h3_s20423_bf16"])
def test_i8qk_chain(name):
    """table -> norm + rotary -> INT8 q', k' -> INT8-score attention, against the oracle's
    attention on its own q', k' stored in bf16 and quantised (bf16 tolerance), and against
    exact attention within the oracle's own INT8 error on the same rows plus the bf16
    path's mean-rel tolerance."""
    import torch

    w = configs.ALL[name]
    T = configs.make_tensors(w)
    log(f"[i8 chain] {name} S={w.tokens}")
    q, k, v = (to_device(x, w.dtype) for x in (T.q, T.k, T.v))
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    cu = h3a().build_rope_table(w.segments, w.rot_dims, w.base, tab)
    # the fused q path (norm + rotary writing INT8 q), then the bf16 pass (in place) and the
    # row quantiser: the same output bit for bit
    q8f, kn_f = h3a().qk_rmsnorm_rope_i8q(q, k, gq, gk, w.eps, tab, w.rot_dim)
    o_f = h3a().varlen_attn_fwd_i8qk(q8f, h3a().quantize_i8_keys(kn_f, cu), v, cu, w.scale)
    qn_d, kn_d = h3a().qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim)
    o_d = h3a().varlen_attn_fwd_i8qk(h3a().quantize_i8_rows(qn_d), h3a().quantize_i8_keys(kn_d, cu), v, cu, w.scale)
    assert torch.equal(o_f, o_d)
    o = to_f64(o_d)
    qf, kf, vf = (rng.as_f64(x, w.dtype) for x in (T.q, T.k, T.v))
    ocu, cos, sin = oracle.rope_table(w.segments, w.rot_dims, w.base)
    qn, kn = oracle.qk_rmsnorm_rope(qf, kf, T.gamma_q, T.gamma_k, w.eps, cos, sin, w.rot_dim)
    rows = sample_rows(ocu, every=97)
    qi, ki = oracle.i8_round_q(oracle.bf16_round(qn)), oracle.i8_round_k(oracle.bf16_round(kn), ocu)
    ref_i8 = oracle.varlen_attention_rows(qi, ki, vf, ocu, w.scale, rows)
    compare(o[rows], ref_i8, "bf16", f"o vs INT8 oracle ({len(rows)} rows)")
    exact = oracle.varlen_attention_rows(qn, kn, vf, ocu, w.scale, rows)
    own = float(np.abs(ref_i8 - exact).sum() / np.abs(exact).sum())
    got = float(np.abs(o[rows] - exact).sum() / np.abs(exact).sum())
    log(f"  mean-rel vs exact attention: {got:.3e} (oracle's INT8 rounding alone: {own:.3e})")
    assert got <= own + TOL_BF16_MEANREL, (got, own)
    assert own < 0.02, own  # per-token / per-block INT8: several times below E4M3 scores
