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
from tests.test_gpu_fp8 import TOL_FP8PV_MEANREL, weight_rounding_bound
from tests.test_gpu_fp8 import check as check_bound

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


# ---------------------------------------------------------------------------
# INT8 scores with the PV product in FP8 (E4M3 weights, transposed E4M3 V)


def gpu_i8qk_fp8pv(qb, kb, vb, cu, scale, causal=False):
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    return h3a().varlen_attn_fwd_i8qk_fp8pv(h3a().quantize_i8_rows(q), h3a().quantize_i8_keys(k, cu),
                                           h3a().prepare_vt_e4m3(v, cu), cu, scale, causal=causal)


def i8_mx_operands(qb, kb, vb, cu):
    """The oracle's INT8-rounded q (per token), k (per 64-key block) and E4M3-rounded v (per
    32-key block of each segment)."""
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    return oracle.i8_round_q(qf), oracle.i8_round_k(kf, cu), oracle.mx_round_keys(vf, cu)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2)])
def test_i8qk_fp8pv_vs_oracle(D, Hq, Hkv, causal):
    """Against attention on the oracle's rounded operands (varlen_attention_i8qk_mxv), within
    the per-element bound of the weights' E4M3 rounding."""
    cu, qb, kb, vb = _inputs(900 + D + Hq + (1 if causal else 0), EDGE_LENS, Hq, Hkv, D)
    log(f"[i8qk fp8pv] D={D} Hq={Hq} Hkv={Hkv} causal={causal} S={int(cu[-1])}")
    o = to_f64(gpu_i8qk_fp8pv(qb, kb, vb, cu, 1.0 / np.sqrt(D), causal))
    bound, ref = weight_rounding_bound(*i8_mx_operands(qb, kb, vb, cu), cu, 1.0 / np.sqrt(D), causal)
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    assert np.allclose(ref, oracle.varlen_attention_i8qk_mxv(qf, kf, vf, cu, 1.0 / np.sqrt(D), causal),
                       rtol=0, atol=1e-12)
    check_bound(o, ref, "o vs INT8 + E4M3 oracle", bound, TOL_FP8PV_MEANREL)


@pytest.mark.parametrize("vmag", [1e-3, 1e3])
def test_i8qk_fp8pv_magnitudes_far_from_one(vmag):
    """v at 1e-3 and 1e3, q at 1e-3 and k at 1e3: the scales keep every operand's relative
    precision, so the outputs divided by vmag meet the magnitude-one bounds."""
    cu = np.concatenate([[0], np.cumsum([300, 129, 64, 1, 700])]).astype(np.int64)
    S, Hq, Hkv, D = int(cu[-1]), 4, 2, 128
    seed = 950 + (1 if vmag > 1 else 0)
    log(f"[i8qk fp8pv magnitudes] v*{vmag:g} q*1e-3 k*1e3 S={S}")

    def scaled(tag, shape, m):
        return rng.f32_to_bf16_bits(rng.bf16_bits_to_f32(rng.normal_tensor(seed, tag, shape, "bf16")) * np.float32(m))

    qb, kb = scaled(rng.TAG_Q, (S, Hq, D), 1e-3), scaled(rng.TAG_K, (S, Hkv, D), 1e3)
    vb = scaled(rng.TAG_V, (S, Hkv, D), vmag)
    o = to_f64(gpu_i8qk_fp8pv(qb, kb, vb, cu, 1.0 / np.sqrt(D)))
    bound, ref = weight_rounding_bound(*i8_mx_operands(qb, kb, vb, cu), cu, 1.0 / np.sqrt(D))
    check_bound(o / vmag, ref / vmag, "o / vmag vs INT8 + E4M3 oracle", bound / vmag, TOL_FP8PV_MEANREL)


@pytest.mark.parametrize("pv8", [False, True])
def test_i8qk_zero_rows_and_key_blocks(pv8):
    """All-zero query rows and an all-zero last (partial) key block have scale 0: their
    scores are 0, and the masked keys of that partial tile stay excluded (no 0 * -inf)."""
    lens = [100, 70, 129]
    cu, qb, kb, vb = _inputs(1401 + pv8, lens, 2, 2, 128)
    qb[100 + 5:100 + 10, 1] = 0      # segment 1, rows 5..9, head 1
    qb[200 + 3, 0] = 0               # segment 2, row 3, head 0
    kb[64:100, 0] = 0                # segment 0's last block (keys 64..99; tile 1 is partial), head 0
    kb[100 + 64:170, 1] = 0          # segment 1's last block (keys 64..69), head 1
    log(f"[i8 zero scales] pv8={pv8}")
    scale = 0.088
    if not pv8:
        o = to_f64(gpu_i8qk(qb, kb, vb, cu, scale))
        qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
        ref = oracle.varlen_attention_i8qk(qf, kf, vf, cu, scale)
        assert np.all(np.isfinite(o))
        compare(o, ref, "bf16", "o vs INT8 oracle, zero rows and blocks")
        return
    o = to_f64(gpu_i8qk_fp8pv(qb, kb, vb, cu, scale))
    assert np.all(np.isfinite(o))
    bound, ref = weight_rounding_bound(*i8_mx_operands(qb, kb, vb, cu), cu, scale)
    check_bound(o, ref, "o vs INT8 + E4M3 oracle, zero rows and blocks", bound, TOL_FP8PV_MEANREL)


def test_i8qk_fp8pv_split_plans_nan_and_determinism():
    """Forced key-range splits against the unsplit result (at the weights' bound: a range
    item's reference max differs), bitwise equal across runs; a NaN query element makes its
    row NaN and a NaN key element its segment's rows of that head, nothing else."""
    import torch

    lens = [3000, 700, 257]
    cu, qb, kb, vb = _inputs(1501, lens, 4, 2, 128)
    log("[i8qk fp8pv split / nan]")
    bound, ref = weight_rounding_bound(*i8_mx_operands(qb, kb, vb, cu), cu, 0.088)
    try:
        h3a().set_split_policy(h3a().H3A_SPLIT_ALWAYS)
        a = gpu_i8qk_fp8pv(qb, kb, vb, cu, 0.088)
        b = gpu_i8qk_fp8pv(qb, kb, vb, cu, 0.088)
    finally:
        h3a().set_split_policy(h3a().H3A_SPLIT_AUTO)
    assert torch.equal(a, b)
    check_bound(to_f64(a), ref, "split o vs INT8 + E4M3 oracle", bound, TOL_FP8PV_MEANREL)
    nan = _f32_bits_to_bf16(np.array([np.nan], np.float32))[0]
    q2, k2 = qb.copy(), kb.copy()
    q2[10, 1, 7] = nan
    k2[3000 + 70, 0, 3] = nan  # segment 1, kv head 0 (query heads 0, 1)
    o = gpu_i8qk_fp8pv(q2, k2, vb, cu, 0.088)
    bad = torch.zeros(o.shape, dtype=torch.bool, device=o.device)
    bad[10, 1] = True
    bad[3000:3700, 0:2] = True
    assert torch.isnan(o[bad]).all() and not torch.isnan(o[~bad]).any()


@pytest.mark.parametrize("name", ["two_seg_bf16", "h3_s20423_bf16"])
def test_i8qk_fp8pv_chain(name):
    """table -> norm + rotary writing INT8 q -> INT8 k codes, E4M3 V^T -> attention: against
    the oracle's rounded operands within the weights' bound, and against exact attention
    within the oracle's own rounding error plus 3e-2 for the E4M3 weights."""
    import torch

    w = configs.ALL[name]
    T = configs.make_tensors(w)
    log(f"[i8qk fp8pv chain] {name} S={w.tokens}")
    q, k, v = (to_device(x, w.dtype) for x in (T.q, T.k, T.v))
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    cu = h3a().build_rope_table(w.segments, w.rot_dims, w.base, tab)
    q8, kn_d = h3a().qk_rmsnorm_rope_i8q(q, k, gq, gk, w.eps, tab, w.rot_dim)
    o = to_f64(h3a().varlen_attn_fwd_i8qk_fp8pv(q8, h3a().quantize_i8_keys(kn_d, cu), h3a().prepare_vt_e4m3(v, cu),
                                                cu, w.scale))
    qf, kf, vf = (rng.as_f64(x, w.dtype) for x in (T.q, T.k, T.v))
    ocu, cos, sin = oracle.rope_table(w.segments, w.rot_dims, w.base)
    qn, kn = oracle.qk_rmsnorm_rope(qf, kf, T.gamma_q, T.gamma_k, w.eps, cos, sin, w.rot_dim)
    rows = sample_rows(ocu, every=97)
    qi, ki = oracle.i8_round_q(oracle.bf16_round(qn)), oracle.i8_round_k(oracle.bf16_round(kn), ocu)
    bound, ref8 = weight_rounding_bound(qi, ki, oracle.mx_round_keys(vf, ocu), ocu, w.scale, rows=rows)
    check_bound(o[rows], ref8, f"o vs INT8 + E4M3 oracle ({len(rows)} rows)", bound, TOL_FP8PV_MEANREL)
    exact = oracle.varlen_attention_rows(qn, kn, vf, ocu, w.scale, rows)
    own = float(np.abs(ref8 - exact).sum() / np.abs(exact).sum())
    got = float(np.abs(o[rows] - exact).sum() / np.abs(exact).sum())
    log(f"  mean-rel vs exact attention: {got:.3e} (oracle's INT8 + E4M3 operand rounding alone: {own:.3e})")
    assert got <= own + 3e-2, (got, own)


def test_many_segments_key_blocks_and_attention():
    """150 ragged segments (three launches of the key-block quantiser, 64 segments each),
    one of them empty, grouped K/V: codes and scales bit-exact, attention against the
    oracle at the bf16 tolerance."""
    lens = [int(x) for x in 1 + (rng.uniform(79, rng.TAG_LENS, 150) * 300).astype(np.int64)]
    lens[7] = 0
    cu, qb, kb, vb = _inputs(80, lens, 4, 2, 64)
    log(f"[i8 many segments] S={int(cu[-1])} nseg={len(lens)} blocks={h3a().i8_key_blocks(cu)}")
    k8 = h3a().quantize_i8_keys(to_device(kb, "bf16"), cu)
    wc, ws = oracle.i8_quantize_key_blocks(rng.as_f64(kb, "bf16"), cu)
    _codes_and_scales_equal(k8[0], k8[1], wc, ws, "k blocks, 150 segments")
    o = to_f64(gpu_i8qk(qb, kb, vb, cu, 0.125))
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    compare(o, oracle.varlen_attention_i8qk(qf, kf, vf, cu, 0.125), "bf16", "o vs INT8 oracle, 150 segments")


# ---------------------------------------------------------------------------
# centred keys (segment means subtracted before the key codes)


def _offset_keys(seed, lens, H, D, offset=20.0):
    """bf16 keys N(0,1) plus a per-(head, dim) offset of `offset` sigma, as real key
    activations carry per-channel offsets."""
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S = int(cu[-1])
    base = rng.bf16_bits_to_f32(rng.normal_tensor(seed, rng.TAG_K, (S, H, D), "bf16"))
    off = rng.bf16_bits_to_f32(rng.normal_tensor(seed + 1, rng.TAG_K, (1, H, D), "bf16")) * np.float32(offset)
    return cu, rng.f32_to_bf16_bits(base + off)


def _mean_bound(kf, cu, mu):
    """Per (segment, head, dim) bound on the fp32 mean's error: every key enters at most
    40 + chunks partial sums (a thread's 16 or 8 keys, 16 or 32 rows of thread sums, the
    chunk sums), each rounded to within 2^-24 of itself, then one division."""
    b = np.zeros_like(mu)
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        if e > a:
            nc = -(-(e - a) // 256)
            b[s] = (40 + nc) * 2.0 ** -24 * np.abs(kf[a:e]).mean(axis=0) + 1e-30
    return b


@pytest.mark.parametrize("D", [64, 128])
def test_segment_key_means(D):
    import torch

    lens = EDGE_LENS + [1000, 3000]
    cu, kb = _offset_keys(1601 + D, lens, 3, D)
    k = to_device(kb, "bf16")
    log(f"[key means] D={D} S={int(cu[-1])} chunks={h3a().i8_key_mean_chunks(cu)}")
    mu = h3a().segment_key_means(k, cu)
    mu2 = h3a().segment_key_means(k, cu)
    torch.cuda.synchronize()
    assert torch.equal(mu, mu2)  # fixed summation order
    kf = rng.as_f64(kb, "bf16")
    want = oracle.segment_key_means(kf, cu)
    got = mu.cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    bound = _mean_bound(kf, cu, want)
    log(f"  max |mu - oracle| = {err.max():.3e}, max err / bound = {(err / np.maximum(bound, 1e-300)).max():.3f}")
    assert np.all(err <= bound)
    assert np.all(got[EDGE_LENS.index(0)] == 0)


@pytest.mark.parametrize("D", [64, 128])
def test_quantize_keys_centered_bit_exact(D):
    """Given the same fp32 means, the centred key codes and scales equal the oracle's bit for bit."""
    import torch

    lens = EDGE_LENS + [1000]
    cu, kb = _offset_keys(1701 + D, lens, 2, D)
    kb[5, 1, 3] = _f32_bits_to_bf16(np.array([np.nan], np.float32))[0]
    kf = rng.as_f64(kb, "bf16")
    mu32 = oracle.segment_key_means(kf, cu).astype(np.float32)
    log(f"[centred key codes] D={D} S={int(cu[-1])}")
    c, s = h3a().quantize_i8_keys(to_device(kb, "bf16"), cu, mu=torch.from_numpy(mu32).cuda())
    wc, ws = oracle.i8_quantize_key_blocks_centered(kf, cu, mu32)
    _codes_and_scales_equal(c, s, wc, ws, "centred k blocks")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("pv8", [False, True])
def test_i8qk_centered_vs_oracle(D, causal, pv8):
    """Keys with per-channel offsets of 20 sigma, grouped K/V: INT8 attention on centred keys
    (the oracle's fp32 means) against the oracle at the bf16 tolerance (FP8 PV: within the
    weights' rounding bound); on the GPU's own means, far closer to exact attention than
    INT8 attention on the plain keys (beyond the E4M3 floor with FP8 PV)."""
    import torch

    lens = EDGE_LENS + [1000]
    cu, kb = _offset_keys(1801 + D + 2 * causal + 4 * pv8, lens, 2, D)
    S = int(cu[-1])
    qb = rng.normal_tensor(1802 + D, rng.TAG_Q, (S, 4, D), "bf16")
    vb = rng.normal_tensor(1803 + D, rng.TAG_V, (S, 2, D), "bf16")
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    scale = 1.0 / np.sqrt(D)
    mu32 = oracle.segment_key_means(kf, cu).astype(np.float32)
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    log(f"[i8 centred] D={D} causal={causal} pv8={pv8} S={S}")

    def run(mu):
        q8, k8 = h3a().quantize_i8_rows(q), h3a().quantize_i8_keys(k, cu, mu=mu)
        if pv8:
            return to_f64(h3a().varlen_attn_fwd_i8qk_fp8pv(q8, k8, h3a().prepare_vt_e4m3(v, cu), cu, scale, causal))
        return to_f64(h3a().varlen_attn_fwd_i8qk(q8, k8, v, cu, scale, causal))

    o = run(torch.from_numpy(mu32).cuda())
    if pv8:
        bound, ref = weight_rounding_bound(oracle.i8_round_q(qf), oracle.i8_round_k_centered(kf, cu, mu32),
                                           oracle.mx_round_keys(vf, cu), cu, scale, causal)
        check_bound(o, ref, "o vs centred INT8 + E4M3 oracle", bound, TOL_FP8PV_MEANREL)
    else:
        compare(o, oracle.varlen_attention_i8qk_centered(qf, kf, vf, cu, scale, causal, mu32=mu32), "bf16",
                "o vs centred INT8 oracle")
    exact = oracle.varlen_attention_gqa(qf, kf, vf, cu, scale, causal)
    own = run(h3a().segment_key_means(k, cu))
    plain = run(None)
    err = lambda x: float(np.abs(x - exact).sum() / np.abs(exact).sum())  # noqa: E731
    log(f"  mean-rel vs exact: centred (GPU means) {err(own):.3e}, plain keys {err(plain):.3e}")
    # with FP8 PV the E4M3 V and weights add their own ~3e-2 (the chain tests) to both
    assert err(own) < 0.3 * err(plain) + (0.03 if pv8 else 0.0)


def test_centered_keys_many_segments():
    """150 ragged segments (three launches of both mean passes and of the quantiser)."""
    import torch

    lens = [int(x) for x in 1 + (rng.uniform(81, rng.TAG_LENS, 150) * 700).astype(np.int64)]
    lens[9] = 0
    cu, kb = _offset_keys(82, lens, 2, 64)
    kf = rng.as_f64(kb, "bf16")
    k = to_device(kb, "bf16")
    log(f"[centred many segments] S={int(cu[-1])} nseg={len(lens)} chunks={h3a().i8_key_mean_chunks(cu)}")
    mu = h3a().segment_key_means(k, cu).cpu().numpy().astype(np.float64)
    want = oracle.segment_key_means(kf, cu)
    assert np.all(np.abs(mu - want) <= _mean_bound(kf, cu, want))
    mu32 = want.astype(np.float32)
    c, s = h3a().quantize_i8_keys(k, cu, mu=torch.from_numpy(mu32).cuda())
    wc, ws = oracle.i8_quantize_key_blocks_centered(kf, cu, mu32)
    _codes_and_scales_equal(c, s, wc, ws, "centred k blocks, 150 segments")
