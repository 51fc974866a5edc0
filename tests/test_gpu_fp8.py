"""GPU parity of the low-precision path with per-block scales: the E4M3 codes
and E8M0 block scales of the quantisers bit for bit against the oracle's
block-scaled codec, FP8-score attention against the oracle's attention on
block-rounded q and k (the bf16 path's tolerance), attention with both
products in FP8 within a derived bound of rounding the softmax weights, inputs
far outside E4M3's range (1e-3, > 448), and the whole chain against exact
attention."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import configs, rng
from tests.gpu_util import TOL_BF16_ABS, compare, log, require_gpu, sample_rows, to_device, to_f64

pytestmark = pytest.mark.gpu

# FP8 scores against exact attention on the norm + rotary chain's N(0,1)-like
# operands: three mantissa bits per q, k element, whatever the block scale, put
# the oracle at 3.9e-2 mean-rel and 1.9e-2 max abs (two_seg, sampled rows).
TOL_FP8_ABS = 5e-2
TOL_FP8_MEANREL = 5e-2

# Both products in FP8: the oracle's block-rounded q, k, v with exact weights
# are 4.7e-2 mean-rel from exact attention; the kernel's E4M3 weights add about
# 2.5e-2 (in quadrature): 5.3e-2 mean-rel, 2.2e-2 max abs on two_seg.
TOL_FP8_EXACT_ABS, TOL_FP8_EXACT_MEANREL = 6e-2, 6.5e-2
# The weights' own rounding, against the oracle on the same block-rounded operands.
TOL_FP8PV_MEANREL = 3.5e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()


def h3a():
    import packed_varlen_attention_head_amd as m

    return m


# ---------------------------------------------------------------------------
# expected codes and scales from the oracle's codec


def mx_codes(bits: np.ndarray):
    """(E4M3 codes [S, H, D], E8M0 scale codes head-major [H, S, D / 32]) of bf16
    bits [S, H, D] in blocks of 32 along D."""
    codes, X = oracle.mx_quantize(rng.bf16_bits_to_f32(bits).astype(np.float64), axis=-1)
    return codes, np.ascontiguousarray((X + 127).astype(np.uint8).transpose(1, 0, 2))


def expected_vt(vbits: np.ndarray, cu):
    """The transposed, segment-padded E4M3 layout of v and its scales: codes
    [H, D, cols], scales [H, cols / 64, 2, 32, D / 32] where entry (h, t, j, r, b)
    belongs to dim 32 b + r and keys 32 j .. 32 j + 31 of column tile t."""
    S, H, D = vbits.shape
    vf = rng.bf16_bits_to_f32(vbits).astype(np.float64)
    lens = np.diff(np.asarray(cu))
    pad = (lens + 63) // 64 * 64
    cols = int(pad.sum())
    codes = np.zeros((H, D, max(cols, 1)), dtype=np.uint8)
    scales = np.zeros((H, max(cols, 64) // 64, 2, 32, D // 32), dtype=np.uint8)
    col = 0
    for s, L in enumerate(lens):
        if L == 0:
            continue
        a, n = int(cu[s]), int(pad[s])
        block = np.zeros((n, H, D))
        block[:L] = vf[a:a + L]
        c, X = oracle.mx_quantize(block, axis=0)  # c [n, H, D], X [n / 32, H, D]
        codes[:, :, col:col + n] = c.transpose(1, 2, 0)
        e = (X + 127).astype(np.uint8).reshape(n // 64, 2, H, D // 32, 32)  # (tile, j, h, b, r)
        scales[:, col // 64:col // 64 + n // 64] = e.transpose(2, 0, 1, 4, 3)
        col += n
    return codes, scales


# ---------------------------------------------------------------------------
# the bound of rounding the softmax weights


def weight_rounding_bound(q, k, v, cu, scale, causal=False, rows=None):
    """Elementwise bound [rows, Hq, D] on |o - o_ref| where o_ref is attention on
    the given (already block-rounded) operands and o the same with every weight
    rounded to E4M3 before the PV product, the row sum taken over the rounded
    weights.

    The kernel holds the weights as p_j = 2^(4 + c s_j - m) against a running
    reference m that never exceeds the row's true max and trails it by at most 4
    (c s in log2 units), so the largest weight is in [16, 256] and the row sum
    L >= 16.  E4M3 rounding moves a normal weight (>= 2^-6) by at most 2^-4 of
    itself and a subnormal one by at most min(p_j, 2^-10).  With exact weights
    w_j = p_j / L this is e_j = max(2^-4 w_j, min(w_j, 2^-14)) relative to L.
    Writing d_j for the rounding, o - o_ref = sum_j d_j (v_j - o_ref) / L~ with
    L~ = L + sum_j d_j >= L (1 - sum_j e_j), hence
    |o - o_ref| <= (sum_j e_j |v_j| + (sum_j e_j) |o_ref|) / (1 - sum_j e_j).
    Added: the bf16 output rounding (2^-8 |o_ref|) and 1e-5 max|v| for fp32
    accumulation.  Returns (bound, o_ref)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    S, Hq, D = q.shape
    grp = Hq // k.shape[1]
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    seg = oracle.segment_of_rows(cu, rows)
    bound = np.empty((len(rows), Hq, v.shape[2]))
    ref = np.empty_like(bound)
    for s in np.unique(seg):
        a, b = int(cu[s]), int(cu[s + 1])
        for c0 in range(0, int(np.sum(seg == s)), 256):  # row blocks bound the memory
            sel = np.nonzero(seg == s)[0][c0:c0 + 256]
            r = rows[sel]
            for h in range(Hq):
                sc = scale * (q[r, h] @ k[a:b, h // grp].T)
                if causal:
                    sc = np.where(np.arange(a, b)[None, :] <= r[:, None], sc, -np.inf)
                w = np.exp(sc - sc.max(axis=1, keepdims=True))
                w /= w.sum(axis=1, keepdims=True)
                vs = v[a:b, h // grp]
                o = w @ vs
                e = np.maximum(2.0 ** -4 * w, np.minimum(w, 2.0 ** -14))
                E = e.sum(axis=1, keepdims=True)
                bound[sel, h] = (e @ np.abs(vs) + E * np.abs(o)) / (1.0 - E) + 2.0 ** -8 * np.abs(o) \
                    + 1e-5 * np.abs(vs).max()
                ref[sel, h] = o
    return bound, ref


def check(g, r, what, tol_abs, tol_rel):
    """tol_abs: a number, or an elementwise bound of the same shape as r."""
    err = np.abs(g - r)
    max_abs, mean_rel = float(err.max()), float(err.sum() / np.abs(r).sum())
    worst = float(np.max(err - tol_abs))
    log(f"  {what}: max_abs={max_abs:.3e} mean_rel={mean_rel:.3e} max(err - bound)={worst:.3e} n={err.size}")
    assert np.all(np.isfinite(g))
    assert worst <= 0 and mean_rel <= tol_rel, (max_abs, mean_rel, worst)


def gpu_fp8qk(qb, kb, vb, cu, scale, causal=False):
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    return h3a().varlen_attn_fwd_fp8qk(h3a().quantize_e4m3(q), h3a().quantize_e4m3(k), v, cu, scale, causal=causal)


def gpu_fp8(qb, kb, vb, cu, scale, causal=False):
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    return h3a().varlen_attn_fwd_fp8(h3a().quantize_e4m3(q), h3a().quantize_e4m3(k), h3a().prepare_vt_e4m3(v, cu),
                                     cu, scale, causal=causal)


def mx_operands(qb, kb, vb, cu):
    """The oracle's block-rounded q, k (32 dims) and v (32 keys of each segment)."""
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    return oracle.mx_round(qf), oracle.mx_round(kf), oracle.mx_round_keys(vf, cu)


# ---------------------------------------------------------------------------
# the quantisers


def bf16_specials_blocks() -> np.ndarray:
    """bf16 bit patterns in blocks of 32 that exercise the codec and the block
    exponent: every finite E4M3 value, the midpoints between neighbours and one
    bf16 step either side of them, in blocks whose first element is +-448 (scale
    2^0, the codes themselves) and again times 2^-20 (scale 2^-20); blocks whose
    largest magnitude sits at the exponent's boundaries 448 * 2^k (scale 2^k) and
    one bf16 step above (2^(k+1)); values past 448 up to 3e38; all-zero, signed
    zero and bf16-subnormal blocks."""
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = 0.5 * (pos[1:] + pos[:-1])
    f = lambda x: rng.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    mid_bits = f(np.concatenate([mids, -mids]))
    body = np.concatenate([f(np.concatenate([pos, -pos, mids, -mids])), mid_bits + 1, mid_bits - 1]).astype(np.uint16)
    body = np.concatenate([body, np.zeros(-len(body) % 31, dtype=np.uint16)]).reshape(-1, 31)
    anchor = np.where(np.arange(len(body)) % 2 == 0, f(448.0), f(-448.0)).astype(np.uint16)[:, None]
    direct = np.concatenate([anchor, body], axis=1)
    # the same blocks times 2^-20: bf16 keeps every value (8 significant bits)
    small = f(rng.bf16_bits_to_f32(direct) * np.float32(2.0 ** -20))
    blocks = [direct, small]
    base = rng.normal_tensor(7, rng.TAG_Q, (64, 32), "bf16")
    for i, k in enumerate(range(-40, 40, 5)):
        for bump in (0, 1):  # amax exactly 448 * 2^k, then the next bf16 value up
            b = f(rng.bf16_bits_to_f32(base[(2 * i + bump) % 64]) * np.float32(2.0 ** k))
            b[5] = f(448.0 * 2.0 ** k) + bump
            blocks.append(b[None])
    big = f(np.array([449.0, 464.0, 480.0, 1e4, 6e4, 1e9, 3e38, -3e38] * 4))
    blocks.append(big[None])
    blocks.append(np.zeros((1, 32), dtype=np.uint16))
    blocks.append(np.full((1, 32), 0x8000, dtype=np.uint16))
    blocks.append(np.arange(1, 33, dtype=np.uint16)[None])  # bf16 subnormals 2^-133 ...
    blocks.append((np.arange(1, 33, dtype=np.uint16) | 0x8000)[None])
    return np.concatenate(blocks, axis=0).astype(np.uint16).reshape(-1)


def test_quantize_codes_and_scales_bit_exact():
    import torch

    special = bf16_specials_blocks()
    magnitudes = [1e-6, 1e-3, 0.05, 1.0, 7.0, 60.0, 300.0, 1e3, 1e5]
    rand = np.concatenate([rng.normal_tensor(11, rng.TAG_Q, (4096,), "bf16", 0.0, s) for s in magnitudes])
    bits = np.concatenate([special, rand])
    D = 128
    S = -(-len(bits) // D)
    bits = np.concatenate([bits, np.zeros(S * D - len(bits), dtype=np.uint16)]).reshape(S, 1, D)
    x = to_device(bits, "bf16")
    # padded output rows: 128 code bytes + 128 guard bytes
    ybuf = torch.full((S, 2 * D), 0xA5, dtype=torch.uint8, device="cuda")
    y = ybuf[:, :D].view(S, 1, D)
    y8, ys = h3a().quantize_e4m3(x, out=y)
    torch.cuda.synchronize()
    want, want_s = mx_codes(bits)
    got, got_s = y8.cpu().numpy(), ys.cpu().numpy()
    bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
    bad_s = np.nonzero(got_s.reshape(-1) != want_s.reshape(-1))[0]
    log(f"[quantize] {got.size} codes, {len(bad)} mismatches; {got_s.size} scales, {len(bad_s)} mismatches; "
        f"scale codes {int(want_s.min())}..{int(want_s.max())}")
    assert len(bad_s) == 0, (bad_s[:8], got_s.reshape(-1)[bad_s[:8]], want_s.reshape(-1)[bad_s[:8]])
    assert len(bad) == 0, (bad[:8], got.reshape(-1)[bad[:8]], want.reshape(-1)[bad[:8]])
    assert torch.all(ybuf[:, D:] == 0xA5)
    # the scale range the inputs reach: bf16 subnormals (-127) up to 3e38 (120)
    assert int(want_s.min()) == 0 and int(want_s.max()) == 247


@pytest.mark.parametrize("name,kv", [("h3_s20423_bf16", 24), ("two_seg_bf16", 8)])
def test_fused_norm_rope_e4m3_equals_two_passes(name, kv):
    """The norm + rotary pass that writes E4M3 codes and scales gives the same bytes
    as the bf16 pass followed by the quantiser, and leaves q, k untouched."""
    import torch

    w = configs.ALL[name].replace(kv_heads=kv)
    T = configs.make_tensors(w)
    log(f"[fused e4m3] {name} Hq={w.heads} Hk={w.kv}")
    q, k = to_device(T.q, "bf16"), to_device(T.k, "bf16")
    q0, k0 = q.clone(), k.clone()
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    h3a().build_rope_table(w.segments, w.rot_dims, w.base, tab)
    (q8, qs), (k8, ks) = h3a().qk_rmsnorm_rope_e4m3(q, k, gq, gk, w.eps, tab, w.rot_dim)
    qn, kn = torch.empty_like(q), torch.empty_like(k)
    h3a().qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim, q_out=qn, k_out=kn)
    (q8b, qsb), (k8b, ksb) = h3a().quantize_e4m3(qn), h3a().quantize_e4m3(kn)
    torch.cuda.synchronize()
    assert torch.equal(q, q0) and torch.equal(k, k0)
    assert torch.equal(q8, q8b) and torch.equal(k8, k8b)
    assert torch.equal(qs, qsb) and torch.equal(ks, ksb)


def magnitude_segments(vbits: np.ndarray, cu, mags) -> np.ndarray:
    """v scaled per segment by mags[s % len(mags)] (bf16 bits)."""
    vf = rng.bf16_bits_to_f32(vbits)
    for s in range(len(cu) - 1):
        vf[int(cu[s]):int(cu[s + 1])] *= np.float32(mags[s % len(mags)])
    return rng.f32_to_bf16_bits(vf)


@pytest.mark.parametrize("D", [64, 128])
def test_prepare_vt_layout_bit_exact(D):
    """Codes and scales of the transposed V layout, segments at magnitudes from
    1e-3 to 1e3 (past 448: no element saturates under its block's scale)."""
    import torch

    lens = [1, 63, 64, 65, 0, 129, 700, 33, 31]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S, H = int(cu[-1]), 3
    vb = magnitude_segments(rng.normal_tensor(41 + D, rng.TAG_V, (S, H, D), "bf16"), cu, [1e-3, 1.0, 1e3, 30.0])
    vt, vs = h3a().prepare_vt_e4m3(to_device(vb, "bf16"), cu)
    torch.cuda.synchronize()
    want, want_s = expected_vt(vb, cu)
    got, got_s = vt.cpu().numpy(), vs.cpu().numpy()
    log(f"[vt layout] D={D} columns={want.shape[2]} code mismatches={int(np.sum(got != want))} "
        f"scale mismatches={int(np.sum(got_s != want_s))}")
    assert got.shape == want.shape and np.array_equal(got, want)
    assert got_s.shape == want_s.shape and np.array_equal(got_s, want_s)


# ---------------------------------------------------------------------------
# FP8 scores, bf16 weights and V


EDGE_LENS = [1, 63, 64, 65, 127, 128, 129, 0, 255, 256, 257, 700]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8qk_vs_mx_oracle(D, Hq, Hkv, causal):
    """Seeded bf16 q, k, v: the GPU quantises and attends; the oracle attends on the
    same q, k rounded per 32-dim block (its own codec), exactly."""
    cu = np.concatenate([[0], np.cumsum(EDGE_LENS)]).astype(np.int64)
    S = int(cu[-1])
    seed = 300 + D + Hq + (1 if causal else 0)
    log(f"[fp8qk] D={D} Hq={Hq} Hkv={Hkv} causal={causal} S={S} seed={seed}")
    qb = rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), "bf16")
    kb = rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), "bf16")
    vb = rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), "bf16")
    scale = 1.0 / np.sqrt(D)
    o = to_f64(gpu_fp8qk(qb, kb, vb, cu, scale, causal))
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    compare(o, oracle.varlen_attention_mx_qk(qf, kf, vf, cu, scale, causal=causal), "bf16", "o vs block-scaled oracle")


@pytest.mark.parametrize("name", ["two_seg_bf16", "h3_s20423_bf16"])
def test_fp8qk_chain(name):
    """table -> norm + rotary -> block-scaled E4M3 q', k' -> FP8-score attention,
    against the oracle's attention on its own q', k' stored in bf16 and rounded per
    block (the code decision in the kernel's precision; bf16 tolerance) and against
    exact attention (the looser FP8 tolerance)."""
    import torch

    w = configs.ALL[name]
    T = configs.make_tensors(w)
    log(f"[fp8 chain] {name} S={w.tokens}")
    q, k, v = (to_device(x, w.dtype) for x in (T.q, T.k, T.v))
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    cu = h3a().build_rope_table(w.segments, w.rot_dims, w.base, tab)
    q8, k8 = h3a().qk_rmsnorm_rope_e4m3(q, k, gq, gk, w.eps, tab, w.rot_dim)
    o = to_f64(h3a().varlen_attn_fwd_fp8qk(q8, k8, v, cu, w.scale))
    qf, kf, vf = (rng.as_f64(x, w.dtype) for x in (T.q, T.k, T.v))
    ocu, cos, sin = oracle.rope_table(w.segments, w.rot_dims, w.base)
    qn, kn = oracle.qk_rmsnorm_rope(qf, kf, T.gamma_q, T.gamma_k, w.eps, cos, sin, w.rot_dim)
    rows = sample_rows(ocu, every=97)
    q8o, k8o = (oracle.mx_round(oracle.bf16_round(x)) for x in (qn, kn))
    ref_q = oracle.varlen_attention_rows(q8o, k8o, vf, ocu, w.scale, rows)
    compare(o[rows], ref_q, "bf16", f"o vs block-scaled oracle ({len(rows)} rows)")
    ref = oracle.varlen_attention_rows(qn, kn, vf, ocu, w.scale, rows)
    check(o[rows], ref, "o vs exact attention", TOL_FP8_ABS, TOL_FP8_MEANREL)


def test_fp8qk_segment_isolation_and_determinism():
    import torch

    lens = [900, 500]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S, H, D = 1400, 4, 128
    qb = rng.normal_tensor(5, rng.TAG_Q, (S, H, D), "bf16")
    kb = rng.normal_tensor(5, rng.TAG_K, (S, H, D), "bf16")
    vb = rng.normal_tensor(5, rng.TAG_V, (S, H, D), "bf16")
    for fn in (gpu_fp8qk, gpu_fp8):
        a = fn(qb, kb, vb, cu, 0.088)
        b = fn(qb, kb, vb, cu, 0.088)
        kb2 = kb.copy()
        kb2[1000] ^= 0x0040
        c = fn(qb, kb2, vb, cu, 0.088)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        assert torch.equal(a[:900], c[:900]) and not torch.equal(a[900:], c[900:])


# ---------------------------------------------------------------------------
# both products in FP8


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_vs_mx_oracle(D, Hq, Hkv, causal):
    cu = np.concatenate([[0], np.cumsum(EDGE_LENS)]).astype(np.int64)
    S = int(cu[-1])
    seed = 500 + D + Hq + (1 if causal else 0)
    log(f"[fp8 pv] D={D} Hq={Hq} Hkv={Hkv} causal={causal} S={S} seed={seed}")
    qb = rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), "bf16")
    kb = rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), "bf16")
    vb = rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), "bf16")
    o = to_f64(gpu_fp8(qb, kb, vb, cu, 1.0 / np.sqrt(D), causal))
    bound, ref = weight_rounding_bound(*mx_operands(qb, kb, vb, cu), cu, 1.0 / np.sqrt(D), causal)
    check(o, ref, "o vs block-scaled oracle", bound, TOL_FP8PV_MEANREL)


@pytest.mark.parametrize("mode", ["fp8qk", "fp8"])
@pytest.mark.parametrize("vmag", [1e-3, 1e3])
def test_magnitudes_far_from_one(mode, vmag):
    """v at 1e-3 (below E4M3's normal range unscaled) and at 1e3 (past 448), q at
    1e-3 and k at 1e3 (their product N(0,1)): the block scales keep every element's
    relative precision, so the outputs divided by vmag meet the same bounds as at
    magnitude one."""
    cu = np.concatenate([[0], np.cumsum([300, 129, 64, 1, 700])]).astype(np.int64)
    S, Hq, Hkv, D = int(cu[-1]), 4, 2, 128
    seed = 700 + (1 if mode == "fp8" else 0) + (2 if vmag > 1 else 0)
    log(f"[magnitudes] {mode} v*{vmag:g} q*1e-3 k*1e3 S={S}")

    def scaled(tag, shape, m):
        return rng.f32_to_bf16_bits(rng.bf16_bits_to_f32(rng.normal_tensor(seed, tag, shape, "bf16")) * np.float32(m))

    qb, kb, vb = scaled(rng.TAG_Q, (S, Hq, D), 1e-3), scaled(rng.TAG_K, (S, Hkv, D), 1e3), scaled(rng.TAG_V, (S, Hkv, D),
                                                                                                 vmag)
    scale = 1.0 / np.sqrt(D)
    if mode == "fp8qk":
        o = to_f64(gpu_fp8qk(qb, kb, vb, cu, scale))
        qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
        ref = oracle.varlen_attention_mx_qk(qf, kf, vf, cu, scale)
        compare(o / vmag, ref / vmag, "bf16", "o / vmag vs block-scaled oracle")
        return
    o = to_f64(gpu_fp8(qb, kb, vb, cu, scale))
    bound, ref = weight_rounding_bound(*mx_operands(qb, kb, vb, cu), cu, scale)
    check(o / vmag, ref / vmag, "o / vmag vs block-scaled oracle", bound / vmag, TOL_FP8PV_MEANREL)


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
    q8o, k8o = (oracle.mx_round(oracle.bf16_round(x)) for x in (qn, kn))
    bound, ref8 = weight_rounding_bound(q8o, k8o, oracle.mx_round_keys(vf, ocu), ocu, w.scale, rows=rows)
    check(o[rows], ref8, f"o vs block-scaled oracle ({len(rows)} rows)", bound, TOL_FP8PV_MEANREL)
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
    want, want_s = expected_vt(vb, cu)
    assert np.array_equal(vt[0].cpu().numpy(), want) and np.array_equal(vt[1].cpu().numpy(), want_s)
    o = h3a().varlen_attn_fwd_fp8(h3a().quantize_e4m3(q), h3a().quantize_e4m3(k), vt, cu, 0.125)
    bound, ref = weight_rounding_bound(*mx_operands(qb, kb, vb, cu), cu, 0.125)
    check(to_f64(o), ref, "o vs block-scaled oracle", bound, TOL_FP8PV_MEANREL)
