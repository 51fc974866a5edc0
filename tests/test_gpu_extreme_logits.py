"""GPU parity with logits that rise along the keys (a per-key gain on k) and one
64-key tile far above the rest: every variant's running-max machinery (the lazy
reference, its rescale, the tile recompute of the bf16 steady loop, the
lane-pair row max) is exercised many times per row, including a jump of ~2^130
that overflows any probability taken against a stale reference.  Each variant
is compared with the oracle at its own tolerance, and the fused Q path with the
unfused one bit for bit."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import rng
from tests.gpu_util import compare, log, require_gpu, to_device, to_f64

pytestmark = pytest.mark.gpu

LENS = [700, 300, 129, 65]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()


def h3a():
    import packed_varlen_attention_head_amd as m

    return m


def rising_inputs(seed, Hq, Hkv, D, dtype="bf16"):
    """q, v ~ N(0,1); k ~ N(0,1) times a gain that ramps 1 -> 15 along the first
    segment's keys and is 40 on keys 192..255 of the second."""
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int64)
    S = int(cu[-1])
    q = rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), dtype)
    k0 = rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), dtype)
    v = rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), dtype)
    gain = np.ones(S)
    gain[: LENS[0]] = 1.0 + np.arange(LENS[0]) / 50.0
    gain[LENS[0] + 192: LENS[0] + 256] = 40.0
    kf = (rng.as_f64(k0, dtype) * gain[:, None, None]).astype(np.float32)
    k = rng.f32_to_bf16_bits(kf) if dtype == "bf16" else kf
    return cu, q, k, v


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2)])
def test_rising_logits_bf16_f32(dtype, causal, Hq, Hkv):
    D = 128
    cu, q, k, v = rising_inputs(21 + Hq + (2 if causal else 0), Hq, Hkv, D, dtype)
    log(f"[rising] dtype={dtype} causal={causal} Hq={Hq} Hkv={Hkv}")
    scale = 1.0 / np.sqrt(D)
    o = to_f64(h3a().varlen_attn_fwd_ex(*(to_device(x, dtype) for x in (q, k, v)), cu, scale, causal=causal))
    qf, kf, vf = (rng.as_f64(x, dtype) for x in (q, k, v))
    ref = oracle.varlen_attention_gqa(qf, kf, vf, cu, scale, causal=causal)
    if dtype == "bf16":
        compare(o, ref, dtype, "o")
        return
    # fp32: the raw scores reach ~1,600 here (key gain 40), so one fp32 rounding of a
    # score alone moves it by ~1e-4 and the 1e-5 bound of N(0,1) logits does not apply
    # to every row.  Per row i the bound grows with that row's own largest absolute dot
    # product A_i = max_j sum_d |q_id k_jd| over the keys it sees: four fp32 ulps of A_i
    # per logit (the sum's final rounding plus the accumulation), and a logit error d
    # moves an output by at most 2 d max|v|.  Rows whose keys are N(0,1) keep ~1e-5; an
    # overflow or rescale mistake moves outputs by O(1e-3 - 1) and fails.
    bound = 1e-5 + 4.0 * 2.0 ** -24 * scale * 2.0 * row_abs_dot_max(qf, kf, cu, causal)[:, :, None] \
        * np.abs(vf).max()
    err = np.abs(o - ref)
    mean_rel = float(err.sum() / np.abs(ref).sum())
    log(f"  o: max_abs={err.max():.3e} mean_rel={mean_rel:.3e} bound range=[{bound.min():.2e}, {bound.max():.2e}] "
        f"max err/bound={float((err / bound).max()):.3f}")
    assert np.all(np.isfinite(o))
    assert np.all(err <= bound) and mean_rel <= 1e-5


def row_abs_dot_max(qf, kf, cu, causal):
    """[S, Hq]: for each query row and head, max over the keys it sees of
    sum_d |q_d k_d| (K/V head h // (Hq/Hkv))."""
    S, Hq, _ = qf.shape
    grp = Hq // kf.shape[1]
    out = np.zeros((S, Hq))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for h in range(Hq):
            m = np.abs(qf[a:b, h]) @ np.abs(kf[a:b, h // grp]).T
            if causal:
                m = np.where(np.tril(np.ones((b - a, b - a), dtype=bool)), m, 0.0)
            out[a:b, h] = m.max(axis=1)
    return out


def test_rising_logits_fp8_scores():
    """FP8 score product, bf16 probabilities: against attention on block-rounded q, k."""
    D, H = 128, 2
    cu, q, k, v = rising_inputs(31, H, H, D)
    log("[rising] fp8 scores")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o = to_f64(h3a().varlen_attn_fwd_fp8qk(h3a().quantize_e4m3(qd), h3a().quantize_e4m3(kd), vd, cu, 1.0 / np.sqrt(D)))
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (q, k, v))
    compare(o, oracle.varlen_attention_mx_qk(qf, kf, vf, cu, 1.0 / np.sqrt(D)), "bf16", "o vs block-scaled oracle")


def test_rising_logits_fp8_both():
    """Both products in FP8: within the bound of rounding the weights to E4M3, against
    attention on block-rounded q, k, v.  The rising keys make the running reference
    climb many times per row, so every rescale of the FP8 accumulators is crossed."""
    from tests.test_gpu_fp8 import TOL_FP8PV_MEANREL, check, mx_operands, weight_rounding_bound

    D, H = 128, 2
    cu, q, k, v = rising_inputs(41, H, H, D)
    log("[rising] fp8 scores and output")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o = to_f64(h3a().varlen_attn_fwd_fp8(h3a().quantize_e4m3(qd), h3a().quantize_e4m3(kd),
                                         h3a().prepare_vt_e4m3(vd, cu), cu, 1.0 / np.sqrt(D)))
    bound, ref = weight_rounding_bound(*mx_operands(q, k, v, cu), cu, 1.0 / np.sqrt(D))
    check(o, ref, "o vs block-scaled oracle", bound, TOL_FP8PV_MEANREL)


@pytest.mark.parametrize("causal", [False, True])
def test_rising_logits_int8_scores(causal):
    """INT8 score product (per-tile score multiplier in the probabilities' FMA), bf16
    probabilities: against attention on what the codes stand for.  The gain-40 tile sets
    its own key-block scale, so its scores jump as in the bf16 case."""
    D, Hq, Hkv = 128, 4, 2
    cu, q, k, v = rising_inputs(61 + causal, Hq, Hkv, D)
    log(f"[rising] int8 scores causal={causal}")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o = to_f64(h3a().varlen_attn_fwd_i8qk(h3a().quantize_i8_rows(qd), h3a().quantize_i8_keys(kd, cu), vd, cu,
                                          1.0 / np.sqrt(D), causal=causal))
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (q, k, v))
    compare(o, oracle.varlen_attention_i8qk(qf, kf, vf, cu, 1.0 / np.sqrt(D), causal), "bf16", "o vs INT8 oracle")


def test_rising_logits_int8_scores_fp8_output():
    """INT8 scores with FP8 PV: within the weight-rounding bound of attention on the INT8
    q, k and block-rounded v."""
    from tests.test_gpu_fp8 import TOL_FP8PV_MEANREL, check, weight_rounding_bound

    D, H = 128, 2
    cu, q, k, v = rising_inputs(71, H, H, D)
    log("[rising] int8 scores, fp8 output")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o = to_f64(h3a().varlen_attn_fwd_i8qk_fp8pv(h3a().quantize_i8_rows(qd), h3a().quantize_i8_keys(kd, cu),
                                                h3a().prepare_vt_e4m3(vd, cu), cu, 1.0 / np.sqrt(D)))
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (q, k, v))
    bound, ref = weight_rounding_bound(oracle.i8_round_q(qf), oracle.i8_round_k(kf, cu), oracle.mx_round_keys(vf, cu),
                                       cu, 1.0 / np.sqrt(D))
    check(o, ref, "o vs INT8 + E4M3 oracle", bound, TOL_FP8PV_MEANREL)


def test_rising_logits_fused_q_bitwise():
    """Q norm + rotary inside the attention prologue gives the same bytes as the norm
    pass followed by the attention, on rising keys."""
    import torch

    D, H, R = 128, 2, 96
    cu, q, k, v = rising_inputs(51, H, H, D)
    S = int(cu[-1])
    log("[rising] fused q")
    segs = [(1, 1, L, L) for L in LENS]
    tab = torch.empty((2, S, R // 2), dtype=torch.float32, device="cuda")
    h3a().build_rope_table(segs, (32, 32, 32), 10000.0, tab)
    gq = torch.from_numpy((1.0 + 0.1 * rng.normal(51, rng.TAG_GAMMA_Q, D)).astype(np.float32)).cuda()
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    qn = h3a().rmsnorm_rope(qd, gq, 1e-6, tab, R, x_out=torch.empty_like(qd))
    o_ref = h3a().varlen_attn_fwd(qn, kd, vd, cu, 1.0 / np.sqrt(D))
    o_fused = h3a().varlen_attn_fwd_qnorm(qd, kd, vd, cu, 1.0 / np.sqrt(D), gq, 1e-6, tab, R)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(o_fused.float()))
    assert torch.equal(o_ref, o_fused)
