"""GPU parity on seeded random packings: many segments per launch whose lengths
mix empty, single-token, tile-boundary (63/64/65, 127/128/129) and arbitrary
ragged values, with random head layout (grouped K/V or not), head dim,
causality and dtype per case.  Every output row is compared with the fp64
oracle, so each case covers the planner's item list for that packing, partial
query and key tiles at every segment end, and segment isolation together."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import rng
from tests.gpu_util import compare, log, require_gpu, to_device, to_f64

BOUNDARY = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]
HEADS = [(1, 1), (3, 3), (2, 1), (4, 2), (6, 2)]
N_CASES = 16


@pytest.fixture(scope="module")
def _gpu():
    require_gpu()
    yield
    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()


def layout(case: int):
    """Case parameters from the SplitMix64 stream (tag TAG_LENS): 1..40 segments,
    each either a boundary length or uniform in [0, 700), at most ~6,000 tokens."""
    u = rng.uniform(1000 + case, rng.TAG_LENS, 128)
    nseg = 1 + int(u[0] * 40)
    lens = []
    for i in range(nseg):
        a, b = u[8 + 2 * i], u[9 + 2 * i]
        lens.append(BOUNDARY[int(b * len(BOUNDARY))] if a < 0.5 else int(b * 700))
    Hq, Hkv = HEADS[int(u[1] * len(HEADS))]
    D = 64 if u[2] < 0.5 else 128
    causal = bool(u[3] < 0.4)
    dtype = "f32" if u[4] < 0.25 else "bf16"
    return lens, Hq, Hkv, D, causal, dtype


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_CASES))
def test_random_packing(case, _gpu):
    import packed_varlen_attention_head_amd as h3a

    lens, Hq, Hkv, D, causal, dtype = layout(case)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S = int(cu[-1])
    seed = 2000 + case
    log(f"[random packing] case={case} nseg={len(lens)} S={S} Hq={Hq} Hkv={Hkv} D={D} "
        f"causal={causal} dtype={dtype}")
    if S == 0:
        pytest.skip("empty packing (covered by test_gpu_validation.py)")
    q = rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), dtype)
    k = rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), dtype)
    v = rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), dtype)
    scale = 1.0 / np.sqrt(D)
    o = to_f64(h3a.varlen_attn_fwd_ex(*(to_device(x, dtype) for x in (q, k, v)), cu, scale, causal=causal))
    ref = oracle.varlen_attention_gqa(*(rng.as_f64(x, dtype) for x in (q, k, v)), cu, scale, causal=causal)
    assert np.all(np.isfinite(o))
    compare(o, ref, dtype, "o")


def test_layouts_cover_the_edges():
    """The seeded cases together hit the shapes they are meant to (checked on the
    host, so a change of the generator cannot silently thin the coverage)."""
    cases = [layout(c) for c in range(N_CASES)]
    lens = [L for c in cases for L in c[0]]
    assert 0 in lens and 1 in lens
    assert any(L in (63, 65, 127, 129, 255, 257) for L in lens)
    assert any(L > 256 and L % 64 for L in lens)
    assert {c[3] for c in cases} == {64, 128}
    assert {c[4] for c in cases} == {False, True}
    assert {c[5] for c in cases} == {"bf16", "f32"}
    assert any(c[1] != c[2] for c in cases)
    assert max(len(c[0]) for c in cases) >= 20
    assert max(sum(c[0]) for c in cases) <= 30000


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_CASES))
def test_random_packing_fp8(case, _gpu):
    """The same packings through both low-precision kernels (bf16 inputs quantised to
    block-scaled E4M3 on the GPU): FP8 scores against attention on block-rounded q,
    k at the bf16 tolerance; both products in FP8, with V in the per-segment
    transposed layout, within the weight-rounding bound of attention on
    block-rounded q, k, v."""
    import packed_varlen_attention_head_amd as h3a
    from tests.test_gpu_fp8 import TOL_FP8PV_MEANREL, check, mx_operands, weight_rounding_bound

    lens, Hq, Hkv, D, causal, _ = layout(case)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S = int(cu[-1])
    seed = 3000 + case
    log(f"[random packing fp8] case={case} nseg={len(lens)} S={S} Hq={Hq} Hkv={Hkv} D={D} causal={causal}")
    q = rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), "bf16")
    k = rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), "bf16")
    v = rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), "bf16")
    scale = 1.0 / np.sqrt(D)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    q8, k8 = h3a.quantize_e4m3(qd), h3a.quantize_e4m3(kd)
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (q, k, v))
    o = to_f64(h3a.varlen_attn_fwd_fp8qk(q8, k8, vd, cu, scale, causal=causal))
    assert np.all(np.isfinite(o))
    compare(o, oracle.varlen_attention_mx_qk(qf, kf, vf, cu, scale, causal=causal), "bf16", "o, FP8 scores")
    o = to_f64(h3a.varlen_attn_fwd_fp8(q8, k8, h3a.prepare_vt_e4m3(vd, cu), cu, scale, causal=causal))
    assert np.all(np.isfinite(o))
    bound, ref = weight_rounding_bound(*mx_operands(q, k, v, cu), cu, scale, causal)
    check(o, ref, "o, both products FP8", bound, TOL_FP8PV_MEANREL)


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_CASES))
def test_random_packing_int8(case, _gpu):
    """The same packings through the INT8 score kernels (q and k quantised on the GPU,
    per token and per 64-key block of each segment): bf16 PV against attention on what
    the codes stand for at the bf16 tolerance; FP8 PV (transposed E4M3 V) within the
    weight-rounding bound of attention on those q, k and block-rounded v."""
    import packed_varlen_attention_head_amd as h3a
    from tests.test_gpu_fp8 import TOL_FP8PV_MEANREL, check, weight_rounding_bound

    lens, Hq, Hkv, D, causal, _ = layout(case)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S = int(cu[-1])
    seed = 4000 + case
    log(f"[random packing int8] case={case} nseg={len(lens)} S={S} Hq={Hq} Hkv={Hkv} D={D} causal={causal}")
    if S == 0:
        pytest.skip("empty packing (covered by test_gpu_validation.py)")
    q = rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), "bf16")
    k = rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), "bf16")
    v = rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), "bf16")
    scale = 1.0 / np.sqrt(D)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    q8, k8 = h3a.quantize_i8_rows(qd), h3a.quantize_i8_keys(kd, cu)
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (q, k, v))
    o = to_f64(h3a.varlen_attn_fwd_i8qk(q8, k8, vd, cu, scale, causal=causal))
    assert np.all(np.isfinite(o))
    compare(o, oracle.varlen_attention_i8qk(qf, kf, vf, cu, scale, causal=causal), "bf16", "o, INT8 scores")
    o = to_f64(h3a.varlen_attn_fwd_i8qk_fp8pv(q8, k8, h3a.prepare_vt_e4m3(vd, cu), cu, scale, causal=causal))
    assert np.all(np.isfinite(o))
    bound, ref = weight_rounding_bound(oracle.i8_round_q(qf), oracle.i8_round_k(kf, cu), oracle.mx_round_keys(vf, cu),
                                       cu, scale, causal)
    check(o, ref, "o, INT8 scores and FP8 PV", bound, TOL_FP8PV_MEANREL)
