"""Maximum-size case: one packing of 2^18 = 262,144 tokens, a 261,147-token
segment (4,081 key tiles, partial last query and key tiles) followed by a
997-token one.  Offsets, strides and plan sizes well past the benchmark
workloads must stay exact; outputs are checked on sampled rows against the
oracle, which computes each row on its own."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import rng
from tests.gpu_util import compare, log, require_gpu, to_device, to_f64

pytestmark = pytest.mark.gpu

LENS = [261147, 997]
D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()


def rows_to_check(cu):
    """Every 4,099th row, each segment's first two and last eight rows, and rows
    on both sides of the 2^15, 2^16 and 2^17 boundaries."""
    rows = set(range(0, int(cu[-1]), 4099))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        rows.update((a, a + 1))
        rows.update(range(b - 8, b))
    for p in (15, 16, 17):
        rows.update((2 ** p - 1, 2 ** p))
    return np.array(sorted(rows), dtype=np.int64)


def inputs(seed, Hq, Hkv):
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int64)
    S = int(cu[-1])
    assert S == 2 ** 18
    q = rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), "bf16")
    k = rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), "bf16")
    v = rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), "bf16")
    return cu, q, k, v


def test_long_bidirectional_bf16():
    import packed_varlen_attention_head_amd as h3a

    cu, q, k, v = inputs(61, 1, 1)
    rows = rows_to_check(cu)
    log(f"[long] bf16 bidirectional S={int(cu[-1])} rows={len(rows)}")
    o = h3a.varlen_attn_fwd(*(to_device(x, "bf16") for x in (q, k, v)), cu, 1.0 / np.sqrt(D))
    o = to_f64(o[rows.tolist()])
    assert np.all(np.isfinite(o))
    ref = oracle.varlen_attention_rows(*(rng.as_f64(x, "bf16") for x in (q, k, v)), cu, 1.0 / np.sqrt(D), rows)
    compare(o, ref, "bf16", f"o ({len(rows)} rows)")


def test_long_causal_grouped_bf16():
    import packed_varlen_attention_head_amd as h3a

    cu, q, k, v = inputs(62, 2, 1)
    rows = rows_to_check(cu)
    log(f"[long] bf16 causal Hq=2 Hkv=1 S={int(cu[-1])} rows={len(rows)}")
    o = h3a.varlen_attn_fwd_ex(*(to_device(x, "bf16") for x in (q, k, v)), cu, 1.0 / np.sqrt(D), causal=True)
    o = to_f64(o[rows.tolist()])
    assert np.all(np.isfinite(o))
    ref = oracle.varlen_attention_gqa_rows(*(rng.as_f64(x, "bf16") for x in (q, k, v)), cu, 1.0 / np.sqrt(D), rows,
                                           causal=True)
    compare(o, ref, "bf16", f"o ({len(rows)} rows)")


def test_long_fp8_both():
    """Both products in FP8 (V as 262,208 transposed E4M3 columns per dim row, with
    their block scales): within the weight-rounding bound of attention on
    block-rounded q, k, v."""
    import packed_varlen_attention_head_amd as h3a
    from tests.test_gpu_fp8 import TOL_FP8PV_MEANREL, check, weight_rounding_bound

    cu, q, k, v = inputs(63, 1, 1)
    rows = rows_to_check(cu)
    assert h3a.vt_e4m3_columns(cu) == 261184 + 1024
    log(f"[long] fp8 both S={int(cu[-1])} rows={len(rows)}")
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o = h3a.varlen_attn_fwd_fp8(h3a.quantize_e4m3(qd), h3a.quantize_e4m3(kd), h3a.prepare_vt_e4m3(vd, cu), cu,
                                1.0 / np.sqrt(D))
    o = to_f64(o[rows.tolist()])
    # only the sampled query rows are read by the bound's attention
    qf = rng.as_f64(q, "bf16")
    q8 = np.zeros_like(qf)
    q8[rows] = oracle.mx_round(qf[rows])
    k8, v8 = oracle.mx_round(rng.as_f64(k, "bf16")), oracle.mx_round_keys(rng.as_f64(v, "bf16"), cu)
    bound, ref = weight_rounding_bound(q8, k8, v8, cu, 1.0 / np.sqrt(D), rows=rows)
    check(o, ref, f"o ({len(rows)} rows)", bound, TOL_FP8PV_MEANREL)


def test_long_table_and_norm():
    """The rotary table (all 2^18 rows, positions up to t = 96, h = 44, w = 996) and
    the norm + rotary pass (4 query and 2 K/V heads; sampled rows) at this size."""
    import torch

    import packed_varlen_attention_head_amd as h3a

    segs = [(97, 45, 60, LENS[0]), (1, 1, LENS[1], LENS[1])]
    dims, base, eps, R, Hq, Hk = (32, 32, 32), 10000.0, 1e-6, 96, 4, 2
    S = sum(LENS)
    log(f"[long] table + norm S={S}")
    tab = torch.empty((2, S, R // 2), dtype=torch.float32, device="cuda")
    cu = h3a.build_rope_table(segs, dims, base, tab)
    ocu, cos, sin = oracle.rope_table(segs, dims, base)
    assert np.array_equal(cu, ocu)
    g = to_f64(tab)
    err = max(np.abs(g[0] - cos).max(), np.abs(g[1] - sin).max())
    log(f"  table: max |gpu - oracle| = {err:.3e}")
    assert err <= 1.2e-7
    q = rng.normal_tensor(64, rng.TAG_Q, (S, Hq, D), "bf16")
    k = rng.normal_tensor(64, rng.TAG_K, (S, Hk, D), "bf16")
    gq = (1.0 + 0.1 * rng.normal(64, rng.TAG_GAMMA_Q, D)).astype(np.float32)
    gk = (1.0 + 0.1 * rng.normal(64, rng.TAG_GAMMA_K, D)).astype(np.float32)
    qd, kd = to_device(q, "bf16"), to_device(k, "bf16")
    qo, ko = torch.empty_like(qd), torch.empty_like(kd)
    h3a.qk_rmsnorm_rope(qd, kd, torch.from_numpy(gq).cuda(), torch.from_numpy(gk).cuda(), eps, tab, R,
                        q_out=qo, k_out=ko)
    rows = rows_to_check(cu)
    gqo, gko = to_f64(qo[rows.tolist()]), to_f64(ko[rows.tolist()])
    rq, rk = oracle.qk_rmsnorm_rope(rng.as_f64(q[rows], "bf16"), rng.as_f64(k[rows], "bf16"), gq, gk, eps,
                                    cos[rows], sin[rows], R)
    compare(gqo, rq, "bf16", f"q' ({len(rows)} rows)")
    compare(gko, rk, "bf16", f"k' ({len(rows)} rows)")
    for gg, r in ((gqo, rq), (gko, rk)):
        assert np.all(np.abs(gg - r) <= 2.0 ** -8 * np.abs(r) + 1e-5)
