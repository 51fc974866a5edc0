"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, per stage and end to end, for every workload plus edge
cases, isolation, determinism and layout checks."""
from __future__ import annotations

import functools

import numpy as np
import pytest

import oracle
from synth import configs, rng
from tests.gpu_util import compare, log, require_gpu, sample_rows, to_device, to_f64

pytestmark = pytest.mark.gpu

ALL = list(configs.ALL)
SMALL = {"tiny_f32"}


@functools.lru_cache(maxsize=None)
def tensors(name):
    return configs.make_tensors(configs.ALL[name])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()


def h3a():
    import packed_varlen_attention_head_amd as m

    return m


def dev_table(w):
    import torch

    t = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    cu = h3a().build_rope_table(w.segments, w.rot_dims, w.base, t)
    return t, cu


# ---------------------------------------------------------------------------
# a1: rotary table
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ALL)
def test_rope_table(name):
    import torch

    w = configs.ALL[name]
    log(f"[rope_table] {name} S={w.tokens}")
    t, cu = dev_table(w)
    torch.cuda.synchronize()
    ocu, ocos, osin = oracle.rope_table(w.segments, w.rot_dims, w.base)
    assert np.array_equal(cu, ocu)
    g = to_f64(t)
    # fp64 angles rounded once to fp32: within half an fp32 ulp of the fp64 value
    # (plus the last-bit difference of two libm implementations).
    err = max(np.abs(g[0] - ocos).max(), np.abs(g[1] - osin).max())
    log(f"  max |table - oracle| = {err:.3e}")
    assert err <= 1.2e-7


# ---------------------------------------------------------------------------
# a2: fused RMSNorm + rotary
# ---------------------------------------------------------------------------

def run_qk(w, T, **kw):
    import torch

    q = to_device(T.q, w.dtype)
    k = to_device(T.k, w.dtype)
    gq = torch.from_numpy(T.gamma_q).cuda()
    gk = torch.from_numpy(T.gamma_k).cuda()
    tab, _ = dev_table(w)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    h3a().qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim, q_out=qo, k_out=ko, **kw)
    torch.cuda.synchronize()
    return q, k, qo, ko, gq, gk, tab


@pytest.mark.parametrize("name", ALL)
def test_qk_rmsnorm_rope(name):
    w = configs.ALL[name]
    T = tensors(name)
    log(f"[qk_rmsnorm_rope] {name}")
    _, _, qo, ko, _, _, _ = run_qk(w, T)
    rows = np.arange(w.tokens) if name in SMALL else sample_rows(oracle.cu_seqlens(w.segments))
    _, cos, sin = oracle.rope_table(w.segments, w.rot_dims, w.base)
    qf, kf = rng.as_f64(T.q[rows], w.dtype), rng.as_f64(T.k[rows], w.dtype)
    rq, rk = oracle.qk_rmsnorm_rope(qf, kf, T.gamma_q, T.gamma_k, w.eps, cos[rows], sin[rows], w.rot_dim)
    gq, gk = to_f64(qo)[rows], to_f64(ko)[rows]
    compare(gq, rq, w.dtype, "q'")
    compare(gk, rk, w.dtype, "k'")
    if w.dtype == "bf16":
        # one RNE rounding of an fp32 result: within 2^-8 relative (+ fp32 slack)
        for g, r in ((gq, rq), (gk, rk)):
            assert np.all(np.abs(g - r) <= 2.0 ** -8 * np.abs(r) + 1e-5)


def test_qk_in_place_matches_out_of_place():
    w = configs.TWO_SEG
    T = tensors(w.name)
    q, k, qo, ko, gq, gk, tab = run_qk(w, T)
    import torch

    h3a().qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim)  # in place
    torch.cuda.synchronize()
    assert torch.equal(q, qo) and torch.equal(k, ko)


# ---------------------------------------------------------------------------
# a3 + a4: varlen attention
# ---------------------------------------------------------------------------

def run_attn(q, k, v, cu, scale, **kw):
    import torch

    o = h3a().varlen_attn_fwd(q, k, v, cu, scale, **kw)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("name", ALL)
def test_varlen_attention(name):
    w = configs.ALL[name]
    T = tensors(name)
    log(f"[varlen_attention] {name} S={w.tokens} segments={len(w.segments)}")
    cu = oracle.cu_seqlens(w.segments)
    q, k, v = (to_device(x, w.dtype) for x in (T.q, T.k, T.v))
    o = to_f64(run_attn(q, k, v, cu, w.scale))
    qf, kf, vf = (rng.as_f64(x, w.dtype) for x in (T.q, T.k, T.v))
    if name in SMALL:
        ref = oracle.varlen_attention(qf, kf, vf, cu, w.scale)
        compare(o, ref, w.dtype, "o")
    else:
        rows = sample_rows(cu)
        ref = oracle.varlen_attention_rows(qf, kf, vf, cu, w.scale, rows)
        compare(o[rows], ref, w.dtype, f"o ({len(rows)} sampled rows)")
    assert np.all(np.isfinite(o))


EDGE_LENGTHS = [1, 63, 64, 65, 0, 127, 128, 129, 200, 0, 517, 2]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_varlen_attention_edges(dtype, D):
    """Ragged tails, empty and length-1 segments, partial tiles on both sides."""
    H = 3
    cu = np.concatenate([[0], np.cumsum(EDGE_LENGTHS)])
    S = int(cu[-1])
    log(f"[edges] dtype={dtype} D={D} S={S}")
    xs = [rng.normal_tensor(11, tag, (S, H, D), dtype) for tag in (1, 2, 3)]
    o = to_f64(run_attn(*(to_device(x, dtype) for x in xs), cu, 1 / np.sqrt(D)))
    ref = oracle.varlen_attention(*(rng.as_f64(x, dtype) for x in xs), cu, 1 / np.sqrt(D))
    compare(o, ref, dtype, "o")


def test_varlen_attention_single_long_segment():
    H, D, L = 2, 128, 3000
    log(f"[single segment] L={L}")
    xs = [rng.normal_tensor(12, tag, (L, H, D), "bf16") for tag in (1, 2, 3)]
    cu = np.array([0, L])
    o = to_f64(run_attn(*(to_device(x, "bf16") for x in xs), cu, 1 / np.sqrt(D)))
    ref = oracle.varlen_attention(*(rng.as_f64(x, "bf16") for x in xs), cu, 1 / np.sqrt(D))
    compare(o, ref, "bf16", "o")


def test_varlen_attention_sharp_softmax():
    """Logit std ~ 4: peaked rows that exercise the running-max rescale."""
    H, D = 4, 128
    lens = [1000, 333, 64]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S = int(cu[-1])
    log("[sharp softmax]")
    q = rng.normal_tensor(13, 1, (S, H, D), "bf16", std=4.0)
    k, v = (rng.normal_tensor(13, tag, (S, H, D), "bf16") for tag in (2, 3))
    o = to_f64(run_attn(*(to_device(x, "bf16") for x in (q, k, v)), cu, 1 / np.sqrt(D)))
    ref = oracle.varlen_attention(*(rng.as_f64(x, "bf16") for x in (q, k, v)), cu, 1 / np.sqrt(D))
    compare(o, ref, "bf16", "o")
    # the outputs are far from the uniform-attention mean: the check has teeth
    assert np.abs(ref).mean() > 0.2


def test_varlen_attention_rising_logits():
    """Logits that grow along the keys (and one tile 40x larger than the rest):
    later tiles exceed the running reference by far more than the bf16 steady
    loop's bound on a tile's probability sum, so its recompute path runs many
    times, once where an unchecked tile would overflow to infinity."""
    H, D = 2, 128
    lens = [700, 300, 129]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S = int(cu[-1])
    log("[rising logits]")
    q, k0, v = (rng.normal_tensor(14, tag, (S, H, D), "bf16") for tag in (1, 2, 3))
    gain = np.ones(S)
    gain[:700] = 1.0 + np.arange(700) / 50.0      # logit std grows to ~15 along segment 0
    gain[700 + 192:700 + 256] = 40.0              # one 64-key tile of segment 1 dominates
    kf = rng.as_f64(k0, "bf16") * gain[:, None, None]
    k = rng.f32_to_bf16_bits(kf.astype(np.float32))
    o = to_f64(run_attn(*(to_device(x, "bf16") for x in (q, k, v)), cu, 1 / np.sqrt(D)))
    ref = oracle.varlen_attention(*(rng.as_f64(x, "bf16") for x in (q, k, v)), cu, 1 / np.sqrt(D))
    compare(o, ref, "bf16", "o")
    # peaked rows: far from the uniform mean, so the comparison has teeth
    assert np.abs(ref[:700]).mean() > 0.3 and np.abs(ref[700:1000]).mean() > 0.3


def test_varlen_attention_segment_isolation():
    import torch

    H, D = 3, 128
    lens = [300, 200, 129]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S = int(cu[-1])
    log("[segment isolation]")
    xs = [to_device(rng.normal_tensor(14, tag, (S, H, D), "bf16"), "bf16") for tag in (1, 2, 3)]
    base = run_attn(*xs, cu, 0.1)
    for i in range(3):
        ys = [x.clone() for x in xs]
        ys[i][350] += 1.0  # a token of segment 1
        o = run_attn(*ys, cu, 0.1)
        assert torch.equal(o[:300], base[:300]) and torch.equal(o[500:], base[500:])
        assert not torch.equal(o[300:500], base[300:500])


def test_determinism_and_streams():
    import torch

    w = configs.TWO_SEG
    T = tensors(w.name)
    log("[determinism]")
    cu = oracle.cu_seqlens(w.segments)
    q, k, v = (to_device(x, w.dtype) for x in (T.q, T.k, T.v))
    o1 = run_attn(q, k, v, cu, w.scale)
    o2 = run_attn(q, k, v, cu, w.scale)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o3 = h3a().varlen_attn_fwd(q, k, v, cu, w.scale, stream=s)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3)
    _, _, qo1, ko1, gq, gk, tab = run_qk(w, T)
    qo2, ko2 = torch.empty_like(qo1), torch.empty_like(ko1)
    with torch.cuda.stream(s):
        h3a().qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim, q_out=qo2, k_out=ko2, stream=s)
    s.synchronize()
    assert torch.equal(qo1, qo2) and torch.equal(ko1, ko2)


def test_strided_views_and_guard_rows():
    """q, k, v as views of one fused [S, 3, H, D] buffer; outputs with padded
    token stride and guard rows, which must stay untouched."""
    import torch

    H, D = 4, 128
    lens = [150, 0, 77, 300]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S = int(cu[-1])
    log("[strided views]")
    fused = rng.normal_tensor(15, 1, (S, 3, H, D), "bf16")
    qkv = to_device(fused, "bf16")
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    pad = 16
    canary = -1024.0  # exactly representable in bf16
    big = torch.full((S + 2, H * D + pad), canary, dtype=torch.bfloat16, device="cuda")
    out = torch.as_strided(big, (S, H, D), (H * D + pad, D, 1), storage_offset=H * D + pad)
    run_attn(q, k, v, cu, 1 / np.sqrt(D), out=out)
    g = big.float().cpu().numpy()
    assert np.all(g[0] == canary) and np.all(g[S + 1] == canary)
    assert np.all(g[1:S + 1, H * D:] == canary)
    x64 = rng.as_f64(fused, "bf16")
    ref = oracle.varlen_attention(x64[:, 0], x64[:, 1], x64[:, 2], cu, 1 / np.sqrt(D))
    compare(to_f64(out), ref, "bf16", "o")
    # norm + rotary in place on the strided q, k views; v (the third slot) untouched
    tab = torch.empty((2, S, 48), dtype=torch.float32, device="cuda")
    segs = [(1, 10, 15, 150), (1, 1, 1, 0), (7, 11, 1, 77), (3, 10, 10, 300)]
    h3a().build_rope_table(segs, (32, 32, 32), 10000.0, tab)
    g1 = torch.ones(D, device="cuda")
    v_before = v.clone()
    h3a().qk_rmsnorm_rope(q, k, g1, g1, 1e-6, tab, 96)
    torch.cuda.synchronize()
    assert torch.equal(v, v_before)
    _, cos, sin = oracle.rope_table(segs, (32, 32, 32), 10000.0)
    rq, rk = oracle.qk_rmsnorm_rope(x64[:, 0], x64[:, 1], np.ones(D), np.ones(D), 1e-6, cos, sin, 96)
    compare(to_f64(q), rq, "bf16", "q' (strided, in place)")
    compare(to_f64(k), rk, "bf16", "k' (strided, in place)")


# ---------------------------------------------------------------------------
# the whole chain
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_f32", "two_seg_bf16", "h3_s20423_bf16"])
def test_hot_path_end_to_end(name):
    import torch

    w = configs.ALL[name]
    T = tensors(name)
    log(f"[hot path] {name}")
    q, k, v = (to_device(x, w.dtype) for x in (T.q, T.k, T.v))
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    cu = h3a().build_rope_table(w.segments, w.rot_dims, w.base, tab)
    h3a().qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim)
    o = to_f64(run_attn(q, k, v, cu, w.scale))
    qf, kf, vf = (rng.as_f64(x, w.dtype) for x in (T.q, T.k, T.v))
    if name in SMALL:
        ref = oracle.hot_path(qf, kf, vf, T.gamma_q, T.gamma_k, w.segments, w.rot_dims, w.base, w.eps, w.scale)
        compare(o, ref, w.dtype, "o")
    else:
        ocu, cos, sin = oracle.rope_table(w.segments, w.rot_dims, w.base)
        qn, kn = oracle.qk_rmsnorm_rope(qf, kf, T.gamma_q, T.gamma_k, w.eps, cos, sin, w.rot_dim)
        rows = sample_rows(ocu)
        ref = oracle.varlen_attention_rows(qn, kn, vf, ocu, w.scale, rows)
        compare(o[rows], ref, w.dtype, f"o ({len(rows)} sampled rows)")


def test_plan_cache_eviction():
    """More distinct packings than the plan cache holds (256): old plans are evicted (after a
    device synchronisation) and every call still matches the oracle."""
    import torch

    H, D = 2, 64
    S = 300
    qb = rng.normal_tensor(90, rng.TAG_Q, (S, H, D), "bf16")
    kb = rng.normal_tensor(90, rng.TAG_K, (S, H, D), "bf16")
    vb = rng.normal_tensor(90, rng.TAG_V, (S, H, D), "bf16")
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    h3a().release_caches()
    log("[plan cache] 270 packings")
    outs = []
    for i in range(270):
        cu = np.array([0, 1 + i, S], dtype=np.int64)
        outs.append((cu, h3a().varlen_attn_fwd(q, k, v, cu, 0.125)))
    torch.cuda.synchronize()
    for i in (0, 1, 100, 255, 256, 269):
        cu, o = outs[i]
        compare(to_f64(o), oracle.varlen_attention(qf, kf, vf, cu, 0.125), "bf16", f"packing {i}")
    # a packing seen long ago (evicted) is planned again
    cu, _ = outs[0]
    compare(to_f64(h3a().varlen_attn_fwd(q, k, v, cu, 0.125)), oracle.varlen_attention(qf, kf, vf, cu, 0.125),
            "bf16", "packing 0 again")


def test_plan_cache_threads():
    """Four host threads, each on its own stream, attend over 80 distinct packings
    each (320 > the 256 cached plans): lookups, launches and evictions interleave
    across threads.  A plan is looked up and its kernel enqueued under the cache
    lock, and an eviction waits for the device first, so every output must still
    match the oracle."""
    import threading

    import torch

    H, D, S = 2, 64, 300
    qb = rng.normal_tensor(91, rng.TAG_Q, (S, H, D), "bf16")
    kb = rng.normal_tensor(91, rng.TAG_K, (S, H, D), "bf16")
    vb = rng.normal_tensor(91, rng.TAG_V, (S, H, D), "bf16")
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    h3a().release_caches()
    log("[plan cache] 4 threads x 80 packings")
    results, errors = {}, []

    def worker(w):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for i in range(80):
                    cut = 1 + (w * 80 + i) % (S - 1)
                    cu = np.array([0, cut, S], dtype=np.int64)
                    results[(w, i)] = (cu, h3a().varlen_attn_fwd(q, k, v, cu, 0.125, stream=stream))
            stream.synchronize()
        except Exception as e:  # reported after join
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(w,)) for w in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    assert len(results) == 320
    for key in ((0, 0), (1, 40), (2, 79), (3, 79), (3, 0)):
        cu, o = results[key]
        compare(to_f64(o), oracle.varlen_attention(qf, kf, vf, cu, 0.125), "bf16", f"thread {key[0]} packing {key[1]}")
    h3a().release_caches()


def test_release_caches_with_kernels_in_flight():
    """Releasing the plan cache right after queuing attention calls (no host
    synchronisation in between) waits for them: every output still matches."""
    import torch

    H, D, S = 2, 64, 300
    qb = rng.normal_tensor(92, rng.TAG_Q, (S, H, D), "bf16")
    kb = rng.normal_tensor(92, rng.TAG_K, (S, H, D), "bf16")
    vb = rng.normal_tensor(92, rng.TAG_V, (S, H, D), "bf16")
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (qb, kb, vb))
    log("[plan cache] release with 12 launches queued")
    torch.cuda.synchronize()
    outs = []
    for i in range(12):
        cu = np.array([0, 7 + 23 * i, S], dtype=np.int64)
        outs.append((cu, h3a().varlen_attn_fwd(q, k, v, cu, 0.125)))
    h3a().release_caches()
    torch.cuda.synchronize()
    for i in (0, 5, 11):
        cu, o = outs[i]
        compare(to_f64(o), oracle.varlen_attention(qf, kf, vf, cu, 0.125), "bf16", f"packing {i}")
