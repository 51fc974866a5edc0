"""The allocation-free attention entry point (plan in the library's fixed
per-GPU array) against h3a_varlen_attn_fwd_ex, through the C ABI: the same
kernels on the same work items, so the outputs must be equal bit for bit --
on two calls in a row, the second with a smaller input, for bf16 and fp32,
bidirectional and causal, grouped K/V; on two streams back to back (the
second call waits for the first's kernel before rewriting the shared plan);
and on the headline packing (S = 20,423, 24 heads), which is also compared
with the oracle on sampled rows.  The reference calls use the never-split
policy: a split plan's items differ from the fixed-array plan's."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import configs, rng
from tests.gpu_util import compare, log, require_gpu, sample_rows, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import packed_varlen_attention_head_amd as h3a

    # the reference path on the same (unsplit) work items as the fixed-array plan
    h3a.set_split_policy(h3a.H3A_SPLIT_NEVER)
    yield
    h3a.set_split_policy(h3a.H3A_SPLIT_AUTO)
    h3a.release_caches()


def h3a():
    import packed_varlen_attention_head_amd as m

    return m


def _case(seed, lens, Hq, Hkv, D, dtype):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S = int(cu[-1])
    q = rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), dtype)
    k = rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), dtype)
    v = rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), dtype)
    return cu, [to_device(x, dtype) for x in (q, k, v)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_equals_cached_plan_two_calls(dtype, causal):
    import torch

    big = _case(101, [700, 0, 300, 129, 65, 1, 1000], 4, 2, 128, dtype)
    small = _case(102, [200, 37], 2, 1, 64, dtype)
    for name, (cu, (q, k, v)) in (("big", big), ("small", small)):
        D = q.shape[2]
        scale = 1.0 / np.sqrt(D)
        ref = h3a().varlen_attn_fwd_ex(q, k, v, cu, scale, causal=causal)
        out = torch.full_like(ref, float("nan"))
        h3a().varlen_attn_fwd_noalloc(q, k, v, cu, scale, out, causal=causal)
        torch.cuda.synchronize()
        same = torch.equal(out, ref)
        log(f"[noalloc] {dtype} causal={causal} {name}: S={q.shape[0]} H={q.shape[1]}/{k.shape[1]} D={D} "
            f"equal to cached-plan path = {same}")
        assert same


def test_noalloc_two_streams_back_to_back():
    """The second call (another stream, smaller input) is enqueued while the first
    may still run; both results must be the cached-plan results."""
    import torch

    (cu1, (q1, k1, v1)), (cu2, (q2, k2, v2)) = (_case(111, [3000, 2000], 8, 8, 128, "bf16"),
                                                _case(112, [129, 64, 7], 2, 2, 128, "bf16"))
    s = 1.0 / np.sqrt(128)
    ref1 = h3a().varlen_attn_fwd(q1, k1, v1, cu1, s)
    ref2 = h3a().varlen_attn_fwd(q2, k2, v2, cu2, s)
    torch.cuda.synchronize()
    o1, o2 = torch.empty_like(ref1), torch.empty_like(ref2)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        o1.fill_(float("nan"))
        o2.fill_(float("nan"))
        torch.cuda.synchronize()
        h3a().varlen_attn_fwd_noalloc(q1, k1, v1, cu1, s, o1, stream=sa)
        h3a().varlen_attn_fwd_noalloc(q2, k2, v2, cu2, s, o2, stream=sb)
        torch.cuda.synchronize()
        ok = torch.equal(o1, ref1) and torch.equal(o2, ref2)
        log(f"[noalloc] two streams, round {rep}: both equal = {ok}")
        assert ok


def test_noalloc_headline_packing():
    import torch

    w = configs.ALL["h3_s20423_bf16"]
    T = configs.make_tensors(w)
    q, k, v = (to_device(x, "bf16") for x in (T.q, T.k, T.v))
    cu = oracle.cu_seqlens(w.segments)
    ref = h3a().varlen_attn_fwd(q, k, v, cu, w.scale)
    out = torch.empty_like(ref)
    h3a().varlen_attn_fwd_noalloc(q, k, v, cu, w.scale, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    rows = sample_rows(cu)
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (T.q, T.k, T.v))
    compare(to_f64(out)[rows], oracle.varlen_attention_rows(qf, kf, vf, cu, w.scale, rows), "bf16",
            f"noalloc headline ({len(rows)} sampled rows)")
