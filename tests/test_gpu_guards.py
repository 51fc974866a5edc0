"""Every attention variant writes exactly its output rows and columns: outputs go
to a view with a padded token stride inside a buffer filled with a canary, with
a guard row before and after, and every byte outside the view must keep the
canary; inside the view the values equal those of the same call on a contiguous
output bit for bit.  Segment lengths put partial query tiles (rows past a
segment's end, whose lanes must not store) at every segment end."""
from __future__ import annotations

import numpy as np
import pytest

from synth import rng
from tests.gpu_util import log, require_gpu, to_device

pytestmark = pytest.mark.gpu

LENS = [150, 0, 77, 300, 1, 64]
CANARY = -1024.0  # exactly representable in bf16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()


def variants(h3a, q, k, v, cu, scale, D, R, tab, gam):
    """name -> callable(out) running that variant into `out`."""
    q8e, k8e = h3a.quantize_e4m3(q), h3a.quantize_e4m3(k)
    vt8 = h3a.prepare_vt_e4m3(v, cu)
    qi8, ki8 = h3a.quantize_i8_rows(q), h3a.quantize_i8_keys(k, cu)
    return {
        "bf16": lambda o: h3a.varlen_attn_fwd_ex(q, k, v, cu, scale, out=o),
        "causal": lambda o: h3a.varlen_attn_fwd_ex(q, k, v, cu, scale, causal=True, out=o),
        "qnorm": lambda o: h3a.varlen_attn_fwd_qnorm(q, k, v, cu, scale, gam, 1e-6, tab, R, out=o),
        "fp8qk": lambda o: h3a.varlen_attn_fwd_fp8qk(q8e, k8e, v, cu, scale, out=o),
        "fp8": lambda o: h3a.varlen_attn_fwd_fp8(q8e, k8e, vt8, cu, scale, out=o),
        "i8qk": lambda o: h3a.varlen_attn_fwd_i8qk(qi8, ki8, v, cu, scale, out=o),
        "i8qk_fp8pv": lambda o: h3a.varlen_attn_fwd_i8qk_fp8pv(qi8, ki8, vt8, cu, scale, out=o),
        "noalloc": lambda o: h3a.varlen_attn_fwd_noalloc(q, k, v, cu, scale, out=o),
    }


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_outputs_stay_inside_their_view(D, split):
    import torch

    import packed_varlen_attention_head_amd as h3a

    Hq, Hkv, R = 4, 2, 32 if D == 64 else 96
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int64)
    S = int(cu[-1])
    seed = 91 + D
    q = to_device(rng.normal_tensor(seed, rng.TAG_Q, (S, Hq, D), "bf16"), "bf16")
    k = to_device(rng.normal_tensor(seed, rng.TAG_K, (S, Hkv, D), "bf16"), "bf16")
    v = to_device(rng.normal_tensor(seed, rng.TAG_V, (S, Hkv, D), "bf16"), "bf16")
    tab = torch.empty((2, S, R // 2), dtype=torch.float32, device="cuda")
    h3a.build_rope_table([(1, 1, max(L, 1), L) for L in LENS], _dims(R), 10000.0, tab)
    gam = torch.ones(D, dtype=torch.float32, device="cuda")
    scale = 1.0 / np.sqrt(D)
    pad = 24
    runs = variants(h3a, q, k, v, cu, scale, D, R, tab, gam)
    if split:
        h3a.set_split_policy(h3a.H3A_SPLIT_ALWAYS)
    try:
        for name, fn in runs.items():
            if split and name in ("causal", "noalloc"):
                continue  # causal plans and the allocation-free call are never split
            log(f"[guards] D={D} split={split} {name}")
            big = torch.full((S + 2, Hq * D + pad), CANARY, dtype=torch.bfloat16, device="cuda")
            view = torch.as_strided(big, (S, Hq, D), (Hq * D + pad, D, 1), storage_offset=Hq * D + pad)
            fn(view)
            ref = torch.empty((S, Hq, D), dtype=torch.bfloat16, device="cuda")
            fn(ref)
            torch.cuda.synchronize()
            g = big.float().cpu().numpy()
            assert np.all(g[0] == CANARY) and np.all(g[S + 1] == CANARY), name
            assert np.all(g[1:S + 1, Hq * D:] == CANARY), name
            assert torch.equal(view.view(torch.int16), ref.view(torch.int16)), name
    finally:
        h3a.set_split_policy(h3a.H3A_SPLIT_AUTO)


def _dims(R):
    """Rotary axis dims (t, h, w) summing to R, each a multiple of 16."""
    return {96: (32, 32, 32), 32: (16, 0, 16)}[R]
