"""Every output row and head of the headline workload (S = 20,423: video
10x30x54 + six 20x30 references + 623 audio tokens; 24 heads, d = 128,
rot96) against the fp64 oracle -- the attention kernel alone, on the exact
bf16 q', k' the GPU's norm + rotary pass produced, and the whole chain (table,
norm + rotary, attention) against the oracle's chain from the raw inputs.
Each oracle attention costs ~3.3e12 fp64 flop (tens of seconds on the
host's cores)."""
from __future__ import annotations

import functools

import numpy as np
import pytest

import oracle
from synth import configs, rng
from tests.gpu_util import compare, log, require_gpu, to_device, to_f64

pytestmark = pytest.mark.gpu

NAME = "h3_s20423_bf16"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()


@functools.lru_cache(maxsize=None)
def gpu_chain():
    """(q', k' bf16 bits from the GPU, GPU output as fp64) for the headline inputs."""
    import torch

    import packed_varlen_attention_head_amd as h3a

    w = configs.ALL[NAME]
    T = configs.make_tensors(w)
    q, k, v = (to_device(x, w.dtype) for x in (T.q, T.k, T.v))
    gq, gk = torch.from_numpy(T.gamma_q).cuda(), torch.from_numpy(T.gamma_k).cuda()
    tab = torch.empty((2, w.tokens, w.rot_dim // 2), dtype=torch.float32, device="cuda")
    cu = h3a.build_rope_table(w.segments, w.rot_dims, w.base, tab)
    qn, kn = torch.empty_like(q), torch.empty_like(k)
    h3a.qk_rmsnorm_rope(q, k, gq, gk, w.eps, tab, w.rot_dim, q_out=qn, k_out=kn)
    o = h3a.varlen_attn_fwd(qn, kn, v, cu, w.scale)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    return bits(qn), bits(kn), to_f64(o), T


def test_headline_attention_every_row():
    w = configs.ALL[NAME]
    qn_bits, kn_bits, o, T = gpu_chain()
    log(f"[headline full] attention alone, S={w.tokens}, all {w.heads} heads")
    cu = oracle.cu_seqlens(w.segments)
    ref = oracle.varlen_attention(rng.as_f64(qn_bits, "bf16"), rng.as_f64(kn_bits, "bf16"),
                                  rng.as_f64(T.v, "bf16"), cu, w.scale)
    compare(o, ref, "bf16", f"o (every one of {o.shape[0]} x {o.shape[1]} rows)")


def test_headline_chain_every_row():
    w = configs.ALL[NAME]
    _, _, o, T = gpu_chain()
    log(f"[headline full] table + norm/rotary + attention, S={w.tokens}")
    qf, kf, vf = (rng.as_f64(x, "bf16") for x in (T.q, T.k, T.v))
    ref = oracle.hot_path(qf, kf, vf, T.gamma_q, T.gamma_k, w.segments, w.rot_dims, w.base, w.eps, w.scale)
    compare(o, ref, "bf16", f"o (every one of {o.shape[0]} x {o.shape[1]} rows)")
