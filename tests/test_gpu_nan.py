"""NaN and infinity handling of the low-precision path against the bf16 one.

OCP E4M3 ("fn") has no infinities and two NaN codes (0x7f, 0xff).  A block's
scale comes from its largest finite-or-infinite magnitude, NaN ignored: an
infinity gives the block the scale 2^120 and saturates to +-448 under it (the
rest of its block then rounds to zero), and a NaN becomes a NaN code without
changing its block's scale.  So a NaN in q, k or v reaches the attention
output through the FP8 kernels exactly as through the bf16 kernel: a NaN query
element makes that query row NaN, a NaN key element makes every row of its
segment and head NaN, a NaN value element that dim of every row of its segment
and head, and nothing else is touched."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import rng
from tests.gpu_util import log, require_gpu, to_device

pytestmark = pytest.mark.gpu

LENS = [150, 0, 77, 29]
H, D = 2, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    import packed_varlen_attention_head_amd as h3a

    h3a.release_caches()


def h3a():
    import packed_varlen_attention_head_amd as m

    return m


def _bits(x: float) -> int:
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0] >> 16)


def _inputs(seed):
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int64)
    S = int(cu[-1])
    q, k, v = (rng.normal_tensor(seed, tag, (S, H, D), "bf16") for tag in (rng.TAG_Q, rng.TAG_K, rng.TAG_V))
    return cu, q, k, v


def test_quantize_nan_and_infinities():
    import torch

    _, q, _, _ = _inputs(3)
    x = q.copy()
    x[5, 1, 7] = _bits(np.nan)
    x[9, 0, 3] = _bits(np.inf)
    x[11, 1, 100] = _bits(-np.inf)
    codes, scales = (t.cpu().numpy() for t in h3a().quantize_e4m3(to_device(x, "bf16")))
    torch.cuda.synchronize()
    log(f"[nan] codes: nan={codes[5, 1, 7]:#x} +inf={codes[9, 0, 3]:#x} -inf={codes[11, 1, 100]:#x}; "
        f"scales {scales[1, 5, 0]} {scales[0, 9, 0]} {scales[1, 11, 3]}")
    assert codes[5, 1, 7] in (0x7F, 0xFF)
    assert codes[9, 0, 3] == 0x7E and codes[11, 1, 100] == 0xFE
    assert scales[0, 9, 0] == 247 and scales[1, 11, 3] == 247  # 2^120 (scales are [head, token, block])
    # the other elements of an infinity's block, N(0,1) times 2^-120, round to (signed) zero
    for (t, h, b), d in (((9, 0, 0), 3), ((11, 1, 3), 100 - 96)):
        rest = np.delete(codes[t, h, 32 * b:32 * b + 32], d)
        assert np.all((rest & 0x7F) == 0)
    # every other block, the NaN's included (its NaN read as zero), as the oracle's codec
    xf = rng.as_f64(x, "bf16")
    xf[5, 1, 7] = 0.0
    want, X = oracle.mx_quantize(np.where(np.isinf(xf), 0.0, xf), axis=-1)
    keep = np.ones(X.shape, dtype=bool)  # [token, head, block]
    keep[9, 0, 0] = keep[11, 1, 3] = False
    assert np.array_equal(scales.transpose(1, 0, 2)[keep], (X + 127).astype(np.uint8)[keep])
    code_keep = np.repeat(keep, 32, axis=-1)
    code_keep[5, 1, 7] = False
    assert np.array_equal(codes[code_keep], want[code_keep])


def _nan_rows(o, cu, row=None, seg=None, head=0):
    """Expected NaN mask of the output: one query row, or every row of a segment, in one head."""
    m = np.zeros(o.shape[:2], dtype=bool)
    if row is not None:
        m[row, head] = True
    if seg is not None:
        m[int(cu[seg]):int(cu[seg + 1]), head] = True
    return m


@pytest.mark.parametrize("where", ["q", "k", "v"])
def test_nan_propagates_like_bf16(where):
    import torch

    cu, q, k, v = _inputs(7)
    # a NaN in row 160 (segment 2, local row 10), head 1, dim 40
    row, head = 160, 1
    t = {"q": q, "k": k, "v": v}[where]
    t[row, head, 40] = _bits(np.nan)
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    scale = 1.0 / np.sqrt(D)
    seg = int(np.searchsorted(cu, row, side="right") - 1)
    expect = _nan_rows(np.zeros((int(cu[-1]), H)), cu, row=row if where == "q" else None,
                       seg=None if where == "q" else seg, head=head)
    outs = {
        "bf16": h3a().varlen_attn_fwd(qd, kd, vd, cu, scale),
        "fp8qk": h3a().varlen_attn_fwd_fp8qk(h3a().quantize_e4m3(qd), h3a().quantize_e4m3(kd), vd, cu, scale),
        "fp8": h3a().varlen_attn_fwd_fp8(h3a().quantize_e4m3(qd), h3a().quantize_e4m3(kd),
                                         h3a().prepare_vt_e4m3(vd, cu), cu, scale),
    }
    torch.cuda.synchronize()
    for name, o in outs.items():
        nan = torch.isnan(o.float()).cpu().numpy()
        rows_nan = nan.any(axis=2)
        log(f"[nan] {where} {name}: NaN rows {int(rows_nan.sum())} expected {int(expect.sum())}")
        assert np.array_equal(rows_nan, expect), name
        if where == "v":  # o = sum_j p_j v_j: only the NaN's own dim
            assert np.array_equal(nan[:, :, 40], expect) and not nan[:, :, :40].any() and not nan[:, :, 41:].any()
        else:  # a NaN score reaches the row's normaliser: every dim
            assert np.array_equal(nan.all(axis=2), expect), name
