"""Oracle property (CPU): per-block power-of-two scales keep E4M3's relative
precision whatever the operands' magnitude, which unscaled E4M3 does not --
values far below 2^-6 lose their mantissa bits, values past 448 saturate."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth import rng

CU = np.array([0, 300, 429, 493, 494, 700])


def _mean_rel(o, ref):
    return float(np.abs(o - ref).sum() / np.abs(ref).sum())


@pytest.mark.parametrize("vmag", [1e-3, 1.0, 1e3])
def test_block_scales_keep_precision_across_magnitudes(vmag):
    S = int(CU[-1])
    q, k, v = (rng.as_f64(rng.normal_tensor(5, tag, (S, 2, 64), "bf16"), "bf16")
               for tag in (rng.TAG_Q, rng.TAG_K, rng.TAG_V))
    v = v * vmag
    ref = oracle.varlen_attention(q, k, v, CU, 0.125)
    mx = _mean_rel(oracle.varlen_attention_mx(q, k, v, CU, 0.125), ref)
    plain = _mean_rel(oracle.varlen_attention_fp8(q, k, v, CU, 0.125), ref)
    # three mantissa bits on q, k and v: a few percent at every magnitude
    assert 1e-2 < mx < 7e-2, mx
    if vmag == 1.0:
        assert abs(plain - mx) < 1e-2 * mx  # in range, the scales change nothing
    else:
        assert plain > 0.3, plain  # flushed toward subnormals, or saturated at 448
