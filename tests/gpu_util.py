"""Helpers shared by the GPU tests: moving seeded numpy inputs to the device and
comparing device results with the fp64 oracle at the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np

# Tolerances: fp32 path max |g - r| <= 1e-5; bf16 path max |g - r| <= 2e-2 and
# mean-rel = sum|g - r| / sum|r| <= 1e-2.
TOL_F32 = 1e-5
TOL_BF16_ABS = 2e-2
TOL_BF16_MEANREL = 1e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import packed_varlen_attention_head_amd as h3a

    h3a.lib()  # raises if the HIP library is missing: no fallback


def to_device(x: np.ndarray, dtype: str):
    import torch

    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to("cuda")


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(g: np.ndarray, r: np.ndarray, dtype: str, what: str):
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - r)
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.abs(r).sum())
    mean_rel = float(err.sum() / denom) if denom > 0 else 0.0
    log(f"  {what}: max_abs={max_abs:.3e} mean_rel={mean_rel:.3e} n={err.size}")
    if dtype == "f32":
        assert max_abs <= TOL_F32, f"{what}: max abs {max_abs:.3e} > {TOL_F32}"
    else:
        assert max_abs <= TOL_BF16_ABS, f"{what}: max abs {max_abs:.3e} > {TOL_BF16_ABS}"
        assert mean_rel <= TOL_BF16_MEANREL, f"{what}: mean rel {mean_rel:.3e} > {TOL_BF16_MEANREL}"
    return max_abs, mean_rel


def sample_rows(cu, block_m: int = 256, every: int = 97, seed: int = 0) -> np.ndarray:
    """Every `every`-th row, each segment's first and last row, and every row of
    each segment's last (possibly partial) query tile."""
    cu = np.asarray(cu, dtype=np.int64)
    rows = set(range(0, int(cu[-1]), every))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        rows.update((a, b - 1))
        last_tile = a + ((b - a - 1) // block_m) * block_m
        rows.update(range(last_tile, b))
    return np.array(sorted(rows), dtype=np.int64)
