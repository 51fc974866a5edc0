"""The host tile planner (through the C ABI, CPU only): coverage, order and balance."""
import os
from collections import Counter

import numpy as np
import pytest

import packed_varlen_attention_head_amd as h3a
from synth import configs

pytestmark = pytest.mark.skipif(not os.path.exists(h3a.LIB_PATH), reason="libh3a.so not built")


def cu_of(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


CASES = {
    "h3_s20423": configs.H3_S20423.lengths,
    "h3_s25103": configs.H3_S25103.lengths,
    "two_seg": configs.TWO_SEG.lengths,
    "ragged64": configs.RAGGED64.lengths,
    "edges": [0, 1, 63, 64, 65, 0, 127, 128, 129, 0, 200],
    "single": [5000],
    "all_empty_but_one": [0, 0, 3, 0],
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("block_m", [128, 64])
@pytest.mark.parametrize("n_xcd", [1, 8])
def test_plan_covers_every_tile_once(name, block_m, n_xcd):
    lens = CASES[name]
    H = 24 if len(lens) > 2 else 3
    cu = cu_of(lens)
    plan = h3a.plan_tiles(cu, H, block_m, n_xcd)
    real = plan[plan[:, 1] > 0]
    want = Counter()
    for s, L in enumerate(lens):
        for h in range(H):
            for t in range(0, L, block_m):
                want[(int(cu[s]), L, t, h)] += 1
    got = Counter(tuple(int(x) for x in row) for row in real)
    assert got == want
    pad = plan[plan[:, 1] == 0]
    assert np.all(pad == 0)
    if n_xcd == 1:
        assert len(pad) == 0
    else:
        assert len(plan) % n_xcd == 0


@pytest.mark.parametrize("name", sorted(CASES))
def test_single_queue_is_longest_first(name):
    lens = CASES[name]
    plan = h3a.plan_tiles(cu_of(lens), 4, 128, 1)
    seg_len = plan[:, 1]
    assert np.all(np.diff(seg_len) <= 0)


@pytest.mark.parametrize("name", ["h3_s20423", "h3_s25103", "ragged64", "two_seg"])
def test_xcd_queues_balanced_and_longest_first(name):
    lens = CASES[name]
    n_xcd = 8
    plan = h3a.plan_tiles(cu_of(lens), 24, 128, n_xcd)
    loads = []
    for x in range(n_xcd):
        q = plan[x::n_xcd]
        q = q[q[:, 1] > 0]
        # each XCD sees its items in non-increasing segment length
        assert np.all(np.diff(q[:, 1]) <= 0)
        loads.append(float(np.sum(q[:, 1].astype(np.float64) + 128.0)))
    loads = np.array(loads)
    assert loads.max() / loads.mean() < 1.05, loads


def test_plan_skips_empty_segments_and_handles_all_empty():
    plan = h3a.plan_tiles(cu_of([0, 0, 0]), 2, 128, 8)
    assert len(plan) == 0


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("n_xcd", [1, 8])
def test_causal_plan_covers_every_tile_once(name, n_xcd):
    lens = CASES[name]
    H = 8
    cu = cu_of(lens)
    plan = h3a.plan_tiles(cu, H, 128, n_xcd, causal=True)
    real = plan[plan[:, 1] > 0]
    want = Counter((int(cu[s]), L, t, h) for s, L in enumerate(lens) for h in range(H) for t in range(0, L, 128))
    assert Counter(tuple(int(x) for x in row) for row in real) == want


def test_causal_plan_balances_key_work():
    """Each XCD's causal work (keys up to each item's last row) is within 5% of the mean."""
    lens = [8000, 3000, 1000, 700, 64, 1]
    n_xcd = 8
    plan = h3a.plan_tiles(cu_of(lens), 32, 128, n_xcd, causal=True)
    loads = []
    for x in range(n_xcd):
        q = plan[x::n_xcd]
        q = q[q[:, 1] > 0]
        keys = np.minimum(q[:, 1], q[:, 2] + 128).astype(np.float64)
        loads.append(float(np.sum(keys + 128.0)))
        # within one XCD the first item is one of the costliest
        assert keys[0] == keys.max()
    loads = np.array(loads)
    assert loads.max() / loads.mean() < 1.05, loads


def test_causal_and_bidirectional_plans_differ_only_in_order():
    cu = cu_of(CASES["h3_s20423"])
    a = h3a.plan_tiles(cu, 24, 128, 1)
    b = h3a.plan_tiles(cu, 24, 128, 1, causal=True)
    assert sorted(map(tuple, a.tolist())) == sorted(map(tuple, b.tolist()))


def test_oversized_plan_rejected_before_building():
    """A packing whose plan would exceed 2^26 work items is refused up front with
    EUNSUPPORTED, before any host memory is spent building it, also just above
    the bound (8,193 query tiles x 2^13 heads = 2^26 + 2^13 items)."""
    for cu, heads, block_m in (([0, 1 << 20], 1 << 14, 1), ([0, (1 << 20) + 1], 1 << 13, 128)):
        with pytest.raises(h3a.H3AError) as e:
            h3a.plan_tiles(np.array(cu, dtype=np.int64), heads=heads, block_m=block_m, n_xcd=8)
        assert e.value.status == h3a.H3A_EUNSUPPORTED
        assert "work items" in str(e.value)
