"""Host-only checks of the split planner (no GPU): the planner is compiled with
g++ into a small dump tool (tests/native/plan_split_dump.cpp) and its plans are
checked for coverage -- every (segment, head, query tile) sees each of its key
tiles exactly once, in ranges that start on even tiles -- partial-slot
bookkeeping that matches the merge list, and the automatic policy's choices on
the benchmark packings."""
from __future__ import annotations

import os
import shutil
import subprocess
from collections import defaultdict

import pytest

from synth import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "packed_varlen_attention_head_amd", "csrc")
AUTO, NEVER, ALWAYS = 0, 1, 2


@pytest.fixture(scope="module")
def tool(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("plan") / "plan_split_dump")
    cmd = ["g++", "-std=c++17", "-O1", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "native", "plan_split_dump.cpp"), os.path.join(CSRC, "planner.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


def plan(tool, policy, heads, lens, slots=512, n_xcd=8, block_m=128):
    args = [tool, str(policy), str(slots), str(n_xcd), str(heads), str(block_m)] + [str(x) for x in lens]
    lines = subprocess.run(args, check=True, capture_output=True, text=True).stdout.split("\n")
    n = int(lines[0].split()[1])
    items = [tuple(map(int, ln.split())) for ln in lines[1:1 + n]]
    m = int(lines[1 + n].split()[1])
    merges = [tuple(map(int, ln.split())) for ln in lines[2 + n:2 + n + m]]
    parts = int(lines[2 + n + m].split()[1])
    return items, merges, parts


def check_plan(items, merges, parts, heads, lens, block_m=128):
    starts = [sum(lens[:i]) for i in range(len(lens))]
    ranges = defaultdict(list)  # (seg_start, head, q_start) -> [(kt0, kt1, part)]
    length = {}
    for (seg_start, seg_len, q_start, head, _col0, kt0, kt1, part) in items:
        if seg_len == 0:
            continue  # padding item
        nk = -(-seg_len // 64)
        if kt1 == 0:
            assert kt0 == 0 and part == 0
            kt1 = nk
        else:
            assert part > 0 and kt0 % 2 == 0 and 0 <= kt0 < kt1 <= nk
        ranges[(seg_start, head, q_start)].append((kt0, kt1, part))
        length[seg_start] = seg_len
    want = {(starts[s], h, t * block_m) for s, L in enumerate(lens) if L > 0 for h in range(heads)
            for t in range(-(-L // block_m))}
    assert set(ranges) == want
    assert all(length[starts[i]] == L for i, L in enumerate(lens) if L > 0)
    used = []
    merged = {(m[0], m[3], m[2]): m for m in merges}
    for key, rs in ranges.items():
        rs.sort()
        seg_len = length[key[0]]
        assert rs[0][0] == 0 and rs[-1][1] == -(-seg_len // 64)
        assert all(a[1] == b[0] for a, b in zip(rs, rs[1:])), rs  # contiguous, no overlap
        if len(rs) == 1:
            assert rs[0][2] == 0 and key not in merged
            continue
        m = merged[key]
        assert m[1] == seg_len and m[5] == len(rs)
        assert [r[2] - 1 for r in rs] == list(range(m[4], m[4] + m[5]))  # slots in key order
        used += [r[2] - 1 for r in rs]
    assert sorted(used) == list(range(parts))
    assert len(merges) == sum(1 for rs in ranges.values() if len(rs) > 1)


EDGE = [1, 63, 64, 65, 127, 128, 129, 0, 255, 256, 257, 700, 3000]


@pytest.mark.parametrize("policy", [AUTO, NEVER, ALWAYS])
@pytest.mark.parametrize("heads,lens", [(2, EDGE), (6, [3000, 700, 257]), (3, [16200, 600, 623]),
                                        (1, [0, 0, 5]), (24, [4096, 1024])])
def test_split_plan_covers_every_key_once(tool, policy, heads, lens):
    items, merges, parts = plan(tool, policy, heads, lens)
    check_plan(items, merges, parts, heads, lens)
    if policy == NEVER:
        assert not merges and parts == 0


def test_always_cuts_every_item_of_four_tiles_or_more(tool):
    items, merges, _ = plan(tool, ALWAYS, 2, EDGE)
    long_ = {L for L in EDGE if -(-L // 64) >= 4}
    assert {m[1] for m in merges} == long_
    # 700 keys = 11 tiles: ranges [0, 4), [4, 8), [8, 11); 3000 keys = 47 tiles: 16, 16, 15
    r700 = sorted({(i[5], i[6]) for i in items if i[1] == 700})
    assert r700 == [(0, 4), (4, 8), (8, 11)]
    r3000 = sorted({(i[5], i[6]) for i in items if i[1] == 3000})
    assert r3000 == [(0, 16), (16, 32), (32, 47)]


def segs(name):
    return [s[3] for s in configs.ALL[name].segments]


def test_auto_policy_choices(tool):
    """Splits where a few long items would leave most slots idle (one GPU's
    3-head share of the S = 20,423 packing: 486 items for 512 slots, the
    16,200-token segment's items 254 tiles long), and nowhere the items already
    fill the slots (24 heads; two_seg, where the merge would cost more than the
    ragged end of the last round; ragged64)."""
    for h, lens, split in [(3, segs("h3_s20423_bf16"), True), (24, segs("h3_s20423_bf16"), False),
                           (24, segs("two_seg_bf16"), False), (24, segs("ragged64_bf16"), False)]:
        items, merges, parts = plan(tool, AUTO, h, lens)
        check_plan(items, merges, parts, h, lens)
        assert bool(merges) == split, (h, len(lens), len(merges))
        if split:  # only the long segment's items are cut
            assert {m[1] for m in merges} == {16200}


def test_split_partial_slots_are_capped(tool):
    """A forced split that would need more than 16,384 partial slots stays unsplit."""
    items, merges, parts = plan(tool, ALWAYS, 64, [16384] * 3)  # 3 x 128 x 64 items x 3 ranges
    assert not merges and parts == 0
    check_plan(items, merges, parts, 64, [16384] * 3)
    items, merges, parts = plan(tool, ALWAYS, 8, [16384] * 3)  # 3,072 items x 3 ranges = 9,216
    assert parts == 9216 and len(merges) == 3072
