"""Pins for the fp64 oracle: checks against closed forms, brute force, library
routines and invariants, none of which reuses the oracle's own formulas.

Every check takes the oracle's namespace ``O`` as an argument so that
tests/test_oracle_mutations.py can run the same checks against oracles with a
planted mistake and show that each mistake is caught.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# packing and positions
# ---------------------------------------------------------------------------

def check_positions_enumeration(O):
    """Nested loops over (t, h, w), w fastest, truncated to L; restart per segment."""
    segs = [(2, 3, 4, 24), (1, 7, 13, 91), (3, 2, 5, 17), (4, 1, 1, 0), (623, 1, 1, 9), (1, 1, 1, 1)]
    expect = []
    for (T, H, W, L) in segs:
        seg = []
        for t in range(T):
            for h in range(H):
                for w in range(W):
                    seg.append((t, h, w))
        expect.extend(seg[:L])
    got = O.segment_positions(segs)
    assert got.shape == (len(expect), 3)
    assert np.array_equal(got, np.array(expect, dtype=np.int64).reshape(-1, 3))
    running, cu = 0, [0]
    for s in segs:
        running += s[3]
        cu.append(running)
    assert np.array_equal(O.cu_seqlens(segs), np.array(cu))


# ---------------------------------------------------------------------------
# rotary angles
# ---------------------------------------------------------------------------

def check_inverse_frequencies_closed_form(O):
    g = golden()["inverse_frequencies"]
    f = O.axis_inverse_frequencies(g[0]["d_axis"], g[0]["base"])
    assert f.shape == (16,)
    for j, val in g[0]["checks"].items():
        assert abs(f[int(j)] - val) <= 1e-15 * max(1.0, val), (j, f[int(j)], val)
    ratio = f[1:] / f[:-1]
    assert np.allclose(ratio, 10000.0 ** (-1.0 / 16.0), rtol=1e-14, atol=0)
    f4 = O.axis_inverse_frequencies(g[1]["d_axis"], g[1]["base"])
    assert np.allclose(f4, g[1]["values"], rtol=1e-15, atol=0)


def check_angle_layout(O):
    """A unit step along one axis fills exactly that axis's block with its frequencies."""
    dims = (32, 32, 32)
    fr = [10000.0 ** (-2.0 * j / 32.0) for j in range(16)]
    for axis in range(3):
        p = np.zeros((1, 3), dtype=np.int64)
        p[0, axis] = 1
        th = O.rope_angles(p, dims, 10000.0)
        assert th.shape == (1, 48)
        want = np.zeros(48)
        want[16 * axis:16 * axis + 16] = fr
        assert np.allclose(th[0], want, rtol=1e-14, atol=0), axis
    # unequal split: blocks of 8, 4, 12 frequencies
    th = O.rope_angles(np.array([[2, 3, 5]]), (16, 8, 24), 100.0)
    want = np.concatenate([2 * 100.0 ** (-2.0 * np.arange(8) / 16), 3 * 100.0 ** (-2.0 * np.arange(4) / 8),
                           5 * 100.0 ** (-2.0 * np.arange(12) / 24)])
    assert np.allclose(th[0], want, rtol=1e-14, atol=0)


# ---------------------------------------------------------------------------
# other rotary table modes
# ---------------------------------------------------------------------------

def check_linspace_matches_numpy(O):
    """Positions along each axis are numpy.linspace(start, stop, n, endpoint=False), bit for bit."""
    segs = [(3, 2, 5, 30), (7, 1, 16, 100), (1, 9, 1, 9), (5, 3, 3, 44)]
    start, stop = (0.25, -1.0, 0.0), (3.0, 1.0, 1.0 / 3.0)
    p = O.linspace_positions(segs, start, stop)
    cu = O.cu_seqlens(segs)
    for s, (T, H, W, L) in enumerate(segs):
        rows = p[cu[s]:cu[s + 1]]
        ext = (T, H, W)
        n = np.arange(L)
        idx = (n // (H * W), (n // W) % H, n % W)
        for a in range(3):
            ref = np.linspace(start[a], stop[a], ext[a], endpoint=False)
            assert np.array_equal(rows[:, a], ref[idx[a]]), (s, a)


def check_linspace_reduces_to_grid(O):
    """start 0 and stop = the extent give the integer grid: the same table bit for bit."""
    seg = [(4, 6, 10, 200)]
    dims = (32, 32, 32)
    _, c0, s0 = O.rope_table(seg, dims, 10000.0)
    _, c1, s1 = O.rope_table_mode(seg, O.ROPE_LINSPACE, dims, 10000.0, start=(0, 0, 0), stop=(4, 6, 10))
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    # and a shifted, stretched grid is that affine map of the integers
    p = O.linspace_positions(seg, (1.0, 2.0, -3.0), (9.0, 14.0, 17.0))
    ip = O.segment_positions(seg)
    assert np.allclose(p, ip * np.array([2.0, 2.0, 2.0]) + np.array([1.0, 2.0, -3.0]), rtol=0, atol=1e-13)


def check_normalized_golden(O):
    case = golden()["rope_normalized"][0]
    _, c, s = O.rope_table_mode([case["segment"]], O.ROPE_NORMALIZED, case["rot_dims"], case["base"])
    assert np.allclose(c, case["cos"], rtol=0, atol=1e-15), c
    assert np.allclose(s, case["sin"], rtol=0, atol=1e-15), s


def check_normalized_invariants(O):
    """Ids lie in [-1, 1), mirror about the grid centre, and an extent-1 axis is the identity."""
    segs = [(3, 8, 5, 120), (1, 1, 1, 1), (2, 16, 9, 288 + 5)]
    p, inside = O.normalized_positions(segs)
    assert np.all(p[inside] >= -1.0) and np.all(p[inside] < 1.0)
    cu = O.cu_seqlens(segs)
    for s, (T, H, W, L) in enumerate(segs):
        rows = p[cu[s]:cu[s] + T * H * W].reshape(T, H, W, 3)
        assert np.allclose(rows[::-1, :, :, 0], -rows[:, :, :, 0], rtol=0, atol=1e-15)
        assert np.allclose(rows[:, ::-1, :, 1], -rows[:, :, :, 1], rtol=0, atol=1e-15)
        assert np.allclose(rows[:, :, ::-1, 2], -rows[:, :, :, 2], rtol=0, atol=1e-15)
    dims = (16, 16, 16)
    _, c, sn = O.rope_table_mode(segs, O.ROPE_NORMALIZED, dims, 100.0)
    assert np.all(c[120] == 1.0) and np.all(sn[120] == 0.0)  # the 1x1x1 segment
    # suffix tokens: identity; grid tokens as without the suffix
    _, c2, s2 = O.rope_table_mode([(2, 16, 9, 288)], O.ROPE_NORMALIZED, dims, 100.0)
    assert np.array_equal(c[121:121 + 288], c2) and np.array_equal(sn[121:121 + 288], s2)
    assert np.all(c[121 + 288:] == 1.0) and np.all(sn[121 + 288:] == 0.0)
    # four evenly spaced ids: -3/4, -1/4, 1/4, 3/4
    p4, _ = O.normalized_positions([(1, 1, 4, 4)])
    assert np.array_equal(p4[:, 2], [-0.75, -0.25, 0.25, 0.75])


def check_interleaved_golden(O):
    g = golden()["rope_interleaved"]
    case = g[0]
    _, c, s = O.rope_table_mode([case["segment"]], O.ROPE_INTERLEAVED, case["rot_dims"], case["base"])
    th = np.array(case["angles"])
    assert np.allclose(c[case["token"]], np.cos(th), rtol=0, atol=1e-15)
    assert np.allclose(s[case["token"]], np.sin(th), rtol=0, atol=1e-15)
    assert np.array_equal(O.interleaved_axes(g[1]["rot_dims"]), g[1]["axes"])


def check_interleaved_layout(O):
    """A unit step along one axis moves exactly that axis's interleaved slots, and
    equal coordinates on all three axes give plain 1-D rotary over R."""
    R, base = 96, 10000.0
    dims = (32, 32, 32)
    ladder = [base ** (-2.0 * j / R) for j in range(48)]
    segs = [(2, 2, 2, 8)]
    _, c, s = O.rope_table_mode(segs, O.ROPE_INTERLEAVED, dims, base)
    th = np.arctan2(s, c)
    for axis, token in ((0, 4), (1, 2), (2, 1)):  # (1,0,0), (0,1,0), (0,0,1)
        want = np.zeros(48)
        want[axis::3] = ladder[axis::3]
        assert np.allclose(th[token], want, rtol=1e-14, atol=0), axis
    assert np.allclose(th[7], ladder, rtol=1e-14, atol=0)  # (1, 1, 1)
    # shares that cannot be interleaved are rejected
    try:
        O.rope_table_mode(segs, O.ROPE_INTERLEAVED, (4, 8, 4), base)
    except ValueError:
        pass
    else:
        raise AssertionError("shares (4, 8, 4) accepted")


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------

def check_rms_norm_golden(O):
    for case in golden()["rms_norm"]:
        y = O.rms_norm(np.array([case["x"]]), np.array(case["gamma"]), case["eps"])
        assert np.allclose(y[0], case["y"], rtol=1e-15, atol=1e-15), (y, case["y"])


def check_rms_norm_invariants(O):
    r = _rng(1)
    x = r.normal(size=(50, 3, 64))
    g1 = np.ones(64)
    # scale invariance with eps = 0
    assert np.allclose(O.rms_norm(7.25 * x, g1, 0.0), O.rms_norm(x, g1, 0.0), rtol=1e-14, atol=1e-14)
    # with unit gain the output's mean square is ms / (ms + eps)
    eps = 0.37
    y = O.rms_norm(x, g1, eps)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-13, atol=0)
    # the gain multiplies each dim
    g = r.normal(size=64)
    assert np.allclose(O.rms_norm(x, g, eps), O.rms_norm(x, g1, eps) * g, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# rotary
# ---------------------------------------------------------------------------

def _rotation_matrix(theta, rot_dim, head_dim):
    """Independent dense formulation: a block rotation acting on pairs (i, i + R/2)."""
    half = rot_dim // 2
    M = np.eye(head_dim)
    for i in range(half):
        c, s = math.cos(theta[i]), math.sin(theta[i])
        M[i, i] = c
        M[i, i + half] = -s
        M[i + half, i] = s
        M[i + half, i + half] = c
    return M


def check_rope_golden(O):
    case = golden()["rope"][0]
    pos = np.array([case["position"]], dtype=np.int64)
    th = O.rope_angles(pos, case["rot_dims"], case["base"])
    R = sum(case["rot_dims"])
    for c in case["cases"]:
        x = np.zeros((1, 1, case["head_dim"]))
        x[0, 0, c["x_index"]] = 1.0
        y = O.rope_rotate(x, np.cos(th), np.sin(th), R)
        assert np.allclose(y[0, 0], c["y"], rtol=0, atol=1e-15), (c, y)


def check_rope_matches_rotation_matrix(O):
    r = _rng(2)
    for (dims, D) in (((32, 32, 32), 128), ((16, 16, 16), 64), ((8, 4, 12), 32)):
        R = sum(dims)
        pos = r.integers(0, 60, size=(9, 3))
        th = O.rope_angles(pos, dims, 10000.0)
        x = r.normal(size=(9, 2, D))
        y = O.rope_rotate(x, np.cos(th), np.sin(th), R)
        for n in range(9):
            M = _rotation_matrix(th[n], R, D)
            for h in range(2):
                assert np.allclose(y[n, h], M @ x[n, h], rtol=0, atol=1e-13)


def check_rope_identity_and_norm(O):
    r = _rng(3)
    dims = (32, 32, 32)
    _, cos, sin = O.rope_table([(1, 1, 1, 1)], dims, 10000.0)
    x = r.normal(size=(1, 4, 128))
    assert np.array_equal(O.rope_rotate(x, cos, sin, 96), x)  # (0, 0, 0) is the identity
    segs = [(3, 5, 7, 100), (623, 1, 1, 623)]
    _, cos, sin = O.rope_table(segs, dims, 10000.0)
    x = r.normal(size=(723, 2, 128))
    y = O.rope_rotate(x, cos, sin, 96)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14, atol=0)
    pair_x = x[..., :48] ** 2 + x[..., 48:96] ** 2
    pair_y = y[..., :48] ** 2 + y[..., 48:96] ** 2
    assert np.allclose(pair_y, pair_x, rtol=1e-13, atol=1e-15)
    assert np.array_equal(y[..., 96:], x[..., 96:])


def check_rope_single_axis(O):
    """With h = w = 0 only the t block's pairs move."""
    r = _rng(4)
    pos = np.array([[5, 0, 0], [17, 0, 0]])
    th = O.rope_angles(pos, (32, 32, 32), 10000.0)
    x = r.normal(size=(2, 1, 128))
    y = O.rope_rotate(x, np.cos(th), np.sin(th), 96)
    moved = np.nonzero(np.any(np.abs(y - x) > 0, axis=(0, 1)))[0]
    assert set(moved.tolist()) == set(range(0, 16)) | set(range(48, 64))


def check_rope_relative_position(O):
    """<R(p) a, R(p') b> = <a, R(p' - p) b> for integer position vectors."""
    r = _rng(5)
    dims = (32, 32, 32)
    p = r.integers(0, 40, size=(20, 3))
    p2 = p + r.integers(0, 40, size=(20, 3))
    a = r.normal(size=(20, 1, 128))
    b = r.normal(size=(20, 1, 128))

    def rot(x, pos):
        th = O.rope_angles(pos, dims, 10000.0)
        return O.rope_rotate(x, np.cos(th), np.sin(th), 96)

    lhs = np.sum(rot(a, p) * rot(b, p2), axis=-1)
    rhs = np.sum(a * rot(b, p2 - p), axis=-1)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def check_attention_golden(O):
    for case in golden()["attention"]:
        q = np.array(case["q"])[:, None, :]
        k = np.array(case["k"])[:, None, :]
        v = np.array(case["v"])[:, None, :]
        o = O.varlen_attention(q, k, v, np.array(case["cu_seqlens"]), case["scale"])
        assert np.allclose(o[:, 0], case["o"], rtol=0, atol=1e-14), (o[:, 0], case["o"])


def _dense_masked(q, k, v, cu, scale):
    """Independent formulation: one S x S score matrix with -inf off the block diagonal."""
    from scipy.special import softmax

    S, H, _ = q.shape
    seg = np.zeros(S, dtype=np.int64)
    for s in range(len(cu) - 1):
        seg[cu[s]:cu[s + 1]] = s
    mask = seg[:, None] == seg[None, :]
    out = np.zeros((S, H, v.shape[2]))
    for h in range(H):
        sc = scale * np.einsum("id,jd->ij", q[:, h], k[:, h])
        sc = np.where(mask, sc, -np.inf)
        out[:, h] = softmax(sc, axis=1) @ v[:, h]
    return out


def check_attention_dense_bruteforce(O):
    r = _rng(6)
    lens = [37, 0, 91, 1, 64, 65, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S = int(cu[-1])
    q, k, v = (r.normal(size=(S, 3, 16)) * 2 for _ in range(3))
    o = O.varlen_attention(q, k, v, cu, 0.25)
    ref = _dense_masked(q, k, v, cu, 0.25)
    assert np.allclose(o, ref, rtol=1e-13, atol=1e-14)


def check_attention_sdpa(O):
    """One segment without norm or rotary equals torch's scaled_dot_product_attention (fp64, CPU)."""
    import torch

    r = _rng(7)
    L, H, D = 77, 4, 32
    q, k, v = (r.normal(size=(L, H, D)) for _ in range(3))
    o = O.varlen_attention(q, k, v, np.array([0, L]), 1.0 / math.sqrt(D))
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2))) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).numpy().transpose(1, 0, 2)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)


def check_attention_special_cases(O):
    r = _rng(8)
    # length-1 segments return their value rows exactly
    q, k, v = (r.normal(size=(5, 2, 8)) for _ in range(3))
    o = O.varlen_attention(q, k, v, np.arange(6), 0.5)
    assert np.array_equal(o, v)
    # identical keys give the mean value over the segment
    L = 40
    q = r.normal(size=(L, 1, 8))
    k = np.repeat(r.normal(size=(1, 1, 8)), L, axis=0)
    v = r.normal(size=(L, 1, 8))
    o = O.varlen_attention(q, k, v, np.array([0, L]), 0.9)
    assert np.allclose(o[:, 0], np.broadcast_to(v[:, 0].mean(axis=0), (L, 8)), rtol=0, atol=1e-14)
    # softmax rows sum to 1 and are non-negative
    lens = [30, 50]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k = (r.normal(size=(80, 2, 8)) * 3 for _ in range(2))
    for seg in range(2):
        for h in range(2):
            P = O.attention_weights(q, k, cu, 0.7, seg, h)
            assert P.shape == (lens[seg], lens[seg])
            assert np.all(P >= 0)
            assert np.allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def check_attention_segment_isolation(O):
    """Perturbing a token of one segment leaves every output of the others bit-identical."""
    r = _rng(9)
    lens = [40, 33, 27]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = (r.normal(size=(100, 2, 16)) for _ in range(3))
    o = O.varlen_attention(q, k, v, cu, 0.3)
    for x in (q, k, v):
        x2 = x.copy()
        x2[50] += 1.5  # a token of segment 1
        args = [x2 if y is x else y for y in (q, k, v)]
        o2 = O.varlen_attention(*args, cu, 0.3)
        assert np.array_equal(o2[:40], o[:40]) and np.array_equal(o2[73:], o[73:])
        assert not np.array_equal(o2[40:73], o[40:73])


def check_attention_permutations(O):
    r = _rng(10)
    lens = [21, 34, 13]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S = int(cu[-1])
    q, k, v = (r.normal(size=(S, 2, 8)) for _ in range(3))
    o = O.varlen_attention(q, k, v, cu, 0.6)
    # keys/values permuted inside each segment: outputs unchanged
    perm = np.concatenate([cu[s] + r.permutation(lens[s]) for s in range(3)])
    o2 = O.varlen_attention(q, k[perm], v[perm], cu, 0.6)
    assert np.allclose(o2, o, rtol=1e-13, atol=1e-14)
    # queries permuted inside each segment: outputs permute the same way
    o3 = O.varlen_attention(q[perm], k, v, cu, 0.6)
    assert np.allclose(o3, o[perm], rtol=1e-13, atol=1e-14)
    # segment order permuted: per-segment outputs move with their segments
    order = [2, 0, 1]
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in order])
    cu2 = np.concatenate([[0], np.cumsum([lens[s] for s in order])])
    o4 = O.varlen_attention(q[idx], k[idx], v[idx], cu2, 0.6)
    assert np.allclose(o4, o[idx], rtol=1e-13, atol=1e-14)


def check_attention_rows_variant(O):
    r = _rng(11)
    lens = [70, 1, 45]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = (r.normal(size=(116, 3, 16)) for _ in range(3))
    o = O.varlen_attention(q, k, v, cu, 0.25)
    rows = np.array([0, 69, 70, 71, 100, 115, 3])
    assert np.allclose(O.varlen_attention_rows(q, k, v, cu, 0.25, rows), o[rows], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# causal and grouped-query attention
# ---------------------------------------------------------------------------

def check_causal_gqa_bruteforce(O):
    """Scalar loops: query i of a segment sees keys 0..i; K/V head g serves the
    query heads g * group .. g * group + group - 1."""
    r = _rng(14)
    lens = [9, 0, 1, 14, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S, Hkv, group, D = int(cu[-1]), 2, 3, 5
    q = r.normal(size=(S, Hkv * group, D))
    k = r.normal(size=(S, Hkv, D))
    v = r.normal(size=(S, Hkv, 4))
    scale = 0.45
    for causal in (True, False):
        o = O.varlen_attention_gqa(q, k, v, cu, scale, causal=causal)
        ref = np.zeros((S, Hkv * group, 4))
        for sgi in range(len(lens)):
            a, b = int(cu[sgi]), int(cu[sgi + 1])
            for g in range(Hkv):
                for member in range(group):
                    h = g * group + member
                    for i in range(a, b):
                        last = i if causal else b - 1
                        num, den = np.zeros(4), 0.0
                        for j in range(a, last + 1):
                            w = math.exp(scale * sum(q[i, h, d] * k[j, g, d] for d in range(D)))
                            num += w * v[j, g]
                            den += w
                        ref[i, h] = num / den
        assert np.allclose(o, ref, rtol=1e-12, atol=1e-13), causal


def check_causal_prefix_properties(O):
    r = _rng(15)
    lens = [33, 20]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = (r.normal(size=(53, 4, 8)) for _ in range(3))
    o = O.varlen_attention_gqa(q, k, v, cu, 0.7, causal=True)
    # the first query of a segment sees only its own key
    assert np.array_equal(o[0], v[0]) and np.array_equal(o[33], v[33])
    # a change at token 40 leaves every earlier row (and the other segment) bit-identical
    for x in (q, k, v):
        x2 = x.copy()
        x2[40] += 2.0
        args = [x2 if y is x else y for y in (q, k, v)]
        o2 = O.varlen_attention_gqa(*args, cu, 0.7, causal=True)
        assert np.array_equal(o2[:40], o[:40])
        assert not np.array_equal(o2[40:53], o[40:53])
    # the last query of a segment sees the whole segment: the bidirectional result
    ob = O.varlen_attention_gqa(q, k, v, cu, 0.7, causal=False)
    assert np.allclose(o[[32, 52]], ob[[32, 52]], rtol=1e-14, atol=1e-15)


def check_gqa_is_repeated_kv(O):
    """Grouped K/V heads equal plain multi-head attention on K/V repeated per group."""
    r = _rng(16)
    lens = [25, 40, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = r.normal(size=(66, 8, 16))
    k, v = (r.normal(size=(66, 2, 16)) for _ in range(2))
    o = O.varlen_attention_gqa(q, k, v, cu, 0.25)
    ref = O.varlen_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), cu, 0.25)
    assert np.allclose(o, ref, rtol=1e-13, atol=1e-14)
    # one K/V head per query head is the plain function
    k8, v8 = (r.normal(size=(66, 8, 16)) for _ in range(2))
    assert np.allclose(O.varlen_attention_gqa(q, k8, v8, cu, 0.25), O.varlen_attention(q, k8, v8, cu, 0.25),
                       rtol=1e-14, atol=1e-15)


def check_causal_gqa_sdpa(O):
    """One segment: torch's scaled_dot_product_attention(is_causal, enable_gqa) in fp64 on the CPU."""
    import torch

    r = _rng(17)
    L, Hq, Hkv, D = 70, 6, 2, 32
    q = r.normal(size=(L, Hq, D))
    k, v = (r.normal(size=(L, Hkv, D)) for _ in range(2))
    o = O.varlen_attention_gqa(q, k, v, np.array([0, L]), 1.0 / math.sqrt(D), causal=True)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2))) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)
    assert np.allclose(o, ref.numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-13)


def check_gqa_rows_variant(O):
    r = _rng(18)
    lens = [50, 1, 37]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = r.normal(size=(88, 4, 8))
    k, v = (r.normal(size=(88, 1, 8)) for _ in range(2))
    rows = np.array([0, 1, 49, 50, 51, 87, 60])
    for causal in (False, True):
        full = O.varlen_attention_gqa(q, k, v, cu, 0.3, causal=causal)
        part = O.varlen_attention_gqa_rows(q, k, v, cu, 0.3, rows, causal=causal)
        assert np.allclose(part, full[rows], rtol=1e-14, atol=1e-15), causal


# ---------------------------------------------------------------------------
# FP8 E4M3 codec and the low-precision attention
# ---------------------------------------------------------------------------

def check_e4m3_decode_table(O):
    g = golden()["e4m3"]
    for code, val in g["decode"].items():
        got = O.e4m3_decode(np.array([int(code)], dtype=np.uint8))[0]
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)
    for code in g["nan_codes"]:
        assert np.isnan(O.e4m3_decode(np.array([code], dtype=np.uint8))[0])
    v = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0) and v[-1] == 448.0  # 127 increasing non-negative values
    assert np.array_equal(O.e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8)), -v)


def check_e4m3_encode(O):
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = O.e4m3_decode(finite)
    assert np.array_equal(O.e4m3_encode(vals), finite)  # every finite code round-trips
    # midpoints between neighbours go to the even mantissa; just off the midpoint, to the nearer
    pos = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for i in range(len(pos) - 1):
        lo, hi = pos[i], pos[i + 1]
        mid = 0.5 * (lo + hi)
        want = i if i % 2 == 0 else i + 1
        assert O.e4m3_encode(np.array([mid]))[0] == want, (i, mid)
        assert O.e4m3_encode(np.array([mid - (hi - lo) * 1e-3]))[0] == i
        assert O.e4m3_encode(np.array([mid + (hi - lo) * 1e-3]))[0] == i + 1
        assert O.e4m3_encode(np.array([-mid]))[0] == 0x80 | want
    # saturation and flush
    assert list(O.e4m3_encode(np.array([460.0, 1e6, -1e9, 2.0 ** -10, -(2.0 ** -11)]))) == [0x7E, 0x7E, 0xFE, 0, 0x80]


def check_e4m3_matches_torch(O):
    """torch's float8_e4m3fn conversion (round to nearest even) on random in-range values."""
    import torch

    r = _rng(19)
    x = r.normal(size=50000) * np.exp2(r.uniform(-12, 9, size=50000))
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), ref)


def check_bf16_round(O):
    """Against torch's bfloat16 conversion of fp32 values (one rounding), hand-derived ties
    (1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to 1; 1 + 3 * 2^-8 ties to 1 + 2^-6),
    and representable values unchanged."""
    import torch

    r = _rng(21)
    x = (r.normal(size=20000) * np.exp2(r.uniform(-20, 20, size=20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_round(x.astype(np.float64)), ref)
    t = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3.0, 1 + 2.0 ** -7])
    assert np.array_equal(O.bf16_round(t), [1.0, 1 + 2.0 ** -6, -1.0, 3.0, 1 + 2.0 ** -7])


def check_fp8qk_attention(O):
    """E4M3-representable q, k pass through unchanged; otherwise the score product sees the
    rounded operands; the rounding error on normalised inputs stays small."""
    r = _rng(20)
    lens = [40, 1, 77]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S = int(cu[-1])
    q8 = O.e4m3_decode(r.integers(0, 0x7F, size=(S, 4, 16)).astype(np.uint8)) * r.choice([-1, 1], size=(S, 4, 16))
    k8 = O.e4m3_decode(r.integers(0, 0x70, size=(S, 2, 16)).astype(np.uint8))
    v = r.normal(size=(S, 2, 16))
    for causal in (False, True):
        assert np.array_equal(O.varlen_attention_fp8qk(q8, k8, v, cu, 0.05, causal),
                              O.varlen_attention_gqa(q8, k8, v, cu, 0.05, causal))
    q, k = r.normal(size=(S, 4, 16)), r.normal(size=(S, 2, 16))
    a = O.varlen_attention_fp8qk(q, k, v, cu, 0.25)
    b = O.varlen_attention_gqa(q, k, v, cu, 0.25)
    rel = np.abs(a - b).sum() / np.abs(b).sum()
    assert 0 < rel < 0.05, rel
    # and rounding only one operand is not the same thing
    assert not np.allclose(a, O.varlen_attention_gqa(O.e4m3_round(q), k, v, cu, 0.25), rtol=0, atol=1e-9)
    # all three operands: representable values pass through; v's rounding is applied too
    v8 = O.e4m3_decode(r.integers(0, 0x7F, size=(S, 2, 16)).astype(np.uint8))
    assert np.array_equal(O.varlen_attention_fp8(q8, k8, v8, cu, 0.05, True),
                          O.varlen_attention_gqa(q8, k8, v8, cu, 0.05, True))
    a3 = O.varlen_attention_fp8(q, k, v, cu, 0.25)
    assert np.allclose(a3, O.varlen_attention_gqa(O.e4m3_round(q), O.e4m3_round(k), O.e4m3_round(v), cu, 0.25),
                       rtol=0, atol=0)
    assert not np.allclose(a3, a, rtol=0, atol=1e-6)


def check_mx_block_exponent(O):
    """Hand-derived scale exponents, and on 5,000 magnitudes over 2^-110..2^110: the scaled
    maximum never exceeds 448 and doubling it would (the exponent is the smallest one)."""
    g = golden()["mx"]
    for a, X in g["exponent"].items():
        assert int(O.mx_block_exponent(float(a))) == X, (a, X)
    for e, X in g["exponent_pow2"].items():
        assert int(O.mx_block_exponent(2.0 ** int(e))) == X, (e, X)
    r = _rng(31)
    a = r.uniform(1, 2, 5000) * 2.0 ** r.integers(-110, 110, 5000).astype(np.float64)
    scaled = a * 2.0 ** -O.mx_block_exponent(a).astype(np.float64)
    assert np.all(scaled <= 448.0) and np.all(2.0 * scaled > 448.0)


def check_mx_quantize(O):
    """Hand-derived blocks; representable blocks pass through; exact equivariance under powers
    of two; the E4M3 error bound relative to each block's scale; independent blocks; blocks that
    need no scaling give the plain codec's codes."""
    g = golden()["mx"]
    ga, gb = g["block_a"], g["block_b"]
    x = np.zeros(64)
    x[: len(ga["x"])] = ga["x"]
    x[32: 32 + len(gb["x"])] = gb["x"]
    codes, X = O.mx_quantize(x)
    assert list(X) == [ga["X"], gb["X"]]
    assert list(codes[: len(ga["codes"])]) == ga["codes"] and list(codes[32: 32 + len(gb["codes"])]) == gb["codes"]
    vals = O.mx_dequantize(codes, X)
    assert np.array_equal(vals[: len(ga["values"])], ga["values"])
    assert np.array_equal(vals[32: 32 + len(gb["values"])], gb["values"])

    def rnd(v, axis=-1):
        return O.mx_dequantize(*O.mx_quantize(v, axis), axis=axis)

    assert np.array_equal(O.mx_round(x), rnd(x))
    r = _rng(32)
    # representable: random codes whose block max code lies in [224, 448], times 2^X
    codes = r.integers(0, 0x7F, size=(40, 64)).astype(np.uint8)
    codes[:, ::32] = r.integers(0x70, 0x7F, size=(40, 2))
    Xs = r.integers(-60, 60, size=(40, 2))
    x = (O.e4m3_decode(codes).reshape(40, 2, 32) * 2.0 ** Xs[..., None]).reshape(40, 64)
    x *= r.choice([-1.0, 1.0], size=x.shape)
    assert np.array_equal(rnd(x), x)
    # equivariance and error bound on wide-range data
    y = r.normal(size=(50, 128)) * 2.0 ** r.integers(-30, 30, size=(50, 1)).astype(np.float64)
    y[3, 40:60] = 0.0
    for k in (-9, 5, 17):
        assert np.array_equal(rnd(y * 2.0 ** k), rnd(y) * 2.0 ** k)
    c, X = O.mx_quantize(y)
    scale = np.repeat(2.0 ** X.astype(np.float64), 32, axis=-1)
    err = np.abs(rnd(y) - y)
    normal = np.abs(y) >= scale * 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(y[normal]))
    assert np.all(err[~normal] <= scale[~normal] * 2.0 ** -10)
    # blocks are independent, and the block axis can be any axis
    y2 = y.copy()
    y2[:, 32:64] *= 1000.0
    c2, X2 = O.mx_quantize(y2)
    keep = np.r_[0:32, 64:128]
    assert np.array_equal(c2[:, keep], c[:, keep]) and np.array_equal(X2[:, [0, 2, 3]], X[:, [0, 2, 3]])
    assert np.array_equal(rnd(y.T, axis=0), rnd(y).T)
    # no scaling needed -> the plain E4M3 codec
    z = r.uniform(-448, 448, size=(10, 32))
    z[:, 0] = 400.0
    cz, Xz = O.mx_quantize(z)
    assert np.all(Xz == 0) and np.array_equal(cz, O.e4m3_encode(z))


def check_mx_keys_and_attention(O):
    """V blocks of 32 keys start at each segment's start (a segment rounds the same alone or
    packed, checked against a scalar loop); attention on representable operands is the exact
    attention; scaling v by a power of two scales the output exactly, which the unscaled E4M3
    path cannot do for v at 2^-12 or 2^10."""
    r = _rng(33)
    lens = [40, 0, 77, 1, 64]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S, D = int(cu[-1]), 32
    # segments 2^14 apart in magnitude: a block straddling two of them would flush the
    # smaller one's values (scaling commutes with E4M3 rounding only inside its range)
    mag = np.repeat(2.0 ** np.array([-12.0, 0.0, 12.0, 0.0, -6.0]), lens)
    v = r.normal(size=(S, 2, D)) * mag[:, None, None]
    rv = O.mx_round_keys(v, cu)
    assert np.all(np.abs(rv - v) <= 2.0 ** -4 * np.abs(v) + 2.0 ** -20 * np.abs(v).max(axis=0))
    for a, b in zip(cu[:-1], cu[1:]):
        if b > a:
            assert np.array_equal(rv[a:b], O.mx_round_keys(v[a:b], np.array([0, b - a])))
    # scalar loop for one head dim of the 77-key segment
    a0, h, d = int(cu[2]), 1, 5
    for blk in range(3):
        idx = [a0 + blk * 32 + i for i in range(32) if blk * 32 + i < 77]
        amax = max(abs(v[i, h, d]) for i in idx)
        X = int(O.mx_block_exponent(amax))
        for i in idx:
            want = O.e4m3_decode(O.e4m3_encode(np.array([v[i, h, d] * 2.0 ** -X])))[0] * 2.0 ** X
            assert rv[i, h, d] == want
    q, k = r.normal(size=(S, 4, D)), r.normal(size=(S, 2, D))
    qr, kr, vr = O.mx_round(q), O.mx_round(k), O.mx_round_keys(v, cu)
    for causal in (False, True):
        assert np.array_equal(O.varlen_attention_mx(qr, kr, vr, cu, 0.2, causal),
                              O.varlen_attention_gqa(qr, kr, vr, cu, 0.2, causal))
    assert np.array_equal(O.varlen_attention_mx_qk(q, k, v, cu, 0.2), O.varlen_attention_gqa(qr, kr, v, cu, 0.2))
    v1 = r.normal(size=(S, 2, D))
    base = O.varlen_attention_mx(q, k, v1, cu, 0.2)
    # a length-1 segment returns its own value as the block rounding of it stands
    i1 = int(cu[3])
    own = O.mx_round_keys(v1[i1:i1 + 1], np.array([0, 1]))[0]  # [Hkv, D]; query heads 2h, 2h+1 read K/V head h
    assert np.array_equal(base[i1], np.repeat(own, 2, axis=0))
    assert not np.array_equal(base[i1], np.repeat(v1[i1], 2, axis=0))
    exact = O.varlen_attention_gqa(q, k, v1, cu, 0.2)
    for e in (-12, 10):
        assert np.array_equal(O.varlen_attention_mx(q, k, v1 * 2.0 ** e, cu, 0.2), base * 2.0 ** e)
        unscaled = O.varlen_attention_fp8(q, k, v1 * 2.0 ** e, cu, 0.2) / 2.0 ** e
        assert np.abs(unscaled - exact).sum() > 4 * np.abs(base - exact).sum(), e


def check_i8_quantize(O):
    """Hand-derived rows (an fp32 product that ties at 127; integer ties to even); on
    wide-range random rows: codes within +-127, each row's largest magnitude at +-127,
    error at most half a step, the same codes for the row times any power of two;
    zero rows give zeros, a NaN or an infinity poisons only its own row's scale."""
    g = golden()["i8"]
    for row in (g["row_a"], g["row_b"]):
        c, sc = O.i8_quantize_rows(np.array(row["x"])[None, None, :])
        assert list(c[0, 0]) == row["codes"] and float(sc[0, 0]) == row["scale"], (row, c, sc)
    r = _rng(41)
    x = r.normal(size=(30, 3, 64)) * 2.0 ** r.integers(-20, 20, size=(30, 3, 1)).astype(np.float64)
    x = x.astype(np.float32).astype(np.float64)
    c, sc = O.i8_quantize_rows(x)
    assert c.dtype == np.int8 and sc.shape == (3, 30) and sc.dtype == np.float32
    assert np.all(np.abs(c.astype(np.int64)) <= 127)
    top = np.abs(x).argmax(axis=-1)
    assert np.all(np.abs(np.take_along_axis(c, top[..., None], -1)) == 127)
    step = sc.T.astype(np.float64)[..., None]
    err = np.abs(O.i8_dequantize_rows(c, sc) - x)
    assert np.all(err <= 0.5 * step * (1 + 1e-6) + 1e-6 * np.abs(x))
    for k in (-7, 3, 11):
        c2, sc2 = O.i8_quantize_rows(x * 2.0 ** k)
        assert np.array_equal(c2, c) and np.array_equal(sc2, (sc * np.float32(2.0 ** k)).astype(np.float32))
    y = x.copy()
    y[4, 1] = 0.0
    y[5, 2, 7] = np.nan
    y[6, 0, 3] = -np.inf
    cy, sy = O.i8_quantize_rows(y)
    assert np.all(cy[4, 1] == 0) and sy[1, 4] == 0
    assert np.isnan(sy[2, 5]) and np.all(cy[5, 2] == 0)
    assert np.isinf(sy[0, 6]) and np.all(cy[6, 0] == 0)
    keep = np.ones((30, 3), bool)
    keep[[4, 5, 6], [1, 2, 0]] = False
    assert np.array_equal(cy[keep], c[keep]) and np.array_equal(sy.T[keep], sc.T[keep])


def check_i8_key_blocks_and_attention(O):
    """Key blocks: hand-derived numbering; blocks of 64 keys start at each segment's start (a
    segment quantises the same alone as packed) and a scalar loop gives each block's scale;
    attention on operands already on their INT8 grids is the exact attention, and otherwise
    it is the exact attention of what the codes stand for, q and k both rounded."""
    g = golden()["i8"]["key_blocks"]
    cu = np.concatenate([[0], np.cumsum(g["lens"])])
    assert list(O.i8_key_blocks(cu)) == g["first"]
    r = _rng(42)
    lens = [65, 0, 130, 1, 64]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S = int(cu[-1])
    k = (r.normal(size=(S, 2, 32)) * np.repeat(2.0 ** np.array([-5.0, 0, 3.0, 0, 8.0]), lens)[:, None, None])
    k = k.astype(np.float32).astype(np.float64)
    c, sc = O.i8_quantize_key_blocks(k, cu)
    first = O.i8_key_blocks(cu)
    assert sc.shape == (2, int(first[-1]))
    for s, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        a, b = int(a), int(b)
        if b == a:
            continue
        cs, ss = O.i8_quantize_key_blocks(k[a:b], np.array([0, b - a]))
        assert np.array_equal(cs, c[a:b]) and np.array_equal(ss, sc[:, first[s]:first[s + 1]])
        for j, r0 in enumerate(range(a, b, 64)):
            rows = range(r0, min(r0 + 64, b))
            for h in range(2):
                amax = max(abs(float(k[i, h, d])) for i in rows for d in range(32))
                assert float(sc[h, first[s] + j]) == float(np.float32(amax) / np.float32(127))
                assert max(abs(int(c[i, h, d])) for i in rows for d in range(32)) == 127
    # operands on their grids pass through exactly
    q = r.integers(-127, 128, size=(S, 4, 32)).astype(np.float64)
    q[:, :, 0] = 127.0
    kk = r.integers(-127, 128, size=(S, 2, 32)).astype(np.float64)
    kk[:, :, 5] = -127.0
    v = r.normal(size=(S, 2, 32))
    for causal in (False, True):
        assert np.array_equal(O.varlen_attention_i8qk(q, kk, v, cu, 1e-3, causal),
                              O.varlen_attention_gqa(q, kk, v, cu, 1e-3, causal))
    qn, kn = r.normal(size=(S, 4, 32)), r.normal(size=(S, 2, 32))
    got = O.varlen_attention_i8qk(qn, kn, v, cu, 0.2)
    qd = O.i8_dequantize_rows(*O.i8_quantize_rows(qn))
    kd = O.i8_dequantize_key_blocks(*O.i8_quantize_key_blocks(kn, cu), cu)
    assert np.array_equal(got, O.varlen_attention_gqa(qd, kd, v, cu, 0.2))
    exact = O.varlen_attention_gqa(qn, kn, v, cu, 0.2)
    only_q = O.varlen_attention_gqa(qd, kn, v, cu, 0.2)
    assert not np.allclose(got, only_q, rtol=0, atol=1e-9) and not np.allclose(got, exact, rtol=0, atol=1e-6)
    assert np.abs(got - exact).sum() / np.abs(exact).sum() < 0.05


def check_i8_centered_keys(O):
    """Centred keys: segment means against a scalar loop (an empty segment's is 0; a segment
    alone gives the same means as packed); a hand-derived case (keys 1 and 3 of one dim centre
    to -1 and 1, codes -127 and 127, scale 1/127); the centred value is the fp32 difference;
    zero means give the plain codes; any per-segment constant subtracted from k leaves exact
    attention unchanged; with per-channel key offsets of 30 sigma the centred INT8 scores are
    far closer to exact attention than the plain ones."""
    r = _rng(44)
    lens = [70, 0, 5, 129]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S = int(cu[-1])
    k = r.normal(size=(S, 2, 16)) + 3.0 * r.normal(size=(1, 2, 16))
    mu = O.segment_key_means(k, cu)
    assert mu.shape == (4, 2, 16) and np.all(mu[1] == 0)
    for si, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        a, b = int(a), int(b)
        if b == a:
            continue
        for h in range(2):
            for d in range(16):
                tot = 0.0
                for i in range(a, b):
                    tot += float(k[i, h, d])
                assert abs(float(mu[si, h, d]) - tot / (b - a)) <= 1e-12 * max(1.0, abs(tot))
        assert np.array_equal(O.segment_key_means(k[a:b], np.array([0, b - a]))[0], mu[si])
    # hand-derived: one segment of two keys, one head, one dim
    kk = np.array([[[1.0]], [[3.0]]])
    c2 = np.array([0, 2])
    mu2 = O.segment_key_means(kk, c2).astype(np.float32)
    assert float(mu2[0, 0, 0]) == 2.0
    codes, sc = O.i8_quantize_key_blocks_centered(kk, c2, mu2)
    assert codes[:, 0, 0].tolist() == [-127, 127] and float(sc[0, 0]) == float(np.float32(1) / np.float32(127))
    # the centred value is the fp32 difference (here 1 - 2^-30 rounds to 1 in fp32)
    kf = np.array([[[1.0]]])
    tiny = np.array([[[2.0 ** -30]]], dtype=np.float32)
    assert float(O.i8_center_keys(kf, np.array([0, 1]), tiny)[0, 0, 0]) == 1.0
    z = np.zeros((4, 2, 16), dtype=np.float32)
    k32 = k.astype(np.float32).astype(np.float64)
    pc, ps = O.i8_quantize_key_blocks(k32, cu)
    zc, zs = O.i8_quantize_key_blocks_centered(k32, cu, z)
    assert np.array_equal(pc, zc) and np.array_equal(ps, zs)
    # exact attention does not see a per-segment constant subtracted from k
    q, v = r.normal(size=(S, 4, 16)), r.normal(size=(S, 2, 16))
    shift = np.concatenate([np.repeat(r.normal(size=(1, 2, 16)) * 5, L, axis=0) for L in lens])
    for causal in (False, True):
        assert np.allclose(O.varlen_attention_gqa(q, k - shift, v, cu, 0.3, causal),
                           O.varlen_attention_gqa(q, k, v, cu, 0.3, causal), rtol=0, atol=1e-12)
    # accuracy with per-channel offsets
    ko = r.normal(size=(S, 2, 16)) + 30.0 * r.normal(size=(1, 2, 16))
    exact = O.varlen_attention_gqa(q, ko, v, cu, 0.3)
    plain = O.varlen_attention_i8qk(q, ko, v, cu, 0.3)
    cent = O.varlen_attention_i8qk_centered(q, ko, v, cu, 0.3)
    err = lambda x: float(np.abs(x - exact).sum() / np.abs(exact).sum())  # noqa: E731
    assert err(cent) < 0.02 and err(cent) < 0.2 * err(plain), (err(cent), err(plain))
    m32 = O.segment_key_means(ko, cu).astype(np.float32)
    assert np.array_equal(cent, O.varlen_attention_i8qk_centered(q, ko, v, cu, 0.3, mu32=m32))


def check_i8qk_mxv_attention(O):
    """INT8 scores with E4M3 V: operands already on their grids (q, k integers with a 127 in
    every block, v on every segment's 32-key E4M3 block grid) pass through to the exact
    attention; v off its grid changes the result, by less than E4M3's half step allows; q and
    k off their grids change it too (both products rounded, not one)."""
    r = _rng(43)
    lens = [65, 0, 33, 1, 96]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S = int(cu[-1])
    q = r.integers(-127, 128, size=(S, 4, 32)).astype(np.float64)
    q[:, :, 0] = 127.0
    kk = r.integers(-127, 128, size=(S, 2, 32)).astype(np.float64)
    kk[:, :, 5] = -127.0
    # v on the grid: small integers times a power of two per segment are E4M3 values whose
    # block maxima map onto themselves
    v = r.integers(-15, 16, size=(S, 2, 32)).astype(np.float64) * np.repeat(2.0 ** np.array([-3.0, 0, 2.0, 0, 5.0]),
                                                                           lens)[:, None, None]
    assert np.array_equal(O.mx_round_keys(v, cu), v)
    for causal in (False, True):
        assert np.array_equal(O.varlen_attention_i8qk_mxv(q, kk, v, cu, 1e-3, causal),
                              O.varlen_attention_gqa(q, kk, v, cu, 1e-3, causal))
    vn = r.normal(size=(S, 2, 32))
    got = O.varlen_attention_i8qk_mxv(q, kk, vn, cu, 1e-3)
    exact = O.varlen_attention_gqa(q, kk, vn, cu, 1e-3)
    assert not np.allclose(got, exact, rtol=0, atol=1e-9)
    # each output is a convex combination of v rows, each moved by at most 2^-4 of its block max
    bound = np.zeros((S, 2, 32))
    for a, b in zip(cu[:-1], cu[1:]):
        a, b = int(a), int(b)
        for j in range(a, b, 32):
            blk = np.abs(vn[j:min(j + 32, b)]).max(axis=0)
            bound[j:min(j + 32, b)] = 2.0 ** -4 * blk
    for s_, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        a, b = int(a), int(b)
        if b > a:
            lim = bound[a:b].max(axis=0)  # [2, 32]
            assert np.all(np.abs(got[a:b] - exact[a:b]) <= np.repeat(lim, 2, axis=0)[None] + 1e-12)
    # tokens at magnitudes 2^0 .. 2^-23: a 32-key block's scale follows its largest token, so
    # the smaller tokens of the block lose precision (a per-token block would keep it)
    vm = vn * 2.0 ** -(np.arange(S) % 24)[:, None, None]
    qn, kn = r.normal(size=(S, 4, 32)), r.normal(size=(S, 2, 32))
    g2 = O.varlen_attention_i8qk_mxv(qn, kn, vm, cu, 0.2)
    assert np.array_equal(g2, O.varlen_attention_gqa(O.i8_round_q(qn), O.i8_round_k(kn, cu), O.mx_round_keys(vm, cu),
                                                     cu, 0.2))
    assert not np.allclose(g2, O.varlen_attention_gqa(qn, kn, O.mx_round_keys(vm, cu), cu, 0.2), rtol=0, atol=1e-9)


# ---------------------------------------------------------------------------
# the chain
# ---------------------------------------------------------------------------

def check_chain_shift_invariance(O):
    """Shifting all positions of a segment by a constant vector leaves its attention unchanged."""
    r = _rng(12)
    segs = [(2, 4, 5, 37)]
    D, dims = 64, (16, 16, 16)
    q, k, v = (r.normal(size=(37, 2, D)) for _ in range(3))
    g = 1 + 0.1 * r.normal(size=D)
    pos = O.segment_positions(segs)
    cu = O.cu_seqlens(segs)

    def run(p):
        th = O.rope_angles(p, dims, 10000.0)
        qn, kn = O.qk_rmsnorm_rope(q, k, g, g, 1e-6, np.cos(th), np.sin(th), 48)
        return O.varlen_attention(qn, kn, v, cu, 1 / 8)

    base = run(pos)
    shifted = run(pos + np.array([3, 11, 6]))
    assert np.allclose(shifted, base, rtol=1e-11, atol=1e-12)
    # and the rotation is not a no-op: without it the output differs
    qn, kn = O.rms_norm(q, g, 1e-6), O.rms_norm(k, g, 1e-6)
    assert not np.allclose(O.varlen_attention(qn, kn, v, cu, 1 / 8), base, rtol=1e-6, atol=1e-6)


def check_chain_composition(O):
    """hot_path is table -> norm + rotary -> attention, with nothing else in between."""
    r = _rng(13)
    segs = [(1, 37, 1, 37), (1, 7, 13, 91)]
    q, k, v = (r.normal(size=(128, 2, 64)) for _ in range(3))
    gq, gk = 1 + 0.1 * r.normal(size=64), 1 + 0.1 * r.normal(size=64)
    o = O.hot_path(q, k, v, gq, gk, segs, (16, 16, 16), 10000.0, 1e-6, 0.125)
    ms_q = np.mean(q * q, axis=-1, keepdims=True)
    ms_k = np.mean(k * k, axis=-1, keepdims=True)
    qn = q / np.sqrt(ms_q + 1e-6) * gq
    kn = k / np.sqrt(ms_k + 1e-6) * gk
    pos = O.segment_positions(segs)
    th = O.rope_angles(pos, (16, 16, 16), 10000.0)
    for n in range(128):
        M = _rotation_matrix(th[n], 48, 64)
        qn[n] = qn[n] @ M.T
        kn[n] = kn[n] @ M.T
    ref = _dense_masked(qn, kn, v, O.cu_seqlens(segs), 0.125)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)


ALL_CHECKS = [
    check_positions_enumeration,
    check_inverse_frequencies_closed_form,
    check_angle_layout,
    check_linspace_matches_numpy,
    check_linspace_reduces_to_grid,
    check_normalized_golden,
    check_normalized_invariants,
    check_interleaved_golden,
    check_interleaved_layout,
    check_rms_norm_golden,
    check_rms_norm_invariants,
    check_rope_golden,
    check_rope_matches_rotation_matrix,
    check_rope_identity_and_norm,
    check_rope_single_axis,
    check_rope_relative_position,
    check_attention_golden,
    check_attention_dense_bruteforce,
    check_attention_sdpa,
    check_attention_special_cases,
    check_attention_segment_isolation,
    check_attention_permutations,
    check_attention_rows_variant,
    check_causal_gqa_bruteforce,
    check_causal_prefix_properties,
    check_gqa_is_repeated_kv,
    check_causal_gqa_sdpa,
    check_gqa_rows_variant,
    check_e4m3_decode_table,
    check_e4m3_encode,
    check_e4m3_matches_torch,
    check_bf16_round,
    check_fp8qk_attention,
    check_mx_block_exponent,
    check_mx_quantize,
    check_mx_keys_and_attention,
    check_i8_quantize,
    check_i8_key_blocks_and_attention, check_i8qk_mxv_attention, check_i8_centered_keys,
    check_chain_shift_invariance,
    check_chain_composition,
]
