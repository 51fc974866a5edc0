"""fp64 CPU oracle for the packed varlen attention head -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The HIP library never calls it and shares no code with it.

What it computes, step by step, in float64 with numpy (matmul, exp, cos, sin,
sqrt are the only library primitives used):

1. Packing and positions.  Segments are (T, H, W) token grids truncated to L
   tokens, packed back to back; ``cu_seqlens`` is the prefix sum of the L.
   Token n of a segment sits at (t, h, w) in row-major order with w fastest.
   [vllm.cpp PR #26, opening commit: the DiT runs once per step over the whole
   packed sequence, with an fp64 position grid; per-segment grids follow the
   packed fl2va/ref2va layouts named there.]
2. Rotary angles.  The t, h and w axes own d_t, d_h, d_w rotated dims; axis a
   contributes d_a / 2 frequencies f_a[j] = base ** (-2 j / d_a) and the angle
   vector of a token is concat(t * f_t, h * f_h, w * f_w) (R / 2 entries,
   R = d_t + d_h + d_w).  [PR #26 description, "The device-resident forward
   (W2b)": the H3 3D MM-RoPE is plain NeoX rotate-half and only the angles,
   three axes off the fp64 grid, are unusual; encoder-tower commit: the cache
   is cat(freqs, freqs), so cos/sin repeat over the two halves.]
   Three more table modes (fp64 linspace grid, the ViT3D length-normalised
   ids, interleaved M-RoPE) change only the angles; section 2b states each.
3. Per-head RMSNorm: y = x / sqrt(mean_d x_d^2 + eps) * gamma.
   [h3-spark model card, "What this config does": Q RMSNorm then rot96 RoPE.]
4. NeoX rotary on the first R dims: pairs (i, i + R/2) for i < R/2 rotate by
   the angle of entry i; dims >= R pass through.  [same passages as 2.]
5. Attention restricted to each segment, non-causal: for every segment [a, b)
   and head, o_i = sum_j softmax_j(scale <q_i, k_j>) v_j over j in [a, b),
   with the textbook two-pass softmax (row max, exponentials, normalise).
   [PR #26 opening commit: the packed varlen non-causal attention is exactly a
   cu_seqlens varlen flash-attention call with a per-document bidirectional
   contract.]
   The encoder text tower's causal grouped-query attention (query i of a
   segment sees keys 0..i; K/V heads broadcast over their query groups) is
   section 5b; the low-precision variant (Q and K rounded to FP8 E4M3 before
   the score product) is section 5c, its per-block-scaled form section 5d,
   and the INT8 score product with per-token Q and per-key-block K scales
   section 5e (with the PV product on block-scaled E4M3 V as well); keys
   centred on their segment's mean before their INT8 codes are section 5f.

Readings where the pages are silent:
integer per-segment positions starting at 0; base 10000; gains are fp32 [D]
shared by all heads; RMSNorm before RoPE; V gets neither; empty segments are
legal and contribute nothing.

Parity against upstream H3 itself is unpinned (no upstream code or values are
available); the functions here are pinned by closed forms, brute force and
invariants in tests/test_oracle.py.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# 1. Packing and positions
# ----------------------------------------------------------------------------


def cu_seqlens(segments) -> np.ndarray:
    """Prefix sums of the segment lengths: int64 [nseg + 1], starting at 0."""
    lens = np.array([int(s[3]) for s in segments], dtype=np.int64)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def segment_positions(segments) -> np.ndarray:
    """Integer (t, h, w) of every packed token: int64 [S, 3].

    Token n of a (T, H, W) segment is at t = n // (H W), h = (n // W) mod H,
    w = n mod W (row-major, w fastest); positions restart at 0 per segment.
    """
    out = []
    for (T, H, W, L) in segments:
        n = np.arange(int(L), dtype=np.int64)
        out.append(np.stack([n // (H * W), (n // W) % H, n % W], axis=1))
    if not out:
        return np.zeros((0, 3), dtype=np.int64)
    return np.concatenate(out, axis=0)


# ----------------------------------------------------------------------------
# 2. Rotary angles and the cos/sin table
# ----------------------------------------------------------------------------


def axis_inverse_frequencies(d_axis: int, base: float) -> np.ndarray:
    """f[j] = base ** (-2 j / d_axis) for j < d_axis / 2 (fp64)."""
    j = np.arange(d_axis // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * j / np.float64(d_axis))


def rope_angles(positions: np.ndarray, rot_dims, base: float) -> np.ndarray:
    """theta [S, R/2] = concat(t * f_t, h * f_h, w * f_w) in fp64."""
    parts = []
    for axis, d_axis in enumerate(rot_dims):
        f = axis_inverse_frequencies(int(d_axis), base)
        parts.append(positions[:, axis:axis + 1].astype(np.float64) * f[None, :])
    return np.concatenate(parts, axis=1)


def rope_table(segments, rot_dims, base: float):
    """(cu_seqlens, cos, sin) with cos/sin fp64 [S, R/2]."""
    theta = rope_angles(segment_positions(segments), rot_dims, base)
    return cu_seqlens(segments), np.cos(theta), np.sin(theta)


# ----------------------------------------------------------------------------
# 2b. Other rotary table modes
#
# Besides the integer grid above, the pages name three other ways the same
# per-row cos/sin cache gets its angles:
#   LINSPACE     fp64 positions from numpy.linspace(start, stop, n,
#                endpoint=False), i.e. i * step + start with
#                step = (stop - start) / n, in that order  [PR #26
#                description, "Correctness gates": the fp64 grid feeding the
#                rotary is gated bit-exact and follows linspace's order].
#   NORMALIZED   the ViT3D decoder's length-normalised ids: (i + 0.5) / n
#                mapped into [-1, 1), times 2 pi, per-axis frequency blocks
#                concatenated; suffix tokens (registers, cls) carry id 0, an
#                identity rotation  [video-VAE decoder commit, "3D ROPE
#                DETAIL"; pipeline commit on tiling: 2 ((i + 0.5) / n) - 1].
#   INTERLEAVED  M-RoPE: the three axes interleaved [t h w t h w ...] over one
#                frequency ladder, cos/sin repeated over the two halves
#                [encoder-tower commit, "M-RoPE"].
# Readings where the pages stop short: NORMALIZED uses the per-axis
# frequencies base ** (-2 j / d_a) of the grid mode; INTERLEAVED uses the
# global ladder base ** (-2 j / R) and, for unequal axis shares, interleaves
# while the h and w shares last (entry j is h if j % 3 == 1 and j < 3 n_h, w
# if j % 3 == 2 and j < 3 n_w, t otherwise, n_a = d_a / 2); LINSPACE takes
# per-axis (start, stop) shared by all segments, n = the segment's extent on
# that axis.
# ----------------------------------------------------------------------------

ROPE_GRID, ROPE_LINSPACE, ROPE_NORMALIZED, ROPE_INTERLEAVED = 0, 1, 2, 3


def _grid_indices(segments, allow_suffix: bool):
    """Integer (t, h, w) indices [S, 3], segment extents (T, H, W) [S, 3] and
    an in-grid flag [S] (False for suffix tokens past T*H*W)."""
    idx, ext, inside = [], [], []
    for (T, H, W, L) in segments:
        T, H, W, L = int(T), int(H), int(W), int(L)
        n_grid = T * H * W
        if L > n_grid and not allow_suffix:
            raise ValueError(f"segment length {L} exceeds its grid {T}x{H}x{W}")
        n = np.arange(L, dtype=np.int64)
        g = np.minimum(n, max(n_grid - 1, 0))
        idx.append(np.where((n < n_grid)[:, None], np.stack([g // (H * W), (g // W) % H, g % W], axis=1), 0))
        ext.append(np.broadcast_to(np.array([T, H, W], dtype=np.int64), (L, 3)))
        inside.append(n < n_grid)
    if not idx:
        return np.zeros((0, 3), np.int64), np.zeros((0, 3), np.int64), np.zeros(0, bool)
    return np.concatenate(idx), np.concatenate(ext), np.concatenate(inside)


def linspace_positions(segments, start, stop) -> np.ndarray:
    """fp64 [S, 3]: along axis a, index i of an extent-n axis sits at
    i * ((stop[a] - start[a]) / n) + start[a]."""
    idx, ext, _ = _grid_indices(segments, allow_suffix=False)
    start = np.asarray(start, dtype=np.float64)
    stop = np.asarray(stop, dtype=np.float64)
    step = (stop[None, :] - start[None, :]) / ext.astype(np.float64)
    return idx.astype(np.float64) * step + start[None, :]


def normalized_positions(segments):
    """(fp64 [S, 3] of 2 ((i + 0.5) / n) - 1 per axis, in-grid flag [S])."""
    idx, ext, inside = _grid_indices(segments, allow_suffix=True)
    p = ((idx.astype(np.float64) + 0.5) / ext.astype(np.float64)) * 2.0 - 1.0
    return p, inside


def interleaved_axes(rot_dims) -> np.ndarray:
    """Axis (0 t, 1 h, 2 w) of each of the R/2 angles of the interleaved layout."""
    n_t, n_h, n_w = (int(d) // 2 for d in rot_dims)
    half = n_t + n_h + n_w
    ax = np.zeros(half, dtype=np.int64)
    for j in range(half):
        if j % 3 == 1 and j < 3 * n_h:
            ax[j] = 1
        elif j % 3 == 2 and j < 3 * n_w:
            ax[j] = 2
    return ax


def rope_table_mode(segments, mode: int, rot_dims, base: float, start=None, stop=None):
    """(cu_seqlens, cos, sin) fp64 [S, R/2] for any of the four table modes."""
    if mode == ROPE_GRID:
        return rope_table(segments, rot_dims, base)
    if mode == ROPE_LINSPACE:
        theta = rope_angles(linspace_positions(segments, start, stop), rot_dims, base)
    elif mode == ROPE_NORMALIZED:
        p, inside = normalized_positions(segments)
        theta = rope_angles(p * (2.0 * np.pi), rot_dims, base)
        theta[~inside] = 0.0
    elif mode == ROPE_INTERLEAVED:
        pos = segment_positions(segments).astype(np.float64)
        R = int(sum(rot_dims))
        ax = interleaved_axes(rot_dims)
        if [int(np.sum(ax == a)) for a in range(3)] != [int(d) // 2 for d in rot_dims]:
            raise ValueError(f"axis shares {tuple(rot_dims)} cannot be interleaved t, h, w")
        f = axis_inverse_frequencies(R, base)
        theta = pos[:, ax] * f[None, :]
    else:
        raise ValueError(f"unknown rotary table mode {mode}")
    return cu_seqlens(segments), np.cos(theta), np.sin(theta)


# ----------------------------------------------------------------------------
# 3./4. RMSNorm and rotary
# ----------------------------------------------------------------------------


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2 over the last axis) + eps) * gamma, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def rope_rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, rot_dim: int) -> np.ndarray:
    """NeoX rotate-half on x [S, heads, D] over its first rot_dim dims.

    With half = rot_dim / 2 and a = x[..., :half], b = x[..., half:rot_dim]:
    a' = a cos - b sin, b' = b cos + a sin (cos/sin [S, half] broadcast over
    heads); dims >= rot_dim are copied.
    """
    x = np.asarray(x, dtype=np.float64)
    half = rot_dim // 2
    c = cos[:, None, :]
    s = sin[:, None, :]
    a = x[..., :half]
    b = x[..., half:rot_dim]
    out = x.copy()
    out[..., :half] = a * c - b * s
    out[..., half:rot_dim] = b * c + a * s
    return out


def qk_rmsnorm_rope(q, k, gamma_q, gamma_k, eps, cos, sin, rot_dim):
    """RMSNorm each head vector of q and k with its own gain, then rotate."""
    qn = rope_rotate(rms_norm(q, gamma_q, eps), cos, sin, rot_dim)
    kn = rope_rotate(rms_norm(k, gamma_k, eps), cos, sin, rot_dim)
    return qn, kn


# ----------------------------------------------------------------------------
# 5. Attention restricted to each segment
# ----------------------------------------------------------------------------


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Two-pass softmax along the last axis: subtract the row max, exponentiate, normalise."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def segment_head_attention(q, k, v, scale: float, row_block: int = 2048):
    """softmax(scale q k^T) v for one segment and one head; q, k, v [L, D].

    Query rows are independent, so they are processed ``row_block`` at a time
    only to bound memory; nothing else is blocked.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    for r0 in range(0, q.shape[0], row_block):
        s = scale * (q[r0:r0 + row_block] @ k.T)
        out[r0:r0 + row_block] = _softmax_rows(s) @ v
    return out


def varlen_attention(q, k, v, cu, scale: float) -> np.ndarray:
    """o [S, heads, Dv] for q, k [S, heads, D], v [S, heads, Dv] packed by cu_seqlens."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o = np.zeros(q.shape[:2] + (v.shape[2],), dtype=np.float64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        for h in range(q.shape[1]):
            o[a:b, h] = segment_head_attention(q[a:b, h], k[a:b, h], v[a:b, h], scale)
    return o


def segment_of_rows(cu, rows) -> np.ndarray:
    """Index of the segment that holds each packed row."""
    return np.searchsorted(np.asarray(cu), np.asarray(rows), side="right") - 1


def varlen_attention_rows(q, k, v, cu, scale: float, rows) -> np.ndarray:
    """Output rows ``rows`` only (all heads): o[rows] [len(rows), heads, Dv].

    Each row is computed from its own segment's keys exactly as in
    varlen_attention; used where the full result is too large to compute.
    """
    rows = np.asarray(rows, dtype=np.int64)
    seg = segment_of_rows(cu, rows)
    out = np.empty((len(rows), q.shape[1], v.shape[2]), dtype=np.float64)
    for s in np.unique(seg):
        a, b = int(cu[s]), int(cu[s + 1])
        sel = np.nonzero(seg == s)[0]
        for h in range(q.shape[1]):
            qs = np.asarray(q[rows[sel], h], dtype=np.float64)
            out[sel, h] = segment_head_attention(qs, k[a:b, h], v[a:b, h], scale)
    return out


def attention_weights(q, k, cu, scale: float, seg: int, head: int) -> np.ndarray:
    """The softmax matrix [L, L] of one segment and head (for invariant checks)."""
    a, b = int(cu[seg]), int(cu[seg + 1])
    qs = np.asarray(q[a:b, head], dtype=np.float64)
    ks = np.asarray(k[a:b, head], dtype=np.float64)
    return _softmax_rows(scale * (qs @ ks.T))


# ----------------------------------------------------------------------------
# 5b. Causal and grouped-query attention
#
# The encoder's text tower runs causal attention with grouped K/V heads: a
# query head attends with the K/V head of its group, the K/V heads being
# broadcast over their query groups (encoder-tower commit, "Causal GQA
# attention"; the tower's layer: per-head q/k RMSNorm and interleaved M-RoPE,
# then causal GQA).  Reading where the pages stop short: causality is per
# packed segment with both ends aligned at the segment start (query i of a
# segment sees keys 0..i of the same segment), and query head h uses K/V head
# h // (Hq / Hkv).
# ----------------------------------------------------------------------------


def segment_head_attention_masked(q, k, v, scale: float, causal: bool, row_block: int = 2048):
    """softmax(scale q k^T + mask) v for one segment and head; the mask is -inf
    above the diagonal when causal (key j > query i), else empty."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    for r0 in range(0, q.shape[0], row_block):
        s = scale * (q[r0:r0 + row_block] @ k.T)
        if causal:
            i = np.arange(r0, r0 + s.shape[0])[:, None]
            j = np.arange(k.shape[0])[None, :]
            s = np.where(j > i, -np.inf, s)
        out[r0:r0 + row_block] = _softmax_rows(s) @ v
    return out


def varlen_attention_gqa(q, k, v, cu, scale: float, causal: bool = False) -> np.ndarray:
    """o [S, Hq, Dv] for q [S, Hq, D] and k [S, Hkv, D], v [S, Hkv, Dv], Hkv | Hq;
    query head h attends with K/V head h // (Hq // Hkv), per segment."""
    q = np.asarray(q, dtype=np.float64)
    Hq, Hkv = q.shape[1], np.asarray(k).shape[1]
    if Hq % Hkv != 0:
        raise ValueError(f"{Hkv} K/V heads do not divide {Hq} query heads")
    group = Hq // Hkv
    o = np.zeros(q.shape[:2] + (np.asarray(v).shape[2],), dtype=np.float64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        for h in range(Hq):
            kh = h // group
            o[a:b, h] = segment_head_attention_masked(q[a:b, h], k[a:b, kh], v[a:b, kh], scale, causal)
    return o


def varlen_attention_gqa_rows(q, k, v, cu, scale: float, rows, causal: bool = False) -> np.ndarray:
    """Rows ``rows`` of varlen_attention_gqa (all query heads)."""
    rows = np.asarray(rows, dtype=np.int64)
    Hq, Hkv = q.shape[1], k.shape[1]
    group = Hq // Hkv
    seg = segment_of_rows(cu, rows)
    out = np.empty((len(rows), Hq, v.shape[2]), dtype=np.float64)
    for n, r in enumerate(rows):
        a, b = int(cu[seg[n]]), int(cu[seg[n] + 1])
        end = r + 1 if causal else b
        for h in range(Hq):
            kh = h // group
            qs = np.asarray(q[r:r + 1, h], dtype=np.float64)
            out[n, h] = segment_head_attention_masked(qs, k[a:end, kh], v[a:end, kh], scale, False)[0]
    return out


# ----------------------------------------------------------------------------
# 5c. Low-precision attention: QK^T on FP8 e4m3 operands
#
# The low-precision attention the pages' GB10 builds use (SageAttention 2++,
# Comfy Kitchen's INT8 Q/K/V; h3-spark model card, runtime options and "What
# this config does") quantise Q and K before the score product.  Here Q' and
# K' are rounded to OCP FP8 E4M3 ("fn": no infinities; exponent bias 7, three
# mantissa bits, subnormals down to 2^-9, largest finite 448, codes 0x7f and
# 0xff NaN), round to nearest even, saturating at +-448.  Reading where the
# pages stop short: no per-block scale is applied, since RMSNorm bounds every
# element of q' and k' by sqrt(D) max|gamma| (well inside e4m3's range for
# the gains here) and FP8's relative precision does not depend on scale.  The
# rest of the attention is exact.
# ----------------------------------------------------------------------------


def e4m3_decode(codes) -> np.ndarray:
    """fp64 value of each E4M3 code (uint8); NaN for 0x7f and 0xff."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even mantissa), saturating
    at +-448; x must not be NaN."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    # spacing of the codes around a: 2^-9 below 2^-6, else 2^(floor(log2 a) - 3)
    ex = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    ulp = np.exp2(ex - 3.0)
    n = np.rint(a / ulp)  # np.rint rounds halves to even
    v = np.minimum(n * ulp, 448.0)
    # code from the rounded magnitude
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    sub = v < 2.0 ** -6
    mant = np.where(sub, v / 2.0 ** -9, v / np.exp2(e) * 8.0 - 8.0)
    expf = np.where(sub, 0, e + 7)
    code = (expf.astype(np.int64) << 3) + np.rint(mant).astype(np.int64)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def e4m3_round(x) -> np.ndarray:
    """x rounded to the nearest E4M3 value (saturating), as fp64."""
    return e4m3_decode(e4m3_encode(x))


def bf16_round(x) -> np.ndarray:
    """x rounded to the nearest bfloat16 value (8 significant bits, ties to even),
    directly from fp64; normal-range values (the storage precision of q' and k'
    whose E4M3 codes the low-precision path takes)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    ex = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    ulp = np.exp2(ex - 7.0)
    return np.copysign(np.rint(a / ulp) * ulp, x)


def varlen_attention_fp8qk(q, k, v, cu, scale: float, causal: bool = False) -> np.ndarray:
    """varlen_attention_gqa with q and k rounded to E4M3 first."""
    return varlen_attention_gqa(e4m3_round(q), e4m3_round(k), v, cu, scale, causal=causal)


def varlen_attention_fp8(q, k, v, cu, scale: float, causal: bool = False) -> np.ndarray:
    """varlen_attention_gqa with q, k and v rounded to E4M3 first (the operands of
    both products); the softmax weights stay exact.  (A kernel that also rounds the
    weights to E4M3 for the PV product differs from this by that rounding.)"""
    return varlen_attention_gqa(e4m3_round(q), e4m3_round(k), e4m3_round(v), cu, scale, causal=causal)


# ----------------------------------------------------------------------------
# 5d. Low-precision attention with per-block scales
#
# The pages' GB10 builds run their low-precision attention with per-block
# quantisation calibrated on the activations themselves (SageAttention 2++
# "quality attention with real-activation calibration", Comfy Kitchen's INT8
# Q/K/V kernel; h3-spark model card, "What this config does" and runtime
# options).  Reading where the pages stop short: every block of 32 consecutive
# elements along the contraction of a product -- 32 head dims of one token
# and head for q and k, 32 keys of one head dim for v, the key blocks aligned
# at the segment start -- shares one power-of-two scale 2^X, the smallest that
# brings the block's largest magnitude to at most 448 (E4M3's largest finite
# value), so no element saturates.  Each element is x * 2^-X rounded to E4M3
# (nearest even) and stands for decode(code) * 2^X.  An all-zero block has
# X = -127.  The softmax weights stay exact here, as in section 5c.
# ----------------------------------------------------------------------------

MX_BLOCK = 32


def mx_block_exponent(amax) -> np.ndarray:
    """X = ceil(log2(amax / 448)) for amax > 0, from amax's binary exponent E and
    mantissa M in [1, 2): X = E - 8 while M * 2^8 <= 448 (M <= 1.75), else
    E - 7; -127 for amax == 0; clamped to [-127, 127]."""
    a = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(a)  # a = m * 2^e, m in [0.5, 1)
    X = np.where(2.0 * m <= 1.75, e - 1 - 8, e - 1 - 7)
    X = np.where(a == 0, -127, X)
    return np.clip(X, -127, 127).astype(np.int64)


def mx_quantize(x, axis: int = -1):
    """(codes uint8 of x's shape, exponents X int64 with the block axis shortened
    by 32): blocks of 32 consecutive elements along `axis` (length a multiple
    of 32)."""
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    assert n % MX_BLOCK == 0, "block axis must be a multiple of 32"
    blocks = x.reshape(x.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    X = mx_block_exponent(np.abs(blocks).max(axis=-1))
    codes = e4m3_encode(blocks * np.exp2(-X.astype(np.float64))[..., None]).reshape(x.shape)
    return np.moveaxis(codes, -1, axis), np.moveaxis(X, -1, axis)


def mx_dequantize(codes, X, axis: int = -1) -> np.ndarray:
    """The values codes stand for: decode(code) * 2^X of the code's block."""
    c = np.moveaxis(np.asarray(codes), axis, -1)
    e = np.moveaxis(np.asarray(X), axis, -1)
    v = e4m3_decode(c).reshape(c.shape[:-1] + (c.shape[-1] // MX_BLOCK, MX_BLOCK))
    v = v * np.exp2(e.astype(np.float64))[..., None]
    return np.moveaxis(v.reshape(c.shape), -1, axis)


def mx_round(x, axis: int = -1) -> np.ndarray:
    """x rounded through per-block-scaled E4M3 along `axis`."""
    return mx_dequantize(*mx_quantize(x, axis), axis=axis)


def mx_round_keys(v, cu) -> np.ndarray:
    """v [S, H, D] rounded with blocks of 32 keys per head dim, aligned at each
    segment's start; a segment's last block is padded with zeros (which leave
    its largest magnitude unchanged)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    for a, b in zip(cu[:-1], cu[1:]):
        a, b = int(a), int(b)
        if b == a:
            continue
        n = -(-(b - a) // MX_BLOCK) * MX_BLOCK
        pad = np.zeros((n,) + v.shape[1:])
        pad[: b - a] = v[a:b]
        out[a:b] = mx_round(pad, axis=0)[: b - a]
    return out


def varlen_attention_mx_qk(q, k, v, cu, scale: float, causal: bool = False) -> np.ndarray:
    """varlen_attention_gqa with q and k rounded per 32-dim block (section 5d)."""
    return varlen_attention_gqa(mx_round(q), mx_round(k), v, cu, scale, causal=causal)


def varlen_attention_mx(q, k, v, cu, scale: float, causal: bool = False) -> np.ndarray:
    """varlen_attention_gqa with q, k rounded per 32-dim block and v per 32-key
    block of each segment; exact softmax weights.  (A kernel that also rounds
    the weights to E4M3 for the PV product differs from this by that rounding.)"""
    return varlen_attention_gqa(mx_round(q), mx_round(k), mx_round_keys(v, cu), cu, scale, causal=causal)


# ----------------------------------------------------------------------------
# 5e. INT8 scores with per-token Q and per-key-block K scales
#
# The pages' GB10 image offers INT8 attention beside its FP8-class Sage
# kernels: Comfy Kitchen's approximate INT8 Q/K/V kernel, a Sol-Attn switch
# for INT8 QK, and a fused Q RMSNorm + rot96 RoPE -> "Sage Q-INT8" tail
# (H3 Blackwell Runtime README, request-level attention backends; h3-spark
# model card, "What this config does").  Reading where the pages stop short
# (SageAttention's per-block smoothing-free form): every query row (token and
# head) of q shares one scale, and every block of 64 consecutive keys of one
# k head (aligned at the segment start; a segment's last block may be
# shorter) shares one scale over its keys and head dims.  With amax the
# block's largest magnitude, in fp32: scale = amax / 127 and code =
# rint(x * (127 / amax)) (nearest, ties to even) clamped to [-127, 127]; each
# element stands for code * scale.  An all-zero block has scale 0 and codes
# 0.  A block holding a NaN has a NaN scale, one holding an infinity an
# infinite scale, and codes 0 there: the non-finite value reaches the scores
# as NaN.  v, the softmax and the PV product stay as in section 5.
# Key blocks are numbered segment by segment: block j of segment s is
# sum over earlier segments of ceil(L / 64), plus j.
# ----------------------------------------------------------------------------

I8_KEY_BLOCK = 64


def _i8_quantize(x32, amax):
    """(codes int8, scale float32) of fp32 values x32 whose block maxima amax
    (fp32, broadcast against x32) are given."""
    with np.errstate(all="ignore"):
        inv = np.where(amax == 0, np.float32(0), np.float32(127) / amax).astype(np.float32)
        r = np.rint((x32 * inv).astype(np.float32))
        codes = np.where(np.isfinite(r), np.clip(r, -127, 127), 0).astype(np.int8)
        scale = (amax / np.float32(127)).astype(np.float32)
    return codes, scale


def i8_quantize_rows(x):
    """x [S, H, D] -> (codes int8 [S, H, D], scales float32 [H, S]): one scale
    per token and head."""
    x32 = np.asarray(x, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        amax = np.abs(x32).max(axis=-1, keepdims=True)  # NaN propagates
    codes, scale = _i8_quantize(x32, amax)
    return codes, np.ascontiguousarray(scale[..., 0].T)


def i8_key_blocks(cu) -> np.ndarray:
    """Number of the first 64-key block of each segment, and the total: int64
    [nseg + 1]."""
    lens = np.diff(np.asarray(cu, dtype=np.int64))
    return np.concatenate([[0], np.cumsum(-(-lens // I8_KEY_BLOCK))]).astype(np.int64)


def i8_quantize_key_blocks(x, cu):
    """x [S, H, D] -> (codes int8 [S, H, D], scales float32 [H, n_blocks]): one
    scale per block of 64 keys of a segment and head."""
    x32 = np.asarray(x, dtype=np.float32)
    first = i8_key_blocks(cu)
    codes = np.zeros(x32.shape, dtype=np.int8)
    scales = np.zeros((x32.shape[1], int(first[-1])), dtype=np.float32)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for j, r0 in enumerate(range(a, b, I8_KEY_BLOCK)):
            r1 = min(r0 + I8_KEY_BLOCK, b)
            blk = x32[r0:r1]  # [rows, H, D]
            with np.errstate(invalid="ignore"):
                amax = np.abs(blk).max(axis=(0, 2))  # [H]
            c, sc = _i8_quantize(blk, amax[None, :, None])
            codes[r0:r1] = c
            scales[:, first[s] + j] = sc[0, :, 0]
    return codes, scales


def i8_dequantize_rows(codes, scales) -> np.ndarray:
    """code * scale of its token and head, fp64."""
    return codes.astype(np.float64) * np.asarray(scales, dtype=np.float64).T[..., None]


def i8_dequantize_key_blocks(codes, scales, cu) -> np.ndarray:
    """code * scale of its key block and head, fp64."""
    first = i8_key_blocks(cu)
    out = np.zeros(codes.shape, dtype=np.float64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for j, r0 in enumerate(range(a, b, I8_KEY_BLOCK)):
            r1 = min(r0 + I8_KEY_BLOCK, b)
            out[r0:r1] = codes[r0:r1].astype(np.float64) * np.asarray(scales, dtype=np.float64)[:, first[s] + j][
                None, :, None]
    return out


def i8_round_q(q) -> np.ndarray:
    """q through its INT8 codes (per-token scales), fp64."""
    return i8_dequantize_rows(*i8_quantize_rows(q))


def i8_round_k(k, cu) -> np.ndarray:
    """k through its INT8 codes (per-64-key-block scales), fp64."""
    return i8_dequantize_key_blocks(*i8_quantize_key_blocks(k, cu), cu)


def varlen_attention_i8qk(q, k, v, cu, scale: float, causal: bool = False) -> np.ndarray:
    """varlen_attention_gqa with q and k replaced by what their INT8 codes stand
    for (section 5e); v and the softmax exact."""
    return varlen_attention_gqa(i8_round_q(q), i8_round_k(k, cu), v, cu, scale, causal=causal)


def varlen_attention_i8qk_mxv(q, k, v, cu, scale: float, causal: bool = False) -> np.ndarray:
    """INT8 scores with the PV product on block-scaled E4M3 values (SageAttention
    2's split between the two products, among the pages' INT8/FP8 Sage backends):
    varlen_attention_gqa with q and k replaced by what their INT8 codes stand for
    (section 5e) and v rounded per 32-key block of each segment (section 5d);
    exact softmax weights.  (A kernel that also rounds the weights to E4M3 for
    the PV product differs from this by that rounding.)"""
    return varlen_attention_gqa(i8_round_q(q), i8_round_k(k, cu), mx_round_keys(v, cu), cu, scale, causal=causal)


# ----------------------------------------------------------------------------
# 5f. Centred keys for the INT8 scores (SageAttention's K smoothing)
#
# SageAttention, among the pages' attention backends (H3 Blackwell Runtime
# README, request-level attention backends; h3-spark model card, "What this
# config does"), subtracts the mean key from K before quantising it.  Within
# one softmax every score then moves by the same q . mean, which the softmax
# cancels, so attention is unchanged while K's per-channel offsets no longer
# set the INT8 block scales.  Reading for packed segments: the mean is taken
# per segment (every key a query sees belongs to its own segment), per head
# and head dim, over the segment's keys; an empty segment has mean 0.  The
# quantised value of a key is the fp32 difference x - mean (x the bf16 key,
# mean given in fp32), quantised as in section 5e.
# ----------------------------------------------------------------------------

def segment_key_means(k, cu) -> np.ndarray:
    """[nseg, H, D] fp64: the mean of k over each segment's keys (0 if empty)."""
    k = np.asarray(k, dtype=np.float64)
    mu = np.zeros((len(cu) - 1,) + k.shape[1:])
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b > a:
            mu[s] = k[a:b].mean(axis=0)
    return mu


def i8_center_keys(k, cu, mu32) -> np.ndarray:
    """[S, H, D] fp32: each key minus its segment's mean (mu32 [nseg, H, D]
    fp32), the difference rounded once to fp32."""
    k32 = np.asarray(k, dtype=np.float32)
    mu32 = np.asarray(mu32, dtype=np.float32)
    out = np.empty_like(k32)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        out[a:b] = k32[a:b] - mu32[s][None]
    return out


def i8_quantize_key_blocks_centered(k, cu, mu32):
    """(codes, scales) of the centred keys, blocks as i8_quantize_key_blocks."""
    return i8_quantize_key_blocks(i8_center_keys(k, cu, mu32), cu)


def i8_round_k_centered(k, cu, mu32) -> np.ndarray:
    """What the centred keys' INT8 codes stand for, fp64 (the mean not added back)."""
    return i8_dequantize_key_blocks(*i8_quantize_key_blocks_centered(k, cu, mu32), cu)


def varlen_attention_i8qk_centered(q, k, v, cu, scale: float, causal: bool = False, mu32=None) -> np.ndarray:
    """INT8 scores with centred keys: varlen_attention_gqa on what q's codes and
    the centred keys' codes stand for; mu32 defaults to the segment means
    rounded to fp32.  Exact attention is unchanged by the centring; only the
    rounding differs from varlen_attention_i8qk."""
    if mu32 is None:
        mu32 = segment_key_means(k, cu).astype(np.float32)
    return varlen_attention_gqa(i8_round_q(q), i8_round_k_centered(k, cu, mu32), v, cu, scale, causal=causal)


def hot_path(q, k, v, gamma_q, gamma_k, segments, rot_dims, base, eps, scale):
    """The whole chain: table, norm + rotary on q and k, then varlen attention."""
    cu, cos, sin = rope_table(segments, rot_dims, base)
    qn, kn = qk_rmsnorm_rope(q, k, gamma_q, gamma_k, eps, cos, sin, int(sum(rot_dims)))
    return varlen_attention(qn, kn, v, cu, scale)
