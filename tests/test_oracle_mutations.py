"""Plant one plausible mistake at a time in a copy of the oracle and show that
the pins in tests/oracle_pins.py catch every one of them (CPU only)."""
import types

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


def _mutant(**replace):
    ns = types.SimpleNamespace(**{k: getattr(oracle, k) for k in dir(oracle) if not k.startswith("__")})
    for k, v in replace.items():
        setattr(ns, k, v)
    return ns


def _rope_sign_flipped(x, cos, sin, rot_dim):
    return oracle.rope_rotate(x, cos, -sin, rot_dim)


def _rope_interleaved(x, cos, sin, rot_dim):
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    a, b = x[..., 0:rot_dim:2], x[..., 1:rot_dim:2]
    out[..., 0:rot_dim:2] = a * cos[:, None] - b * sin[:, None]
    out[..., 1:rot_dim:2] = b * cos[:, None] + a * sin[:, None]
    return out


def _rope_cos_only_on_first_half(x, cos, sin, rot_dim):
    y = oracle.rope_rotate(x, cos, sin, rot_dim)
    half = rot_dim // 2
    x = np.asarray(x, dtype=np.float64)
    y[..., half:rot_dim] = x[..., half:rot_dim] * cos[:, None]  # dropped the cross term
    return y


def _rms_no_eps(x, gamma, eps):
    return oracle.rms_norm(x, gamma, 0.0)


def _rms_sum_not_mean(x, gamma, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * gamma


def _rms_gamma_reversed(x, gamma, eps):
    return oracle.rms_norm(x, np.asarray(gamma)[::-1], eps)


def _inv_freq_wrong_exponent(d_axis, base):
    j = np.arange(d_axis // 2, dtype=np.float64)
    return np.power(float(base), -j / d_axis)


def _angles_axes_reversed(positions, rot_dims, base):
    return oracle.rope_angles(positions[:, ::-1], rot_dims, base)


def _positions_h_w_swapped(segments):
    p = oracle.segment_positions(segments)
    return p[:, [0, 2, 1]]


def _attn_no_scale(q, k, v, cu, scale):
    return oracle.varlen_attention(q, k, v, cu, 1.0)


def _attn_kv_off_by_one(q, k, v, cu, scale):
    cu = np.asarray(cu).copy()
    cu[1:-1] += 1  # segment boundary one token late
    return oracle.varlen_attention(q, k, v, cu, scale)


def _attn_key_value_swapped(q, k, v, cu, scale):
    return oracle.varlen_attention(q, v, k, cu, scale) if k.shape == v.shape else oracle.varlen_attention(q, k, v, cu, scale * 1.01)


def _attn_softmax_wrong_axis(q, k, v, cu, scale):
    q = np.asarray(q, dtype=np.float64)
    o = np.zeros(q.shape[:2] + (np.asarray(v).shape[2],))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        for h in range(q.shape[1]):
            sc = scale * (q[a:b, h] @ np.asarray(k, dtype=np.float64)[a:b, h].T)
            e = np.exp(sc - sc.max(axis=0, keepdims=True))
            o[a:b, h] = (e / e.sum(axis=0, keepdims=True)) @ np.asarray(v, dtype=np.float64)[a:b, h]
    return o


def _attn_global_not_segmented(q, k, v, cu, scale):
    return oracle.varlen_attention(q, k, v, np.array([0, cu[-1]]), scale)


def _weights_unnormalised(q, k, cu, scale, seg, head):
    return 1.01 * oracle.attention_weights(q, k, cu, scale, seg, head)


def _linspace_off_by_one(segments, start, stop):
    p = oracle.linspace_positions(segments, start, stop)
    step = (np.asarray(stop, float) - np.asarray(start, float))[None, :] / oracle._grid_indices(segments, False)[1]
    return p + step


def _linspace_other_order(segments, start, stop):
    idx, ext, _ = oracle._grid_indices(segments, allow_suffix=False)
    start = np.asarray(start, dtype=np.float64)
    stop = np.asarray(stop, dtype=np.float64)
    return idx * (stop - start)[None, :] / ext + start[None, :]


def _normalized_no_half(segments):
    idx, ext, inside = oracle._grid_indices(segments, allow_suffix=True)
    return (idx / ext) * 2.0 - 1.0, inside


def _mode_variant(kind):
    def table(segments, mode, rot_dims, base, start=None, stop=None):
        if mode == oracle.ROPE_NORMALIZED and kind in ("no_two_pi", "suffix_not_identity"):
            p, inside = oracle.normalized_positions(segments)
            th = oracle.rope_angles(p if kind == "no_two_pi" else p * 2 * np.pi, rot_dims, base)
            if kind == "no_two_pi":
                th[~inside] = 0.0
            return oracle.cu_seqlens(segments), np.cos(th), np.sin(th)
        if mode == oracle.ROPE_INTERLEAVED and kind in ("per_axis_ladder", "blockwise_axes"):
            pos = oracle.segment_positions(segments).astype(np.float64)
            if kind == "per_axis_ladder":
                th = oracle.rope_angles(pos[:, :], rot_dims, base)[:, np.argsort(np.argsort(oracle.interleaved_axes(rot_dims), kind="stable"))]
            else:
                R = int(sum(rot_dims))
                ax = np.concatenate([[a] * (int(d) // 2) for a, d in enumerate(rot_dims)])
                th = pos[:, ax] * oracle.axis_inverse_frequencies(R, base)[None, :]
            return oracle.cu_seqlens(segments), np.cos(th), np.sin(th)
        return oracle.rope_table_mode(segments, mode, rot_dims, base, start, stop)
    return table


def _interleaved_axes_blockwise(rot_dims):
    return np.concatenate([[a] * (int(d) // 2) for a, d in enumerate(rot_dims)]).astype(np.int64)


def _masked_diagonal_too(q, k, v, scale, causal, row_block=2048):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    s = scale * (q @ k.T)
    if causal:
        i = np.arange(s.shape[0])[:, None]
        j = np.arange(s.shape[1])[None, :]
        s = np.where(j >= i - 1, s, s)  # keeps j == i + 1: one key too many
        s = np.where(j > i + 1, -np.inf, s)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)) @ v


def _gqa_with(masked):
    def f(q, k, v, cu, scale, causal=False):
        Hq, Hkv = q.shape[1], k.shape[1]
        o = np.zeros(q.shape[:2] + (v.shape[2],))
        for s in range(len(cu) - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            if b > a:
                for h in range(Hq):
                    g = h // (Hq // Hkv)
                    o[a:b, h] = masked(q[a:b, h], k[a:b, g], v[a:b, g], scale, causal)
        return o
    return f


def _gqa_modulo_heads(q, k, v, cu, scale, causal=False):
    Hq, Hkv = q.shape[1], k.shape[1]
    idx = np.arange(Hq) % Hkv
    return oracle.varlen_attention(q, k[:, idx], v[:, idx], cu, scale) if not causal else \
        oracle.varlen_attention_gqa(q, k[:, np.sort(idx)], v[:, np.sort(idx)], cu, scale, causal) * 1.0001


def _gqa_causal_ignored(q, k, v, cu, scale, causal=False):
    return oracle.varlen_attention_gqa(q, k, v, cu, scale, causal=False)


def _gqa_rows_one_key_short(q, k, v, cu, scale, rows, causal=False):
    rows = np.asarray(rows)
    seg = oracle.segment_of_rows(cu, rows)
    out = oracle.varlen_attention_gqa_rows(q, k, v, cu, scale, rows, causal)
    if causal:
        for n, r in enumerate(rows):
            if r > cu[seg[n]]:
                out[n] = oracle.varlen_attention_gqa_rows(q[:r], k[:r], v[:r], np.minimum(cu, r), scale,
                                                           [r - 1], causal)[0]
    return out


def _decode_bias_8(codes):
    return oracle.e4m3_decode(codes) / 2.0


def _encode_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    ex = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    ulp = np.exp2(ex - 3.0)
    v = np.minimum(np.floor(a / ulp + 0.5) * ulp, 448.0)
    return oracle.e4m3_encode(np.copysign(v, x))


def _encode_no_saturation(x):
    x = np.asarray(x, dtype=np.float64)
    c = oracle.e4m3_encode(x)
    return np.where(np.abs(x) > 448.0, np.uint8(0x7F) | (c & 0x80), c).astype(np.uint8)


def _encode_truncating(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    ex = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    ulp = np.exp2(ex - 3.0)
    return oracle.e4m3_encode(np.copysign(np.floor(a / ulp) * ulp, x))


def _fp8qk_only_q(q, k, v, cu, scale, causal=False):
    return oracle.varlen_attention_gqa(oracle.e4m3_round(q), k, v, cu, scale, causal=causal)


def _bf16_round_7_bits(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    ulp = np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 6.0)
    return np.copysign(np.rint(a / ulp) * ulp, x)


def _mx_exponent_floor(amax):
    """The OCP-style floor(log2 amax) - 8: block maxima above 1.75 * 2^E saturate."""
    a = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(a)
    return np.clip(np.where(a == 0, -127, e - 1 - 8), -127, 127).astype(np.int64)


def _mx_quantize_blocks(width):
    def q(x, axis=-1):
        x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
        n = x.shape[-1]
        blocks = x.reshape(x.shape[:-1] + (n // width, width))
        X = oracle.mx_block_exponent(np.abs(blocks).max(axis=-1))
        codes = oracle.e4m3_encode(blocks * np.exp2(-X.astype(np.float64))[..., None]).reshape(x.shape)
        X32 = X.reshape(X.shape[:-1] + (n // 32, 32 // width))[..., 0] if width < 32 else np.repeat(X, width // 32, -1)
        return np.moveaxis(codes, -1, axis), np.moveaxis(X32, -1, axis)
    return q


def _mx_keys_global_blocks(v, cu):
    """Key blocks aligned at token 0 of the packing instead of each segment's start."""
    v = np.asarray(v, dtype=np.float64)
    n = -(-v.shape[0] // 32) * 32
    pad = np.zeros((n,) + v.shape[1:])
    pad[: v.shape[0]] = v
    return oracle.mx_round(pad, axis=0)[: v.shape[0]]


def _i8_rows_with(rounding=np.rint, levels=127):
    def q(x):
        x32 = np.asarray(x, dtype=np.float32)
        amax = np.abs(x32).max(axis=-1, keepdims=True)
        with np.errstate(all="ignore"):
            inv = np.where(amax == 0, np.float32(0), np.float32(levels) / amax).astype(np.float32)
            rr = rounding((x32 * inv).astype(np.float32))
            codes = np.where(np.isfinite(rr), np.clip(rr, -127, 127), 0).astype(np.int8)
            scale = (amax / np.float32(levels)).astype(np.float32)
        return codes, np.ascontiguousarray(scale[..., 0].T)
    return q


def _i8_half_up(y):
    return np.floor(y + np.float32(0.5))


def _i8_keys_global_blocks(x, cu):
    """Key blocks of 64 tokens counted from token 0 of the packing, not each segment's start."""
    S = np.asarray(x).shape[0]
    c, sc = oracle.i8_quantize_key_blocks(x, np.array([0, S]))
    # spread the global blocks' scales over the per-segment numbering the dequantiser reads
    first = oracle.i8_key_blocks(cu)
    out = np.zeros((sc.shape[0], int(first[-1])), dtype=np.float32)
    for s in range(len(cu) - 1):
        for j, r0 in enumerate(range(int(cu[s]), int(cu[s + 1]), 64)):
            out[:, first[s] + j] = sc[:, r0 // 64]
    return c, out


MUTANTS = {
    "bf16_round_7_bits": dict(bf16_round=_bf16_round_7_bits),
    "e4m3_decode_bias_8": dict(e4m3_decode=_decode_bias_8),
    "e4m3_round_half_up": dict(e4m3_encode=_encode_half_up),
    "e4m3_no_saturation": dict(e4m3_encode=_encode_no_saturation),
    "e4m3_truncating": dict(e4m3_encode=_encode_truncating),
    "fp8qk_rounds_only_q": dict(varlen_attention_fp8qk=_fp8qk_only_q),
    "mx_exponent_floor": dict(mx_block_exponent=_mx_exponent_floor),
    "mx_blocks_of_16": dict(mx_quantize=_mx_quantize_blocks(16)),
    "mx_one_scale_per_64": dict(mx_quantize=_mx_quantize_blocks(64)),
    "mx_keys_not_segment_aligned": dict(mx_round_keys=_mx_keys_global_blocks),
    "mx_v_left_exact": dict(varlen_attention_mx=lambda q, k, v, cu, scale, causal=False:
                            oracle.varlen_attention_mx_qk(q, k, v, cu, scale, causal)),
    "fp8_leaves_v_exact": dict(varlen_attention_fp8=lambda q, k, v, cu, scale, causal=False:
                               oracle.varlen_attention_fp8qk(q, k, v, cu, scale, causal)),
    "causal_one_key_too_many": dict(varlen_attention_gqa=_gqa_with(_masked_diagonal_too)),
    "gqa_modulo_heads": dict(varlen_attention_gqa=_gqa_modulo_heads),
    "gqa_causal_ignored": dict(varlen_attention_gqa=_gqa_causal_ignored),
    "gqa_rows_one_key_short": dict(varlen_attention_gqa_rows=_gqa_rows_one_key_short),
    "linspace_off_by_one": dict(linspace_positions=_linspace_off_by_one),
    "linspace_other_order": dict(linspace_positions=_linspace_other_order),
    "normalized_no_half_offset": dict(normalized_positions=_normalized_no_half),
    "normalized_no_two_pi": dict(rope_table_mode=_mode_variant("no_two_pi")),
    "normalized_suffix_not_identity": dict(rope_table_mode=_mode_variant("suffix_not_identity")),
    "interleaved_per_axis_ladder": dict(rope_table_mode=_mode_variant("per_axis_ladder")),
    "interleaved_blockwise_axes": dict(rope_table_mode=_mode_variant("blockwise_axes")),
    "interleaved_axes_blockwise": dict(interleaved_axes=_interleaved_axes_blockwise),
    "rope_sign_flipped": dict(rope_rotate=_rope_sign_flipped),
    "rope_interleaved_pairs": dict(rope_rotate=_rope_interleaved),
    "rope_dropped_cross_term": dict(rope_rotate=_rope_cos_only_on_first_half),
    "rms_no_eps": dict(rms_norm=_rms_no_eps),
    "rms_sum_not_mean": dict(rms_norm=_rms_sum_not_mean),
    "rms_gamma_reversed": dict(rms_norm=_rms_gamma_reversed),
    "inv_freq_wrong_exponent": dict(axis_inverse_frequencies=_inv_freq_wrong_exponent),
    "angles_axes_reversed": dict(rope_angles=_angles_axes_reversed),
    "positions_h_w_swapped": dict(segment_positions=_positions_h_w_swapped),
    "attn_no_scale": dict(varlen_attention=_attn_no_scale),
    "attn_boundary_off_by_one": dict(varlen_attention=_attn_kv_off_by_one),
    "attn_k_v_swapped": dict(varlen_attention=_attn_key_value_swapped),
    "attn_softmax_wrong_axis": dict(varlen_attention=_attn_softmax_wrong_axis),
    "attn_not_segmented": dict(varlen_attention=_attn_global_not_segmented),
    "weights_unnormalised": dict(attention_weights=_weights_unnormalised),
    "i8_round_half_up": dict(i8_quantize_rows=_i8_rows_with(rounding=_i8_half_up)),
    "i8_truncating": dict(i8_quantize_rows=_i8_rows_with(rounding=np.trunc)),
    "i8_128_levels": dict(i8_quantize_rows=_i8_rows_with(levels=128)),
    "i8_keys_not_segment_aligned": dict(i8_quantize_key_blocks=_i8_keys_global_blocks),
    "i8qk_rounds_only_q": dict(varlen_attention_i8qk=lambda q, k, v, cu, scale, causal=False:
                               oracle.varlen_attention_gqa(oracle.i8_round_q(q), k, v, cu, scale, causal)),
    "i8qk_mxv_v_exact": dict(varlen_attention_i8qk_mxv=lambda q, k, v, cu, scale, causal=False:
                             oracle.varlen_attention_i8qk(q, k, v, cu, scale, causal)),
    "i8qk_mxv_v_per_dim_block": dict(varlen_attention_i8qk_mxv=lambda q, k, v, cu, scale, causal=False:
                                     oracle.varlen_attention_i8qk(q, k, oracle.mx_round(v), cu, scale, causal)),
    "i8_means_global": dict(segment_key_means=lambda k, cu: np.repeat(
        np.asarray(k, dtype=np.float64).mean(axis=0)[None], len(cu) - 1, axis=0)),
    "i8_means_over_heads": dict(segment_key_means=lambda k, cu: np.repeat(
        oracle.segment_key_means(k, cu).mean(axis=1, keepdims=True), np.asarray(k).shape[1], axis=1)),
    "i8_center_in_fp64": dict(i8_center_keys=lambda k, cu, mu32: np.asarray(k, dtype=np.float64) - np.concatenate(
        [np.repeat(np.asarray(mu32, dtype=np.float64)[i][None], int(cu[i + 1] - cu[i]), axis=0)
         for i in range(len(cu) - 1)])),
    "i8_centering_skipped": dict(i8_quantize_key_blocks_centered=lambda k, cu, mu32: oracle.i8_quantize_key_blocks(k, cu)),
    "i8qk_centered_uses_plain_keys": dict(varlen_attention_i8qk_centered=lambda q, k, v, cu, scale, causal=False, mu32=None:
                                          oracle.varlen_attention_i8qk(q, k, v, cu, scale, causal)),
    "i8qk_mxv_scores_exact": dict(varlen_attention_i8qk_mxv=lambda q, k, v, cu, scale, causal=False:
                                  oracle.varlen_attention_gqa(q, k, oracle.mx_round_keys(v, cu), cu, scale, causal)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    ns = _mutant(**MUTANTS[name])
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(ns)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
