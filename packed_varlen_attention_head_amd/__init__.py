"""Python binding of libh3a (the packed varlen attention head for MI355X).

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch tensors on the GPU in token-major [S, H, D] layout whose
last two dims are contiguous (token stride = ``tensor.stride(0)``); torch
supplies device memory and the current stream.  The names mirror the C ABI in
include/h3a.h.

If libh3a.so has not been built this module still imports, but every call
raises ``H3ALibraryMissing``: there is no CPU fallback.  Build it with
``python -m packed_varlen_attention_head_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# H3A_LIBRARY names another build of the same library (the host-sanitizer
# build of the CPU tests); by default the in-tree libh3a.so.
LIB_PATH = os.environ.get("H3A_LIBRARY") or os.path.join(_HERE, "libh3a.so")

H3A_OK, H3A_EINVAL, H3A_ESHAPE, H3A_EDTYPE, H3A_EUNSUPPORTED, H3A_EHIP = range(6)
H3A_F32, H3A_BF16 = 0, 1
STATUS_NAMES = {0: "OK", 1: "EINVAL", 2: "ESHAPE", 3: "EDTYPE", 4: "EUNSUPPORTED", 5: "EHIP"}

# Query rows per attention work item (must match the kernels).
BLOCK_M = {H3A_BF16: 128, H3A_F32: 64}

H3A_ROPE_GRID, H3A_ROPE_LINSPACE, H3A_ROPE_NORMALIZED, H3A_ROPE_INTERLEAVED = range(4)

EXPORTS = (
    "h3a_build_rope_table",
    "h3a_build_rope_table_ex",
    "h3a_qk_rmsnorm_rope",
    "h3a_qk_rmsnorm_rope_ex",
    "h3a_rmsnorm_rope",
    "h3a_varlen_attn_fwd",
    "h3a_varlen_attn_fwd_ex",
    "h3a_varlen_attn_fwd_noalloc",
    "h3a_varlen_attn_fwd_qnorm",
    "h3a_varlen_attn_fwd_fp8qk",
    "h3a_quantize_e4m3",
    "h3a_qk_rmsnorm_rope_e4m3",
    "h3a_vt_e4m3_columns",
    "h3a_prepare_vt_e4m3",
    "h3a_varlen_attn_fwd_fp8",
    "h3a_quantize_i8_rows",
    "h3a_i8_key_blocks",
    "h3a_qk_rmsnorm_rope_i8q",
    "h3a_i8_key_mean_chunks",
    "h3a_segment_key_means",
    "h3a_quantize_i8_keys_centered",
    "h3a_quantize_i8_keys",
    "h3a_varlen_attn_fwd_i8qk",
    "h3a_varlen_attn_fwd_i8qk_fp8pv",
    "h3a_plan_tiles",
    "h3a_plan_tiles_ex",
    "h3a_last_error",
    "h3a_release_caches",
    "h3a_set_split_policy",
    "h3a_version",
)


class H3AError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"h3a {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class H3ALibraryMissing(ImportError):
    pass


class RopeSpec(ctypes.Structure):
    """h3a_rope_spec: table mode, per-axis rotated dims, base, linspace start/stop."""
    _fields_ = [("mode", ctypes.c_int32), ("axis_dims", ctypes.c_int32 * 3), ("base", ctypes.c_double),
                ("start", ctypes.c_double * 3), ("stop", ctypes.c_double * 3)]


_lib = None

_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p
_i32, _i64, _f32, _f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double


def lib() -> ctypes.CDLL:
    """The loaded library with argument types declared (loaded once)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise H3ALibraryMissing(
            f"{LIB_PATH} is not built; run `python -m packed_varlen_attention_head_amd.build` "
            "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    L.h3a_build_rope_table.argtypes = [_c_i32p, _i32, _c_i32p, _f64, _vp, _i64, _c_i32p, _vp]
    L.h3a_build_rope_table_ex.argtypes = [_c_i32p, _i32, ctypes.POINTER(RopeSpec), _vp, _i64, _c_i32p, _vp]
    L.h3a_qk_rmsnorm_rope.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i64, _i64, _i64, _i64,
                                      _vp, _vp, _f32, _vp, _i32, _vp]
    L.h3a_qk_rmsnorm_rope_ex.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _i64, _i64, _i64,
                                         _i64, _vp, _vp, _f32, _vp, _i32, _vp]
    L.h3a_rmsnorm_rope.argtypes = [_vp, _vp, _i32, _i64, _i32, _i32, _i64, _i64, _vp, _f32, _vp, _i32, _vp]
    L.h3a_varlen_attn_fwd_qnorm.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _i64, _i64, _i64,
                                            _i64, _c_i32p, _i32, _f32, _vp, _f32, _vp, _i32, _vp]
    L.h3a_qk_rmsnorm_rope_e4m3.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _i64, _i64,
                                           _i64, _vp, _vp, _f32, _vp, _i32, _vp]
    L.h3a_vt_e4m3_columns.argtypes = [_c_i32p, _i32, _c_i64p]
    L.h3a_prepare_vt_e4m3.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, _i64, _i64, _c_i32p, _i32, _vp]
    L.h3a_varlen_attn_fwd_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _i64,
                                          _i64, _i64,
                                          _c_i32p, _i32, _f32, _i32, _vp]
    L.h3a_quantize_e4m3.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, _i64, _i64, _vp]
    L.h3a_varlen_attn_fwd_fp8qk.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _i64,
                                            _i64, _i64,
                                            _c_i32p, _i32, _f32, _i32, _vp]
    L.h3a_quantize_i8_rows.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, _i64, _i64, _vp]
    L.h3a_i8_key_blocks.argtypes = [_c_i32p, _i32, _c_i64p]
    L.h3a_qk_rmsnorm_rope_i8q.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _i64, _i64, _i64,
                                          _vp, _vp, _f32, _vp, _i32, _vp]
    L.h3a_quantize_i8_keys.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, _i64, _i64, _i64, _c_i32p, _i32, _vp]
    L.h3a_quantize_i8_keys_centered.argtypes = [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i64, _i64, _i64, _c_i32p, _i32,
                                                _vp]
    L.h3a_i8_key_mean_chunks.argtypes = [_c_i32p, _i32, _c_i64p]
    L.h3a_segment_key_means.argtypes = [_vp, _vp, _vp, _i64, _i32, _i32, _i64, _i64, _c_i32p, _i32, _vp]
    L.h3a_varlen_attn_fwd_i8qk.argtypes = L.h3a_varlen_attn_fwd_fp8qk.argtypes
    L.h3a_varlen_attn_fwd_i8qk_fp8pv.argtypes = L.h3a_varlen_attn_fwd_fp8.argtypes
    L.h3a_varlen_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i64, _i64, _i64, _i64,
                                      _c_i32p, _i32, _f32, _vp]
    L.h3a_varlen_attn_fwd_ex.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _i64, _i64, _i64,
                                         _i64, _c_i32p, _i32, _f32, _i32, _vp]
    L.h3a_varlen_attn_fwd_noalloc.argtypes = L.h3a_varlen_attn_fwd_ex.argtypes
    L.h3a_plan_tiles.argtypes = [_c_i32p, _i32, _i32, _i32, _i32, _c_i32p, _i64, _c_i64p]
    L.h3a_plan_tiles_ex.argtypes = [_c_i32p, _i32, _i32, _i32, _i32, _i32, _c_i32p, _i64, _c_i64p]
    for name in ("h3a_build_rope_table", "h3a_build_rope_table_ex", "h3a_qk_rmsnorm_rope", "h3a_qk_rmsnorm_rope_ex",
                 "h3a_rmsnorm_rope", "h3a_varlen_attn_fwd_qnorm", "h3a_varlen_attn_fwd",
                 "h3a_quantize_e4m3", "h3a_varlen_attn_fwd_fp8qk", "h3a_qk_rmsnorm_rope_e4m3",
                 "h3a_vt_e4m3_columns", "h3a_prepare_vt_e4m3", "h3a_varlen_attn_fwd_fp8",
                 "h3a_quantize_i8_rows", "h3a_i8_key_blocks", "h3a_quantize_i8_keys", "h3a_varlen_attn_fwd_i8qk",
                 "h3a_qk_rmsnorm_rope_i8q", "h3a_varlen_attn_fwd_i8qk_fp8pv", "h3a_i8_key_mean_chunks",
                 "h3a_segment_key_means", "h3a_quantize_i8_keys_centered",
                 "h3a_varlen_attn_fwd_ex", "h3a_varlen_attn_fwd_noalloc", "h3a_plan_tiles", "h3a_plan_tiles_ex"):
        getattr(L, name).restype = ctypes.c_int
    L.h3a_last_error.restype = ctypes.c_char_p
    L.h3a_last_error.argtypes = []
    L.h3a_release_caches.restype = None
    L.h3a_release_caches.argtypes = []
    L.h3a_version.restype = ctypes.c_int32
    L.h3a_version.argtypes = []
    L.h3a_set_split_policy.restype = ctypes.c_int
    L.h3a_set_split_policy.argtypes = [_i32]
    _lib = L
    return L


def last_error() -> str:
    return lib().h3a_last_error().decode()


def _check(status: int):
    if status != H3A_OK:
        raise H3AError(status, last_error())


def version() -> int:
    return int(lib().h3a_version())


def release_caches() -> None:
    lib().h3a_release_caches()


H3A_SPLIT_AUTO, H3A_SPLIT_NEVER, H3A_SPLIT_ALWAYS = range(3)


def set_split_policy(policy: int) -> None:
    """Key-range splitting of attention plans built from now on (H3A_SPLIT_*)."""
    _check(lib().h3a_set_split_policy(int(policy)))


def _i32_array(values) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(values, dtype=np.int32))


def _ptr_i32(a: np.ndarray):
    return a.ctypes.data_as(_c_i32p)


def _stream_handle(stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return H3A_BF16
    if t.dtype == torch.float32:
        return H3A_F32
    raise H3AError(H3A_EDTYPE, f"tensor dtype {t.dtype} (supported: bfloat16, float32)")


def _token_major(name: str, t):
    """(S, H, D, token stride) of a [S, H, D] tensor with contiguous last two dims."""
    if t.dim() != 3:
        raise H3AError(H3A_ESHAPE, f"{name} must be [S, H, D], got shape {tuple(t.shape)}")
    S, H, D = t.shape
    if t.stride(2) != 1 or (H > 1 and t.stride(1) != D):
        raise H3AError(H3A_ESHAPE, f"{name}: heads and dims must be contiguous, strides {t.stride()}")
    if not t.is_cuda:
        raise H3AError(H3A_EINVAL, f"{name} must be a GPU tensor")
    _on_current_device(name, t)
    return S, H, D, t.stride(0)


def _on_current_device(name: str, t):
    import torch

    if t.device.index != torch.cuda.current_device():
        raise H3AError(H3A_EINVAL, f"{name} is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")


def _expect(name: str, t, shape, dtype, contiguous: bool = True):
    """A GPU tensor on the current device with exactly this shape and dtype: the
    library reads or writes its whole extent through a raw pointer."""
    if t is None:
        raise H3AError(H3A_EINVAL, f"{name} is None")
    if not t.is_cuda:
        raise H3AError(H3A_EINVAL, f"{name} must be a GPU tensor")
    _on_current_device(name, t)
    if t.dtype != dtype:
        raise H3AError(H3A_EDTYPE, f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise H3AError(H3A_ESHAPE, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise H3AError(H3A_ESHAPE, f"{name} must be contiguous")


def _gain(name: str, g, D: int) -> int:
    import torch

    _expect(name, g, (D,), torch.float32)
    return g.data_ptr()


def _table(cos_sin, S: int, rot_dim: int):
    """Pointer of the [2, S, rot_dim/2] fp32 rotary table (None allowed when nothing rotates)."""
    import torch

    if cos_sin is None:
        return None
    if rot_dim > 0 and S > 0:
        _expect("cos_sin", cos_sin, (2, S, rot_dim // 2), torch.float32)
    return cos_sin.data_ptr()


def _same(name: str, t, shape, dtype):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise H3AError(H3A_ESHAPE, f"{name} shape/dtype {tuple(t.shape)}/{t.dtype} must be {tuple(shape)}/{dtype}")


# ---------------------------------------------------------------------------
# the three calls of the hot path
# ---------------------------------------------------------------------------

def build_rope_table(segments, axis_dims, base: float, cos_sin, stream=None) -> np.ndarray:
    """Fill ``cos_sin`` (fp32 GPU tensor [2, S, R/2]) and return cu_seqlens (int32 [nseg+1]).

    ``segments``: sequence of (T, H, W, L); ``axis_dims``: rotated dims of the t, h, w axes.
    """
    segs = _i32_array(segments).reshape(-1, 4)
    dims = _i32_array(axis_dims)
    S = int(segs[:, 3].sum()) if len(segs) else 0
    cu = np.zeros(len(segs) + 1, dtype=np.int32)
    ptr = _table(cos_sin, S, int(dims.sum()))
    _check(lib().h3a_build_rope_table(_ptr_i32(segs), len(segs), _ptr_i32(dims), float(base), ptr, S,
                                      _ptr_i32(cu), _stream_handle(stream)))
    return cu


def rope_spec(mode: int, axis_dims, base: float, start=(0.0, 0.0, 0.0), stop=(0.0, 0.0, 0.0)) -> RopeSpec:
    spec = RopeSpec()
    spec.mode = int(mode)
    for a in range(3):
        spec.axis_dims[a] = int(axis_dims[a])
        spec.start[a] = float(start[a])
        spec.stop[a] = float(stop[a])
    spec.base = float(base)
    return spec


def build_rope_table_ex(segments, mode: int, axis_dims, base: float, cos_sin, start=(0.0, 0.0, 0.0),
                        stop=(0.0, 0.0, 0.0), stream=None) -> np.ndarray:
    """Fill ``cos_sin`` in table mode ``mode`` (H3A_ROPE_*); returns cu_seqlens."""
    segs = _i32_array(segments).reshape(-1, 4)
    S = int(segs[:, 3].sum()) if len(segs) else 0
    cu = np.zeros(len(segs) + 1, dtype=np.int32)
    spec = rope_spec(mode, axis_dims, base, start, stop)
    ptr = _table(cos_sin, S, int(sum(int(a) for a in axis_dims)))
    _check(lib().h3a_build_rope_table_ex(_ptr_i32(segs), len(segs), ctypes.byref(spec), ptr, S, _ptr_i32(cu),
                                         _stream_handle(stream)))
    return cu


def qk_rmsnorm_rope(q, k, gamma_q, gamma_k, eps: float, cos_sin, rot_dim: int, q_out=None, k_out=None,
                    stream=None):
    """RMSNorm + NeoX rotary of q and k; in place unless q_out / k_out are given.

    k may have fewer heads than q (grouped K/V heads); then the _ex entry runs."""
    q_out = q if q_out is None else q_out
    k_out = k if k_out is None else k_out
    S, H, D, sq = _token_major("q", q)
    _, Hk, _, sk = _token_major("k", k)
    _, _, _, sqo = _token_major("q_out", q_out)
    _, _, _, sko = _token_major("k_out", k_out)
    for name, t, h in (("k", k, Hk), ("q_out", q_out, H), ("k_out", k_out, Hk)):
        if tuple(t.shape) != (S, h, D) or t.dtype != q.dtype:
            raise H3AError(H3A_ESHAPE, f"{name} shape/dtype {tuple(t.shape)}/{t.dtype} does not match q")
    cs = _table(cos_sin, S, int(rot_dim))
    args = (q.data_ptr(), k.data_ptr(), q_out.data_ptr(), k_out.data_ptr(), _dtype_code(q), S)
    rest = (D, sq, sk, sqo, sko, _gain("gamma_q", gamma_q, D), _gain("gamma_k", gamma_k, D), float(eps), cs,
            int(rot_dim), _stream_handle(stream))
    if Hk == H:
        _check(lib().h3a_qk_rmsnorm_rope(*args, H, *rest))
    else:
        _check(lib().h3a_qk_rmsnorm_rope_ex(*args, H, Hk, *rest))
    return q_out, k_out


def varlen_attn_fwd(q, k, v, cu_seqlens, scale: float, out=None, stream=None):
    """Per-segment bidirectional attention; returns ``out`` ([S, H, D], same dtype as q)."""
    import torch

    S, H, D, sq = _token_major("q", q)
    _, _, _, sk = _token_major("k", k)
    _, _, _, sv = _token_major("v", v)
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (S, H, D) or t.dtype != q.dtype:
            raise H3AError(H3A_ESHAPE, f"{name} shape/dtype {tuple(t.shape)}/{t.dtype} differs from q")
    if out is None:
        out = torch.empty((S, H, D), dtype=q.dtype, device=q.device)
    _, _, _, so = _token_major("out", out)
    _same("out", out, (S, H, D), q.dtype)
    cu = _i32_array(cu_seqlens)
    _check(lib().h3a_varlen_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _dtype_code(q),
                                     S, H, D, sq, sk, sv, so, _ptr_i32(cu), len(cu) - 1, float(scale),
                                     _stream_handle(stream)))
    return out


def rmsnorm_rope(x, gamma, eps: float, cos_sin, rot_dim: int, x_out=None, stream=None):
    """RMSNorm + NeoX rotary of one [S, H, D] tensor; in place unless x_out is given."""
    x_out = x if x_out is None else x_out
    S, H, D, sx = _token_major("x", x)
    _, _, _, sxo = _token_major("x_out", x_out)
    if tuple(x_out.shape) != (S, H, D) or x_out.dtype != x.dtype:
        raise H3AError(H3A_ESHAPE, f"x_out shape/dtype {tuple(x_out.shape)}/{x_out.dtype} differs from x")
    cs = _table(cos_sin, S, int(rot_dim))
    _check(lib().h3a_rmsnorm_rope(x.data_ptr(), x_out.data_ptr(), _dtype_code(x), S, H, D, sx, sxo,
                                  _gain("gamma", gamma, D), float(eps), cs, int(rot_dim), _stream_handle(stream)))
    return x_out


def varlen_attn_fwd_qnorm(q, k, v, cu_seqlens, scale: float, gamma_q, eps: float, cos_sin, rot_dim: int,
                          out=None, stream=None):
    """Bidirectional attention on raw q (normalised and rotated inside the kernel) and prepared k, v."""
    import torch

    S, Hq, D, sq = _token_major("q", q)
    _, Hkv, _, sk = _token_major("k", k)
    _, _, _, sv = _token_major("v", v)
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (S, Hkv, D) or t.dtype != q.dtype:
            raise H3AError(H3A_ESHAPE, f"{name} shape/dtype {tuple(t.shape)}/{t.dtype} differs from "
                                       f"{(S, Hkv, D)}/{q.dtype}")
    if out is None:
        out = torch.empty((S, Hq, D), dtype=q.dtype, device=q.device)
    _, _, _, so = _token_major("out", out)
    _same("out", out, (S, Hq, D), q.dtype)
    cu = _i32_array(cu_seqlens)
    cs = _table(cos_sin, S, int(rot_dim))
    _check(lib().h3a_varlen_attn_fwd_qnorm(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                           _dtype_code(q), S, Hq, Hkv, D, sq, sk, sv, so, _ptr_i32(cu), len(cu) - 1,
                                           float(scale), _gain("gamma_q", gamma_q, D), float(eps), cs, int(rot_dim),
                                           _stream_handle(stream)))
    return out


# Low-precision operands are (codes, scales) pairs: uint8 E4M3 codes and one
# uint8 E8M0 scale per 32 elements along the contraction -- head-major
# [H, S, D // 32] for q and k (a tile's keys contiguous), [Hkv, vt_cols // 64, 2, 32, D // 32] for the transposed V.

def _scales(name, t, shape, device):
    """A scale array must be exactly the packed shape the kernels address."""
    import torch

    if t is None:
        return torch.empty(shape, dtype=torch.uint8, device=device)
    _expect(name, t, shape, torch.uint8)
    return t


def _pair(name, x):
    if not (isinstance(x, (tuple, list)) and len(x) == 2):
        raise H3AError(H3A_EINVAL, f"{name} must be a (codes, scales) pair")
    return x[0], x[1]


def quantize_e4m3(x, out=None, scale_out=None, stream=None):
    """bf16 [S, H, D] -> (uint8 [S, H, D] E4M3 codes, uint8 [H, S, D // 32] block scales)."""
    import torch

    S, H, D, sx = _token_major("x", x)
    if x.dtype != torch.bfloat16:
        raise H3AError(H3A_EDTYPE, f"x must be bfloat16, got {x.dtype}")
    if out is None:
        out = torch.empty((S, H, D), dtype=torch.uint8, device=x.device)
    _, _, _, sy = _token_major("out", out)
    if tuple(out.shape) != (S, H, D) or out.dtype != torch.uint8:
        raise H3AError(H3A_ESHAPE, f"out must be uint8 {(S, H, D)}, got {out.dtype} {tuple(out.shape)}")
    sc = _scales("scale_out", scale_out, (H, S, D // 32), x.device)
    _check(lib().h3a_quantize_e4m3(x.data_ptr(), out.data_ptr(), sc.data_ptr(), S, H, D, sx, sy,
                                   _stream_handle(stream)))
    return out, sc


def qk_rmsnorm_rope_e4m3(q, k, gamma_q, gamma_k, eps: float, cos_sin, rot_dim: int, q8=None, k8=None,
                         q_scale=None, k_scale=None, stream=None):
    """Norm + rotary of bf16 q [S, Hq, D], k [S, Hk, D] written as block-scaled E4M3;
    returns ((q8, q_scale), (k8, k_scale))."""
    import torch

    S, Hq, D, sq = _token_major("q", q)
    _, Hk, _, sk = _token_major("k", k)
    q8 = torch.empty((S, Hq, D), dtype=torch.uint8, device=q.device) if q8 is None else q8
    k8 = torch.empty((S, Hk, D), dtype=torch.uint8, device=q.device) if k8 is None else k8
    _, _, _, sq8 = _token_major("q8", q8)
    _, _, _, sk8 = _token_major("k8", k8)
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16:
        raise H3AError(H3A_EDTYPE, f"q/k must be bfloat16, got {q.dtype}/{k.dtype}")
    if tuple(k.shape) != (S, Hk, D):
        raise H3AError(H3A_ESHAPE, f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    _same("q8", q8, (S, Hq, D), torch.uint8)
    _same("k8", k8, (S, Hk, D), torch.uint8)
    qs = _scales("q_scale", q_scale, (Hq, S, D // 32), q.device)
    ks = _scales("k_scale", k_scale, (Hk, S, D // 32), q.device)
    cs = _table(cos_sin, S, int(rot_dim))
    _check(lib().h3a_qk_rmsnorm_rope_e4m3(q.data_ptr(), k.data_ptr(), q8.data_ptr(), k8.data_ptr(), qs.data_ptr(),
                                          ks.data_ptr(), S, Hq, Hk, D, sq, sk, sq8, sk8,
                                          _gain("gamma_q", gamma_q, D), _gain("gamma_k", gamma_k, D),
                                          float(eps), cs, int(rot_dim), _stream_handle(stream)))
    return (q8, qs), (k8, ks)


def vt_e4m3_columns(cu_seqlens) -> int:
    """Columns of the transposed E4M3 V layout for cu_seqlens (segments padded to 64 keys)."""
    cu = _i32_array(cu_seqlens)
    n = ctypes.c_int64(0)
    _check(lib().h3a_vt_e4m3_columns(_ptr_i32(cu), len(cu) - 1, ctypes.byref(n)))
    return int(n.value)


def prepare_vt_e4m3(v, cu_seqlens, out=None, scale_out=None, stream=None):
    """bf16 v [S, Hkv, D] -> (uint8 [Hkv, D, vt_cols] transposed E4M3 codes, segment-padded;
    uint8 [Hkv, vt_cols // 64, 2, 32, D // 32] block scales)."""
    import torch

    S, Hkv, D, sv = _token_major("v", v)
    if v.dtype != torch.bfloat16:
        raise H3AError(H3A_EDTYPE, f"v must be bfloat16, got {v.dtype}")
    cu = _i32_array(cu_seqlens)
    cols = vt_e4m3_columns(cu)
    if out is None:
        out = torch.empty((Hkv, D, max(cols, 1)), dtype=torch.uint8, device=v.device)
    # rows of exactly `cols` columns (one column when every segment is empty)
    _expect("out", out, (Hkv, D, max(cols, 1)), torch.uint8)
    sc = _scales("scale_out", scale_out, (Hkv, max(cols, 64) // 64, 2, 32, D // 32), v.device)
    _check(lib().h3a_prepare_vt_e4m3(v.data_ptr(), out.data_ptr(), sc.data_ptr(), S, Hkv, D, sv, cols, _ptr_i32(cu),
                                     len(cu) - 1, _stream_handle(stream)))
    return out, sc


def varlen_attn_fwd_fp8(q8, k8, vt8, cu_seqlens, scale: float, causal: bool = False, out=None, stream=None):
    """Attention with q8, k8 (codes, scales) pairs [S, H, D] and vt8 (codes, scales) from
    prepare_vt_e4m3; bf16 output."""
    import torch

    (q8, qs), (k8, ks), (vt8, vs) = _pair("q8", q8), _pair("k8", k8), _pair("vt8", vt8)
    S, Hq, D, sq = _token_major("q8", q8)
    _, Hkv, _, sk = _token_major("k8", k8)
    if q8.dtype != torch.uint8 or k8.dtype != torch.uint8:
        raise H3AError(H3A_EDTYPE, f"q8/k8 must hold uint8 E4M3 codes, got {q8.dtype}/{k8.dtype}")
    if tuple(k8.shape) != (S, Hkv, D):
        raise H3AError(H3A_ESHAPE, f"k8 shape {tuple(k8.shape)} does not match q8 {tuple(q8.shape)}")
    cu = _i32_array(cu_seqlens)
    cols = vt_e4m3_columns(cu)
    # the kernel addresses vt8 with exactly `cols` columns per row
    _expect("vt8", vt8, (Hkv, D, max(cols, 1)), torch.uint8)
    qs = _scales("q_scale", qs, (Hq, S, D // 32), q8.device)
    ks = _scales("k_scale", ks, (Hkv, S, D // 32), q8.device)
    vs = _scales("vt_scale", vs, (Hkv, max(cols, 64) // 64, 2, 32, D // 32), q8.device)
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=q8.device)
    _, _, _, so = _token_major("out", out)
    _same("out", out, (S, Hq, D), torch.bfloat16)
    _check(lib().h3a_varlen_attn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), qs.data_ptr(), ks.data_ptr(),
                                         vs.data_ptr(), out.data_ptr(), S, Hq, Hkv, D, sq, sk, cols, so, _ptr_i32(cu),
                                         len(cu) - 1, float(scale), int(bool(causal)), _stream_handle(stream)))
    return out


def varlen_attn_fwd_fp8qk(q8, k8, v, cu_seqlens, scale: float, causal: bool = False, out=None, stream=None):
    """Attention with q8 [S, Hq, D] and k8 [S, Hkv, D] as (codes, scales) pairs, v bf16 [S, Hkv, D]."""
    import torch

    (q8, qs), (k8, ks) = _pair("q8", q8), _pair("k8", k8)
    S, Hq, D, sq = _token_major("q8", q8)
    _, Hkv, _, sk = _token_major("k8", k8)
    _, _, _, sv = _token_major("v", v)
    if q8.dtype != torch.uint8 or k8.dtype != torch.uint8:
        raise H3AError(H3A_EDTYPE, f"q8/k8 must hold uint8 E4M3 codes, got {q8.dtype}/{k8.dtype}")
    if tuple(k8.shape) != (S, Hkv, D) or tuple(v.shape) != (S, Hkv, D) or v.dtype != torch.bfloat16:
        raise H3AError(H3A_ESHAPE, f"k8 {tuple(k8.shape)} / v {tuple(v.shape)} {v.dtype} do not match q8")
    qs = _scales("q_scale", qs, (Hq, S, D // 32), q8.device)
    ks = _scales("k_scale", ks, (Hkv, S, D // 32), q8.device)
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=v.device)
    _, _, _, so = _token_major("out", out)
    _same("out", out, (S, Hq, D), torch.bfloat16)
    cu = _i32_array(cu_seqlens)
    _check(lib().h3a_varlen_attn_fwd_fp8qk(q8.data_ptr(), k8.data_ptr(), qs.data_ptr(), ks.data_ptr(), v.data_ptr(),
                                           out.data_ptr(), S, Hq, Hkv, D, sq, sk, sv, so, _ptr_i32(cu), len(cu) - 1,
                                           float(scale), int(bool(causal)), _stream_handle(stream)))
    return out


# INT8 operands are (codes, scales) pairs too: int8 codes and fp32 scales,
# [H, S] per token for q and [H, n_blocks] per 64-key block of a segment for k.

def _f32_scales(name, t, shape, device):
    import torch

    if t is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    _expect(name, t, shape, torch.float32)
    return t


def _i8_out(name, out, x, S, H, D):
    import torch

    if out is None:
        out = torch.empty((S, H, D), dtype=torch.int8, device=x.device)
    _, _, _, sy = _token_major(name, out)
    if tuple(out.shape) != (S, H, D) or out.dtype != torch.int8:
        raise H3AError(H3A_ESHAPE, f"{name} must be int8 {(S, H, D)}, got {out.dtype} {tuple(out.shape)}")
    return out, sy


def quantize_i8_rows(x, out=None, scale_out=None, stream=None):
    """bf16 [S, H, D] -> (int8 [S, H, D] codes, fp32 [H, S] per-token scales)."""
    import torch

    S, H, D, sx = _token_major("x", x)
    if x.dtype != torch.bfloat16:
        raise H3AError(H3A_EDTYPE, f"x must be bfloat16, got {x.dtype}")
    out, sy = _i8_out("out", out, x, S, H, D)
    sc = _f32_scales("scale_out", scale_out, (H, S), x.device)
    _check(lib().h3a_quantize_i8_rows(x.data_ptr(), out.data_ptr(), sc.data_ptr(), S, H, D, sx, sy,
                                      _stream_handle(stream)))
    return out, sc


def qk_rmsnorm_rope_i8q(q, k, gamma_q, gamma_k, eps: float, cos_sin, rot_dim: int, q8=None, q_scale=None,
                        k_out=None, stream=None):
    """Norm + rotary of bf16 q [S, Hq, D], k [S, Hk, D] with q written as INT8 codes and per-token
    scales, k as bf16 (k_out may be k); returns ((q8, q_scale), k_out)."""
    import torch

    S, Hq, D, sq = _token_major("q", q)
    _, Hk, _, sk = _token_major("k", k)
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16:
        raise H3AError(H3A_EDTYPE, f"q/k must be bfloat16, got {q.dtype}/{k.dtype}")
    if tuple(k.shape) != (S, Hk, D):
        raise H3AError(H3A_ESHAPE, f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    q8, sq8 = _i8_out("q8", q8, q, S, Hq, D)
    qs = _f32_scales("q_scale", q_scale, (Hq, S), q.device)
    k_out = torch.empty_like(k, memory_format=torch.contiguous_format) if k_out is None else k_out
    _, _, _, sko = _token_major("k_out", k_out)
    _same("k_out", k_out, (S, Hk, D), torch.bfloat16)
    cs = _table(cos_sin, S, int(rot_dim))
    _check(lib().h3a_qk_rmsnorm_rope_i8q(q.data_ptr(), k.data_ptr(), q8.data_ptr(), k_out.data_ptr(), qs.data_ptr(),
                                         S, Hq, Hk, D, sq, sk, sq8, sko, _gain("gamma_q", gamma_q, D),
                                         _gain("gamma_k", gamma_k, D), float(eps), cs, int(rot_dim),
                                         _stream_handle(stream)))
    return (q8, qs), k_out


def i8_key_blocks(cu_seqlens) -> int:
    """Number of 64-key blocks of cu_seqlens (each segment's keys in blocks from its start)."""
    cu = _i32_array(cu_seqlens)
    n = ctypes.c_int64(0)
    _check(lib().h3a_i8_key_blocks(_ptr_i32(cu), len(cu) - 1, ctypes.byref(n)))
    return int(n.value)


def quantize_i8_keys(x, cu_seqlens, out=None, scale_out=None, mu=None, stream=None):
    """bf16 [S, H, D] -> (int8 [S, H, D] codes, fp32 [H, n_blocks] scales, one per 64 keys of a segment);
    with mu (fp32 [nseg, H, D], e.g. segment_key_means) the codes of the centred keys x - mu[segment]."""
    import torch

    S, H, D, sx = _token_major("x", x)
    if x.dtype != torch.bfloat16:
        raise H3AError(H3A_EDTYPE, f"x must be bfloat16, got {x.dtype}")
    cu = _i32_array(cu_seqlens)
    nb = i8_key_blocks(cu)
    out, sy = _i8_out("out", out, x, S, H, D)
    sc = _f32_scales("scale_out", scale_out, (H, max(nb, 1)), x.device)
    if mu is None:
        _check(lib().h3a_quantize_i8_keys(x.data_ptr(), out.data_ptr(), sc.data_ptr(), S, H, D, sx, sy, nb,
                                          _ptr_i32(cu), len(cu) - 1, _stream_handle(stream)))
    else:
        _expect("mu", mu, (len(cu) - 1, H, D), torch.float32)
        _check(lib().h3a_quantize_i8_keys_centered(x.data_ptr(), mu.data_ptr(), out.data_ptr(), sc.data_ptr(), S, H,
                                                   D, sx, sy, nb, _ptr_i32(cu), len(cu) - 1, _stream_handle(stream)))
    return out, sc


def i8_key_mean_chunks(cu_seqlens) -> int:
    """Number of 256-key chunks of cu_seqlens (the workspace rows of segment_key_means)."""
    cu = _i32_array(cu_seqlens)
    n = ctypes.c_int64(0)
    _check(lib().h3a_i8_key_mean_chunks(_ptr_i32(cu), len(cu) - 1, ctypes.byref(n)))
    return int(n.value)


def segment_key_means(k, cu_seqlens, out=None, workspace=None, stream=None):
    """bf16 k [S, H, D] -> fp32 [nseg, H, D]: each segment's mean key (0 for an empty segment)."""
    import torch

    S, H, D, sk = _token_major("k", k)
    if k.dtype != torch.bfloat16:
        raise H3AError(H3A_EDTYPE, f"k must be bfloat16, got {k.dtype}")
    cu = _i32_array(cu_seqlens)
    nc = i8_key_mean_chunks(cu)
    out = _f32_scales("out", out, (len(cu) - 1, H, D), k.device)
    ws = _f32_scales("workspace", workspace, (max(nc, 1), H, D), k.device)
    _check(lib().h3a_segment_key_means(k.data_ptr(), ws.data_ptr(), out.data_ptr(), S, H, D, sk, nc, _ptr_i32(cu),
                                       len(cu) - 1, _stream_handle(stream)))
    return out


def varlen_attn_fwd_i8qk(q8, k8, v, cu_seqlens, scale: float, causal: bool = False, out=None, stream=None):
    """Attention with q8 = quantize_i8_rows(q) and k8 = quantize_i8_keys(k, cu_seqlens) pairs, bf16 v."""
    import torch

    (q8, qs), (k8, ks) = _pair("q8", q8), _pair("k8", k8)
    S, Hq, D, sq = _token_major("q8", q8)
    _, Hkv, _, sk = _token_major("k8", k8)
    _, _, _, sv = _token_major("v", v)
    if q8.dtype != torch.int8 or k8.dtype != torch.int8:
        raise H3AError(H3A_EDTYPE, f"q8/k8 must hold int8 codes, got {q8.dtype}/{k8.dtype}")
    if tuple(k8.shape) != (S, Hkv, D) or tuple(v.shape) != (S, Hkv, D) or v.dtype != torch.bfloat16:
        raise H3AError(H3A_ESHAPE, f"k8 {tuple(k8.shape)} / v {tuple(v.shape)} {v.dtype} do not match q8")
    cu = _i32_array(cu_seqlens)
    nb = i8_key_blocks(cu)
    qs = _f32_scales("q_scale", qs, (Hq, S), q8.device)
    ks = _f32_scales("k_scale", ks, (Hkv, max(nb, 1)), q8.device)
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=v.device)
    _, _, _, so = _token_major("out", out)
    _same("out", out, (S, Hq, D), torch.bfloat16)
    _check(lib().h3a_varlen_attn_fwd_i8qk(q8.data_ptr(), k8.data_ptr(), qs.data_ptr(), ks.data_ptr(), v.data_ptr(),
                                          out.data_ptr(), S, Hq, Hkv, D, sq, sk, sv, so, _ptr_i32(cu), len(cu) - 1,
                                          float(scale), int(bool(causal)), _stream_handle(stream)))
    return out


def varlen_attn_fwd_i8qk_fp8pv(q8, k8, vt8, cu_seqlens, scale: float, causal: bool = False, out=None,
                              stream=None):
    """Attention with INT8 q8 = quantize_i8_rows(q), k8 = quantize_i8_keys(k, cu_seqlens) pairs and
    vt8 = prepare_vt_e4m3(v, cu_seqlens) (E4M3 V^T codes, scales); bf16 output."""
    import torch

    (q8, qs), (k8, ks), (vt8, vs) = _pair("q8", q8), _pair("k8", k8), _pair("vt8", vt8)
    S, Hq, D, sq = _token_major("q8", q8)
    _, Hkv, _, sk = _token_major("k8", k8)
    if q8.dtype != torch.int8 or k8.dtype != torch.int8:
        raise H3AError(H3A_EDTYPE, f"q8/k8 must hold int8 codes, got {q8.dtype}/{k8.dtype}")
    if tuple(k8.shape) != (S, Hkv, D):
        raise H3AError(H3A_ESHAPE, f"k8 shape {tuple(k8.shape)} does not match q8 {tuple(q8.shape)}")
    cu = _i32_array(cu_seqlens)
    cols = vt_e4m3_columns(cu)
    nb = cols // 64
    _expect("vt8", vt8, (Hkv, D, max(cols, 1)), torch.uint8)
    qs = _f32_scales("q_scale", qs, (Hq, S), q8.device)
    ks = _f32_scales("k_scale", ks, (Hkv, max(nb, 1)), q8.device)
    vs = _scales("vt_scale", vs, (Hkv, max(cols, 64) // 64, 2, 32, D // 32), q8.device)
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=q8.device)
    _, _, _, so = _token_major("out", out)
    _same("out", out, (S, Hq, D), torch.bfloat16)
    _check(lib().h3a_varlen_attn_fwd_i8qk_fp8pv(q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), qs.data_ptr(),
                                                ks.data_ptr(), vs.data_ptr(), out.data_ptr(), S, Hq, Hkv, D, sq, sk,
                                                cols, so, _ptr_i32(cu), len(cu) - 1, float(scale),
                                                int(bool(causal)), _stream_handle(stream)))
    return out


def varlen_attn_fwd_ex(q, k, v, cu_seqlens, scale: float, causal: bool = False, out=None, stream=None,
                       _entry="h3a_varlen_attn_fwd_ex"):
    """Grouped-K/V (k, v: [S, Hkv, D], Hkv | Hq) and optionally causal per-segment attention."""
    import torch

    S, Hq, D, sq = _token_major("q", q)
    _, Hkv, _, sk = _token_major("k", k)
    _, _, _, sv = _token_major("v", v)
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (S, Hkv, D) or t.dtype != q.dtype:
            raise H3AError(H3A_ESHAPE, f"{name} shape/dtype {tuple(t.shape)}/{t.dtype} differs from "
                                       f"{(S, Hkv, D)}/{q.dtype}")
    if out is None:
        out = torch.empty((S, Hq, D), dtype=q.dtype, device=q.device)
    _, _, _, so = _token_major("out", out)
    _same("out", out, (S, Hq, D), q.dtype)
    cu = _i32_array(cu_seqlens)
    _check(getattr(lib(), _entry)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _dtype_code(q),
                                  S, Hq, Hkv, D, sq, sk, sv, so, _ptr_i32(cu), len(cu) - 1, float(scale),
                                  int(bool(causal)), _stream_handle(stream)))
    return out


def varlen_attn_fwd_noalloc(q, k, v, cu_seqlens, scale: float, out, causal: bool = False, stream=None):
    """varlen_attn_fwd_ex without device allocation: `out` must be given, and the
    tile plan goes into the library's fixed per-GPU array (at most 256 non-empty
    segments and 65,536 work items)."""
    return varlen_attn_fwd_ex(q, k, v, cu_seqlens, scale, causal=causal, out=out, stream=stream,
                              _entry="h3a_varlen_attn_fwd_noalloc")


def plan_tiles(cu_seqlens, heads: int, block_m: int, n_xcd: int, causal: bool = False) -> np.ndarray:
    """The attention tile plan as int32 [n, 4] rows (seg start, seg len, q start, head); host only."""
    cu = _i32_array(cu_seqlens)
    n = ctypes.c_int64(0)
    c = int(bool(causal))
    st = lib().h3a_plan_tiles_ex(_ptr_i32(cu), len(cu) - 1, heads, block_m, n_xcd, c, None, 0, ctypes.byref(n))
    if st not in (H3A_OK, H3A_ESHAPE):
        _check(st)
    out = np.zeros((max(n.value, 1), 4), dtype=np.int32)
    _check(lib().h3a_plan_tiles_ex(_ptr_i32(cu), len(cu) - 1, heads, block_m, n_xcd, c, _ptr_i32(out), n.value,
                                   ctypes.byref(n)))
    return out[:n.value]
