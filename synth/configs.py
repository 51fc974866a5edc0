"""Workload descriptions (segment grids, head geometry) and their seeded tensors.

Each workload is a packed sequence of segments; a segment is a (T, H, W) token
grid truncated to L tokens.  The shapes follow the requests the MiniMax H3 DiT
serves: a 864x480, 124-frame render with six reference images and an audio
track packed into S = 20,423 tokens (h3-spark model card, "Measured on one DGX
Spark"), 24 heads of 128 dims with rotary on the first 96.  The tensors are
synthetic: Q, K, V ~ N(0, 1) and the RMSNorm gains ~ 1 + N(0, 0.1).

Only descriptions and random draws live here.  The packing prefix sums, token
positions and everything downstream are computed separately by the oracle and
by the HIP library.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

from . import rng


@dataclass(frozen=True)
class Workload:
    name: str
    segments: tuple  # ((T, H, W, L), ...)
    heads: int
    head_dim: int
    rot_dims: tuple  # rotated dims owned by the t, h and w axes
    dtype: str  # "f32" or "bf16"
    base: float = 10000.0
    eps: float = 1e-6
    seed: int = 0
    gamma_mean: float = 1.0
    gamma_std: float = 0.1
    kv_heads: int = 0  # K/V heads (grouped-query attention); 0: as many as query heads
    causal: bool = False  # per-segment causal mask aligned at the segment start
    rope_mode: int = 0  # 0 grid, 1 linspace, 2 length-normalised, 3 interleaved (h3a_rope_mode)
    lin_start: tuple = (0.0, 0.0, 0.0)
    lin_stop: tuple = (0.0, 0.0, 0.0)
    note: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        return int(sum(s[3] for s in self.segments))

    @property
    def rot_dim(self) -> int:
        return int(sum(self.rot_dims))

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def lengths(self) -> list:
        return [int(s[3]) for s in self.segments]

    @property
    def kv(self) -> int:
        return self.kv_heads or self.heads

    def attention_flops(self) -> float:
        """QK^T plus PV multiply-adds at 2 flop each over the visible (query, key)
        pairs: 4 * D * heads * sum(L^2), or sum(L (L + 1) / 2) pairs when causal."""
        pairs = sum(L * (L + 1) // 2 if self.causal else L * L for L in self.lengths)
        return 4.0 * self.head_dim * self.heads * float(pairs)

    def with_segments(self, segments, name=None) -> "Workload":
        d = dict(self.__dict__)
        d["segments"] = tuple(tuple(int(v) for v in s) for s in segments)
        d["name"] = name or self.name
        return Workload(**d)

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def ragged_segments(seed: int, n: int = 64, lo: int = 128, hi: int = 2048, rows: int = 16):
    """n segments with integer lengths uniform in [lo, hi], each a 1 x rows x ceil(L/rows) grid."""
    u = rng.uniform(seed, rng.TAG_LENS, n)
    lens = lo + np.floor(u * (hi - lo + 1)).astype(np.int64)
    return tuple((1, rows, -(-int(L) // rows), int(L)) for L in lens)


def _h3_request(video_thw, ref_hw, audio_len):
    t, h, w = video_thw
    segs = [(t, h, w, t * h * w)]
    segs += [(1, ref_hw[0], ref_hw[1], ref_hw[0] * ref_hw[1])] * 6
    # 1-D audio track laid along the temporal axis (its h and w grids are 1).
    segs.append((audio_len, 1, 1, audio_len))
    return tuple(segs)


TINY_F32 = Workload(
    name="tiny_f32",
    segments=((1, 37, 1, 37), (1, 7, 13, 91)),
    heads=2, head_dim=64, rot_dims=(16, 16, 16), dtype="f32",
    note="2 segments [37, 91], 2 heads, D=64, rotary on 48 dims",
)

TWO_SEG = Workload(
    name="two_seg_bf16",
    segments=((4, 32, 32, 4096), (1, 32, 32, 1024)),
    heads=24, head_dim=128, rot_dims=(32, 32, 32), dtype="bf16",
    note="2 segments [4096, 1024]",
)

H3_S20423 = Workload(
    name="h3_s20423_bf16",
    segments=_h3_request((10, 30, 54), (20, 30), 623),
    heads=24, head_dim=128, rot_dims=(32, 32, 32), dtype="bf16",
    note="video 10x30x54 + 6 refs 20x30 + audio 623: S=20,423",
)

H3_S25103 = Workload(
    name="h3_s25103_bf16",
    segments=_h3_request((10, 34, 60), (20, 34), 623),
    heads=24, head_dim=128, rot_dims=(32, 32, 32), dtype="bf16",
    note="video 10x34x60 + 6 refs 20x34 + audio 623: S=25,103",
)

RAGGED64 = Workload(
    name="ragged64_bf16",
    segments=ragged_segments(0),
    heads=24, head_dim=128, rot_dims=(32, 32, 32), dtype="bf16",
    note="64 segments, L ~ U{128..2048}, 1x16xceil(L/16) grids",
)

ALL = {w.name: w for w in (TINY_F32, TWO_SEG, H3_S20423, H3_S25103, RAGGED64)}

# Other attention workloads of the same model family (parity cases of the
# other rotary table modes).  The video VAE's ViT3D decoder: 32 heads of 64,
# rotary on 0.75 of the head dim with theta 100 from length-normalised ids,
# q/k RMSNorm without a gain (video-VAE decoder commit), run per 16x16 latent
# tile (pipeline commit on tiling); three tiles of 4 latent frames are packed
# as segments, each followed by a suffix of 4 register tokens and a cls token
# (the suffix size is not given on the pages: 5 is this workload's choice).
VIT3D_TILES = Workload(
    name="vit3d_tiles_bf16",
    segments=((4, 16, 16, 1024 + 5),) * 3,
    heads=32, head_dim=64, rot_dims=(16, 16, 16), dtype="bf16", base=100.0,
    gamma_std=0.0, rope_mode=2,
    note="3 ViT3D tiles of 4x16x16 latents + 5 suffix tokens; 32 heads x 64; normalised ids",
)

# A packed prompt with M-RoPE's interleaved angles (three images as
# (1, h, w) grids and a text run along t), 16 heads of 128, all 128 dims
# rotated with Qwen-style shares (48, 40, 40) (encoder-tower commit,
# "M-RoPE"); attention per segment as everywhere here.
MROPE_PACKED = Workload(
    name="mrope_packed_bf16",
    segments=((1, 24, 36, 864), (1, 20, 30, 600), (1, 16, 16, 256), (300, 1, 1, 300)),
    heads=16, head_dim=128, rot_dims=(48, 40, 40), dtype="bf16", base=1000000.0,
    rope_mode=3,
    note="3 images + 300 text tokens, interleaved M-RoPE over all 128 dims",
)

MODE_WORKLOADS = {w.name: w for w in (VIT3D_TILES, MROPE_PACKED)}

# Causal grouped-query attention as in the encoder's text tower (per-head q/k
# RMSNorm, interleaved M-RoPE, causal GQA: encoder-tower commit).  Packed
# prompts of 2048, 1500, 500, 47 and 1 tokens as (L, 1, 1) grids; 32 query
# heads sharing 8 K/V heads of 128 dims.  Head counts and rotary base are this
# workload's choice (the pages give none for the tower).
CAUSAL_GQA_TEXT = Workload(
    name="causal_gqa_text_bf16",
    segments=tuple((L, 1, 1, L) for L in (2048, 1500, 500, 47, 1)),
    heads=32, kv_heads=8, causal=True, head_dim=128, rot_dims=(48, 40, 40), dtype="bf16", base=1000000.0,
    rope_mode=3,
    note="5 packed prompts (S=4096), 32 q heads / 8 kv heads, causal, interleaved M-RoPE",
)

CAUSAL_GQA_TINY_F32 = Workload(
    name="causal_gqa_tiny_f32",
    segments=((37, 1, 1, 37), (91, 1, 1, 91)),
    heads=4, kv_heads=2, causal=True, head_dim=64, rot_dims=(16, 16, 16), dtype="f32", base=10000.0,
    rope_mode=3,
    note="2 segments [37, 91], 4 q heads / 2 kv heads, causal, fp32",
)

CAUSAL_WORKLOADS = {w.name: w for w in (CAUSAL_GQA_TEXT, CAUSAL_GQA_TINY_F32)}

# The encoder's vision tower: non-causal attention over per-frame cu_seqlens of
# a ragged batch of two images with different h x w (vision-tower commit),
# with a 2-D (h, w) rotary: the grid table with no t share.  Frames: image A
# 4 x 24 x 36 patches, image B 2 x 20 x 30; 16 heads of 64 (this workload's
# choice; the pages give the tower's shapes only as reduced dimensions).
VISION_FRAMES = Workload(
    name="vision_frames_bf16",
    segments=((1, 24, 36, 864),) * 4 + ((1, 20, 30, 600),) * 2,
    heads=16, head_dim=64, rot_dims=(0, 16, 16), dtype="bf16", base=10000.0,
    note="per-frame segments of two ragged images (4 x 864, 2 x 600), 16 heads x 64, 2-D rotary",
)

# One long causal prompt with the text tower's head layout, large enough to
# time the causal kernel away from launch overhead.
CAUSAL_GQA_16K = CAUSAL_GQA_TEXT.replace(
    name="causal_gqa_16k_bf16", segments=((16384, 1, 1, 16384),),
    note="one 16,384-token causal prompt, 32 q heads / 8 kv heads, interleaved M-RoPE",
)

# One GPU's share of the S = 20,423 request when its 24 heads are spread over
# eight GPUs (head parallelism): 3 heads, the same packing.
H3_S20423_3H = H3_S20423.replace(name="h3_s20423_3heads_bf16", heads=3,
                                 note="S=20,423 packing, 3 of its 24 heads (one GPU of eight)")

# Every bf16 workload, by name (the benchmark can run any of them).
BF16 = {w.name: w for w in (TWO_SEG, H3_S20423, H3_S25103, RAGGED64, VIT3D_TILES, MROPE_PACKED, CAUSAL_GQA_TEXT,
                            CAUSAL_GQA_16K, VISION_FRAMES, H3_S20423_3H)}

# The configuration the headline throughput is quoted on.
HEADLINE = H3_S20423


@dataclass
class Tensors:
    """Seeded inputs of one workload.  Floating tensors are [S, heads, D].

    For bf16 workloads ``q``, ``k``, ``v`` hold uint16 bit patterns; gains are
    always fp32 [D].
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    gamma_q: np.ndarray
    gamma_k: np.ndarray


def make_tensors(w: Workload, with_v: bool = True) -> Tensors:
    shape = (w.tokens, w.heads, w.head_dim)
    kv_shape = (w.tokens, w.kv, w.head_dim)
    q = rng.normal_tensor(w.seed, rng.TAG_Q, shape, w.dtype)
    k = rng.normal_tensor(w.seed, rng.TAG_K, kv_shape, w.dtype)
    v = rng.normal_tensor(w.seed, rng.TAG_V, kv_shape, w.dtype) if with_v else None
    gq = rng.normal_tensor(w.seed, rng.TAG_GAMMA_Q, (w.head_dim,), "f32", w.gamma_mean, w.gamma_std)
    gk = rng.normal_tensor(w.seed, rng.TAG_GAMMA_K, (w.head_dim,), "f32", w.gamma_mean, w.gamma_std)
    return Tensors(q, k, v, gq, gk)
