"""Seeded synthetic inputs and the five workload geometries.

This module is shared by the fp64 oracle and by the HIP path.  It holds no
arithmetic of the attention method itself: only shapes, seeds, random draws
and the rounding of those draws to the storage dtype.  Both sides regenerate
any tensor independently from (config, layer, kind, view, frame).

Workloads (synthetic stand-ins for the multi-camera driving clips the
FlashDrive pages measure on, which are not available here):

  1  tiny fp32 step      V=2 F=4 T=16  P=8    Hq/Hkv/D = 4/2/64    theta 1e4
  2  small bf16 step     V=4 F=4 T=64  P=64   Hq/Hkv/D = 8/2/128   theta 1e6, values x0.5
  3  backbone prefill    V=4 F=4 T=256 P=512  Hq/Hkv/D = 32/8/128  theta 1e6, 36 layers
  4  8-token verify      config-3 window + 200 reasoning rows + 8-row block, 36 layers
  5  rolling stream      V=4 F=8 T=256 P=512  Hq/Hkv/D = 32/8/128  100 windows,
                         K/V with 1 % outliers at +-8 sigma

A view-major window has F frames per camera view (FlashDrive technical
summary, Methodology section 1, "Token Layout"); every window inserts one new
frame per view.  Values are N(0, 1) draws scaled by `scale`, rounded to the
storage dtype (round-to-nearest-even for bf16).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

F32 = "f32"
BF16 = "bf16"

# Tensor kinds; the integer is part of the seed.
KIND = {
    "Kp": 0, "Vp": 1,          # text prefix K/V            [P][Hkv][D]
    "K": 2, "V": 3,            # per-frame K/V (pre-RoPE)   [T][Hkv][D]
    "Q": 4,                    # per-frame queries          [T][Hq][D]
    "Ktail": 5, "Vtail": 6,    # reasoning-token K/V        [R][Hkv][D]
    "Qblk": 7, "Kblk": 8, "Vblk": 9,  # verify block        [B][H*][D]
    "Qpre": 10,                # prefix-token queries (full-window tests only)
    "Xh": 11,                  # hidden states of a frame's tokens [T][hidden] (projection only)
    "Wkv": 12,                 # K and V projection weights [2*Hkv*D][hidden] (projection only)
}


@dataclass(frozen=True)
class Geometry:
    """Shape of one attention layer's streaming window (all sizes in tokens)."""
    n_views: int
    n_frames: int
    tok_per_frame: int
    prefix_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    tail_cap: int
    rope_theta: float
    pos_base: int = 0
    dtype: str = BF16

    @property
    def window(self) -> int:
        """N = P + V*F*T keys in one window."""
        return self.prefix_len + self.n_views * self.n_frames * self.tok_per_frame

    @property
    def cache_rows(self) -> int:
        """Rows of one head's K (or V) cache: window + tail capacity."""
        return self.window + self.tail_cap

    @property
    def n_new(self) -> int:
        """New-frame query tokens per window (one frame per view)."""
        return self.n_views * self.tok_per_frame

    def replace(self, **kw) -> "Geometry":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    geom: Geometry
    scale: float = 1.0
    outlier_frac: float = 0.0
    outlier_sigma: float = 8.0
    layers: int = 1
    # first newest-frame index at which attention runs, and how many windows
    first_t: int = 4
    windows: int = 1
    # verify only
    n_tail: int = 0
    blk_len: int = 0


CONFIGS: dict[int, Workload] = {
    1: Workload(1, "tiny fp32 streaming step",
                Geometry(2, 4, 16, 8, 4, 2, 64, 32, 1e4, dtype=F32),
                first_t=4, windows=1),
    2: Workload(2, "small bf16 streaming step",
                Geometry(4, 4, 64, 64, 8, 2, 128, 64, 1e6, dtype=BF16),
                scale=0.5, first_t=4, windows=1),
    3: Workload(3, "backbone streaming prefill x36 layers",
                Geometry(4, 4, 256, 512, 32, 8, 128, 256, 1e6, dtype=BF16),
                layers=36, first_t=4, windows=1),
    4: Workload(4, "8-token speculative verify x36 layers",
                Geometry(4, 4, 256, 512, 32, 8, 128, 256, 1e6, dtype=BF16),
                layers=36, first_t=4, windows=1, n_tail=200, blk_len=8),
    5: Workload(5, "long rolling stream, 100 windows, 1% 8-sigma K/V outliers",
                Geometry(4, 8, 256, 512, 32, 8, 128, 256, 1e6, dtype=BF16),
                outlier_frac=0.01, outlier_sigma=8.0, first_t=8, windows=100),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _rng(cfg_id: int, layer: int, kind: str, view: int, frame: int) -> np.random.Generator:
    ss = np.random.SeedSequence([cfg_id, layer, KIND[kind], view + 1, frame + 1])
    return np.random.default_rng(ss)


def draw(w: Workload, layer: int, kind: str, view: int, frame: int, shape) -> np.ndarray:
    """One seeded tensor: N(0,1)*scale (+ outliers on K/V kinds), rounded to the dtype.

    `view`/`frame` are -1 where they do not apply (prefix, tail, block).
    Returned as float32; with dtype bf16 every value is exactly a bfloat16.
    """
    rng = _rng(w.cfg_id, layer, kind, view, frame)
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(w.scale)
    if w.outlier_frac > 0 and kind in ("Kp", "Vp", "K", "V", "Ktail", "Vtail", "Kblk", "Vblk"):
        hit = rng.random(shape) < w.outlier_frac
        sign = np.where(rng.random(shape) < 0.5, -1.0, 1.0).astype(np.float32)
        x = np.where(hit, sign * np.float32(w.outlier_sigma * w.scale), x).astype(np.float32)
    if w.geom.dtype == BF16:
        x = round_bf16(x)
    return x


# Convenience accessors with the tensor layouts used everywhere.
def prefix_kv(w: Workload, layer: int):
    g = w.geom
    sh = (g.prefix_len, g.n_kv_heads, g.head_dim)
    return draw(w, layer, "Kp", -1, -1, sh), draw(w, layer, "Vp", -1, -1, sh)


def frame_kv(w: Workload, layer: int, view: int, frame: int):
    g = w.geom
    sh = (g.tok_per_frame, g.n_kv_heads, g.head_dim)
    return draw(w, layer, "K", view, frame, sh), draw(w, layer, "V", view, frame, sh)


def frame_q(w: Workload, layer: int, view: int, frame: int):
    g = w.geom
    return draw(w, layer, "Q", view, frame, (g.tok_per_frame, g.n_q_heads, g.head_dim))


def prefix_q(w: Workload, layer: int):
    g = w.geom
    return draw(w, layer, "Qpre", -1, -1, (g.prefix_len, g.n_q_heads, g.head_dim))


def tail_kv(w: Workload, layer: int, n_tail: int):
    g = w.geom
    sh = (n_tail, g.n_kv_heads, g.head_dim)
    return draw(w, layer, "Ktail", -1, -1, sh), draw(w, layer, "Vtail", -1, -1, sh)


def block_qkv(w: Workload, layer: int, blk_len: int):
    g = w.geom
    return (draw(w, layer, "Qblk", -1, -1, (blk_len, g.n_q_heads, g.head_dim)),
            draw(w, layer, "Kblk", -1, -1, (blk_len, g.n_kv_heads, g.head_dim)),
            draw(w, layer, "Vblk", -1, -1, (blk_len, g.n_kv_heads, g.head_dim)))


def frame_hidden(w: Workload, layer: int, view: int, frame: int, hidden: int):
    """Hidden states [T][hidden] of one frame's tokens (inputs of the K/V projection)."""
    return draw(w, layer, "Xh", view, frame, (w.geom.tok_per_frame, hidden))


def kv_weights(w: Workload, layer: int, hidden: int):
    """K then V projection weights [2*Hkv*D][hidden] (one output feature per row, as a linear
    layer stores them), N(0, 1/hidden) so that projected values are about unit scale."""
    g = w.geom
    rng = _rng(w.cfg_id, layer, "Wkv", -1, -1)
    x = rng.standard_normal((2 * g.n_kv_heads * g.head_dim, hidden), dtype=np.float32) * np.float32(
        1.0 / np.sqrt(hidden))
    return round_bf16(x) if g.dtype == BF16 else x


def new_frames(w: Workload, layer: int, frame: int):
    """K, V [V][T][Hkv][D] and Q [V*T][Hq][D] of frame index `frame` for every view."""
    ks, vs, qs = [], [], []
    for v in range(w.geom.n_views):
        k, vv = frame_kv(w, layer, v, frame)
        ks.append(k)
        vs.append(vv)
        qs.append(frame_q(w, layer, v, frame))
    return np.stack(ks), np.stack(vs), np.concatenate(qs, axis=0)
