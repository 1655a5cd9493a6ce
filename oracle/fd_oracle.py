"""Plain fp64 reference for the streaming-prefill attention hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP path never
imports this module and shares no code with it; the two meet only through
the seeded generators in `streaming_kv_cache_view_amd.synth`.

What is computed, and where the pages state it:

* Streaming window.  Only the newest frame of every camera view is prefilled;
  the K/V of the earlier frames are reused from the previous window
  (FlashDrive README, technique list, "Streaming inference"; FlashDrive
  technical summary, Methodology section 1, "Algorithmic Shortcut").
* View-major layout.  Tokens are grouped per camera view; the new frame goes
  to the end of its own view's segment, not to the end of the whole sequence
  (technical summary, Methodology section 1, "Token Layout").
* Streaming mask.  Cross-view causality is kept: read here as plain causality
  over the logical view-major order, key position <= query position (same
  passage).
* Positions.  Keys are kept before rotary embedding and are rotated when
  used, at the position they hold in the *current* window (technical
  summary, Methodology section 1, "Positional Encoding"; romaanj review,
  "Method").  RoPE is the standard rotate-half form with inverse frequency
  theta^(-2i/D).
* Verify.  The target checks a draft block of 8 tokens in one forward pass
  (README technique list, "Speculative reasoning"; technical summary,
  Methodology section 2): the block attends to the window, the reasoning
  tokens before it, and itself causally.

Readings where the pages are silent (text prefix first and static, causal
mask inside the new frame, GQA head h -> kv head h // (Hq/Hkv), 1/sqrt(D)
scale) are the plainest ones consistent with the above; they are listed with
their reasons in the design notes.

Algorithm, in the pages' order: keep per view the last F frames (a deque, no
ring arithmetic), lay out the logical window, rotate *every* key and query in
fp64 at its logical position, build an explicit boolean mask from positions,
and run dense masked softmax attention.
"""
from __future__ import annotations

from collections import deque

import numpy as np


# ----------------------------------------------------------------------------
# Rotary position embedding (technical summary, Methodology 1, "Positional Encoding")
# ----------------------------------------------------------------------------
def inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Standard RoPE inverse frequencies theta^(-2i/D), i = 0 .. D/2-1, in fp64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / head_dim)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE in fp64.

    x: [n, H, D] (or [n, D]); pos: [n] integer absolute positions.
    For pair (x1_i, x2_i) = (x[i], x[i + D/2]) and angle a = pos * inv_freq_i:
        y1 = x1 cos a - x2 sin a,   y2 = x2 cos a + x1 sin a.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq(d, theta)[None, :]   # [n, D/2]
    c, s = np.cos(ang), np.sin(ang)
    if x.ndim == 3:
        c, s = c[:, None, :], s[:, None, :]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ----------------------------------------------------------------------------
# The logical view-major window (technical summary, Methodology 1, "Token Layout")
# ----------------------------------------------------------------------------
class StreamWindow:
    """The logical window of one layer: static prefix + the last F frames per view.

    Frames are appended per view; the deque drops the oldest one.  The window
    is prefix ++ view 0 (oldest..newest) ++ view 1 ++ ... ++ view V-1.
    """

    def __init__(self, geom, prefix_k, prefix_v):
        self.g = geom
        self.prefix_k = np.asarray(prefix_k, np.float64)
        self.prefix_v = np.asarray(prefix_v, np.float64)
        self.frames = [deque(maxlen=geom.n_frames) for _ in range(geom.n_views)]
        self.frame_ids = [deque(maxlen=geom.n_frames) for _ in range(geom.n_views)]

    def push(self, view: int, frame_id: int, k, v):
        """Append frame `frame_id` of `view`: it becomes the newest entry of that view."""
        self.frames[view].append((np.asarray(k, np.float64), np.asarray(v, np.float64)))
        self.frame_ids[view].append(frame_id)

    def full(self) -> bool:
        return all(len(d) == self.g.n_frames for d in self.frames)

    def kv(self):
        """K, V [N][Hkv][D] in logical order."""
        ks = [self.prefix_k] + [k for d in self.frames for (k, _) in d]
        vs = [self.prefix_v] + [v for d in self.frames for (_, v) in d]
        return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def window_positions(geom, n_keys: int) -> np.ndarray:
    """Position of logical element n is pos_base + n (positions follow the current layout)."""
    return np.int64(geom.pos_base) + np.arange(n_keys, dtype=np.int64)


def new_query_positions(geom) -> np.ndarray:
    """Positions of the new frame's tokens: the last frame slot of each view's segment."""
    g = geom
    v = np.repeat(np.arange(g.n_views, dtype=np.int64), g.tok_per_frame)
    i = np.tile(np.arange(g.tok_per_frame, dtype=np.int64), g.n_views)
    return np.int64(g.pos_base) + g.prefix_len + (v * g.n_frames + g.n_frames - 1) * g.tok_per_frame + i


# ----------------------------------------------------------------------------
# Dense masked attention with GQA
# ----------------------------------------------------------------------------
def attend(q, k, v, q_pos, k_pos, theta) -> np.ndarray:
    """softmax((R q)(R k)^T / sqrt(D) masked by k_pos <= q_pos) V, per query head.

    q: [Nq][Hq][D] pre-RoPE; k, v: [N][Hkv][D] (k pre-RoPE); positions int64.
    Query head h reads kv head h // (Hq / Hkv).  Returns fp64 [Nq][Hq][D].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    nq, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    qr = rope(q, q_pos, theta)
    kr = rope(k, k_pos, theta)
    mask = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]          # [Nq][N]
    out = np.empty((nq, hq, d), np.float64)
    for h in range(hq):
        kv = h // group
        s = (qr[:, h, :] @ kr[:, kv, :].T) / np.sqrt(d)
        s = np.where(mask, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, kv, :]
    return out


def oracle_stream(geom, window: StreamWindow, q_new) -> np.ndarray:
    """Streaming-prefill output for the new frame of every view.

    q_new: [V*T][Hq][D], view-major (row v*T + i is token i of view v's new frame).
    The window must already hold the new frame as the newest entry of each view.
    """
    assert window.full()
    k, v = window.kv()
    return attend(q_new, k, v, new_query_positions(geom), window_positions(geom, k.shape[0]),
                  geom.rope_theta)


def oracle_full_window(geom, window: StreamWindow, q_window) -> np.ndarray:
    """Non-streaming (cold-start) prefill: every token of the window is a query.

    The first window of a stream has no previous window to reuse, so all of it is
    prefilled (README technique list, "Streaming inference": the streaming path prefills
    the newest frame only, reusing the rest); the same mask applies, key position <= query
    position over the logical view-major order.  q_window: [N][Hq][D] in logical order
    (prefix, then view 0 oldest..newest, view 1, ...).  Returns fp64 [N][Hq][D].
    """
    assert window.full()
    k, v = window.kv()
    pos = window_positions(geom, k.shape[0])
    return attend(q_window, k, v, pos, pos, geom.rope_theta)


def oracle_verify(geom, window: StreamWindow, k_tail, v_tail, q_blk, k_blk, v_blk) -> np.ndarray:
    """Verify attention: block queries over window ++ reasoning tail ++ block (causal).

    Tail row r sits at position pos_base + N + r; block token b at pos_base + N + R + b.
    """
    assert window.full()
    k, v = window.kv()
    n = k.shape[0]
    r = np.asarray(k_tail).shape[0]
    b = np.asarray(q_blk).shape[0]
    k_all = np.concatenate([k, np.asarray(k_tail, np.float64), np.asarray(k_blk, np.float64)])
    v_all = np.concatenate([v, np.asarray(v_tail, np.float64), np.asarray(v_blk, np.float64)])
    k_pos = window_positions(geom, n + r + b)
    q_pos = np.int64(geom.pos_base) + n + r + np.arange(b, dtype=np.int64)
    return attend(q_blk, k_all, v_all, q_pos, k_pos, geom.rope_theta)


# ----------------------------------------------------------------------------
# K/V projection of a new frame (Technical Summary, "5. System Optimizations", "Kernel
# Fusion": the Q, K, V projections are merged into single kernels; README, "System
# optimizations": static KV cache).  The projected keys are what the cache stores, before
# rotary embedding (Methodology 1, "Positional Encoding").
# ----------------------------------------------------------------------------
def oracle_kv_projection(x, w_kv, n_kv_heads: int, head_dim: int):
    """K, V [T][Hkv][D] = x [T][hidden] times the K and V weights.

    w_kv: [2*Hkv*D][hidden], one output feature per row: rows [0, Hkv*D) give K (feature
    h*D + d is head h, dimension d), the next Hkv*D rows give V.  fp64, pre-RoPE.
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w_kv, np.float64)
    n = n_kv_heads * head_dim
    k = x @ w[:n].T
    v = x @ w[n: 2 * n].T
    t = x.shape[0]
    return k.reshape(t, n_kv_heads, head_dim), v.reshape(t, n_kv_heads, head_dim)


# ----------------------------------------------------------------------------
# The physical cache image after in-order inserts (bit-exact expectation)
# ----------------------------------------------------------------------------
def expected_ring_rows(geom, newest_frame: int):
    """Which frame each physical slot holds once frames .. newest_frame were inserted.

    A frame is stored at the end of its view's segment; physically each view
    owns F frame slots and frame g sits in slot g mod F.  Returns
    frame_of_slot[s] = newest_frame - ((newest_frame - s) mod F), for s < F.
    """
    f = geom.n_frames
    t = int(newest_frame)
    return [t - ((t - s) % f) for s in range(f)]


def expected_cache(geom, prefix, frame_of, newest_frame: int, fill=np.nan):
    """Expected K (or V) cache [Hkv][S_cap][D] for one layer.

    prefix: [P][Hkv][D]; frame_of(view, frame_id) -> [T][Hkv][D].  Rows outside
    the prefix and the view slots (the tail) are `fill`.
    Row layout: [0,P) prefix | P + (v*F + s)*T + i : token i of the frame in slot s of view v.
    """
    g = geom
    out = np.full((g.n_kv_heads, g.cache_rows, g.head_dim), fill, dtype=np.float64)
    out[:, : g.prefix_len, :] = np.transpose(np.asarray(prefix, np.float64), (1, 0, 2))
    slots = expected_ring_rows(g, newest_frame)
    for v in range(g.n_views):
        for s, fid in enumerate(slots):
            if fid < 0:
                continue
            r0 = g.prefix_len + (v * g.n_frames + s) * g.tok_per_frame
            out[:, r0: r0 + g.tok_per_frame, :] = np.transpose(np.asarray(frame_of(v, fid), np.float64),
                                                                (1, 0, 2))
    return out


# ----------------------------------------------------------------------------
# Whole-workload driver used by tests and the CPU baseline
# ----------------------------------------------------------------------------
def run_stream_workload(workload, layer: int, t_values, synth):
    """Yield (t, fp64 output) for every window t of a streaming workload.

    The window first receives frames 0..F-1 (the warm-up prefill), then one
    new frame per view per window; attention runs for each t in t_values.
    """
    g = workload.geom
    pk, pv = synth.prefix_kv(workload, layer)
    win = StreamWindow(g, pk, pv)
    t_values = list(t_values)
    last = max(t_values)
    for t in range(last + 1):
        for v in range(g.n_views):
            k, vv = synth.frame_kv(workload, layer, v, t)
            win.push(v, t, k, vv)
        if t in t_values:
            q = np.concatenate([synth.frame_q(workload, layer, v, t) for v in range(g.n_views)])
            yield t, oracle_stream(g, win, q)
