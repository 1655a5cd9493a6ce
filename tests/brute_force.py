"""Scalar brute-force attention used to pin the fp64 oracle on tiny inputs.

Written independently of `oracle/`: it walks the window by frame id (no
deques, no array slicing), numbers positions with a running counter, rotates
each (position, frequency) pair with `math.cos`/`math.sin`, and evaluates
every (query, key) score, mask and softmax with Python scalars.  It only
suits inputs with a few thousand (query, key) pairs.
"""
from __future__ import annotations

import math


def _rot(vec, pos, theta):
    """Rotate-half RoPE of one vector (list of floats) at integer position `pos`."""
    d = len(vec)
    h = d // 2
    out = [0.0] * d
    for i in range(h):
        a = pos * (theta ** (-(2.0 * i) / d))
        c, s = math.cos(a), math.sin(a)
        out[i] = vec[i] * c - vec[i + h] * s
        out[i + h] = vec[i + h] * c + vec[i] * s
    return out


def _attend_one(qvec, q_pos, keys, theta):
    """keys: list of (pos, kvec, vvec); returns the attention output vector."""
    d = len(qvec)
    qr = _rot(qvec, q_pos, theta)
    scores = []
    for (kp, kvec, _) in keys:
        if kp > q_pos:
            continue
        kr = _rot(kvec, kp, theta)
        scores.append((sum(qr[j] * kr[j] for j in range(d)) / math.sqrt(d), kp))
    m = max(s for s, _ in scores)
    w = {kp: math.exp(s - m) for s, kp in scores}
    z = sum(w.values())
    out = [0.0] * d
    for (kp, _, vvec) in keys:
        if kp in w:
            for j in range(d):
                out[j] += w[kp] / z * vvec[j]
    return out


def brute_stream(g, prefix_k, prefix_v, frame_kv, frame_q, t):
    """Outputs [V*T][Hq][D] for the new frame t of every view.

    frame_kv(view, frame) -> (k [T][Hkv][D], v); frame_q(view, frame) -> [T][Hq][D].
    The window holds, per view, frames t-F+1 .. t (oldest first), after a prefix.
    """
    group = g.n_q_heads // g.n_kv_heads
    keys_per_head = [[] for _ in range(g.n_kv_heads)]
    qpos_of = {}
    pos = g.pos_base
    for i in range(g.prefix_len):
        for h in range(g.n_kv_heads):
            keys_per_head[h].append((pos, [float(x) for x in prefix_k[i][h]],
                                     [float(x) for x in prefix_v[i][h]]))
        pos += 1
    for v in range(g.n_views):
        for fid in range(t - g.n_frames + 1, t + 1):
            k, vv = frame_kv(v, fid)
            for i in range(g.tok_per_frame):
                if fid == t:
                    qpos_of[(v, i)] = pos
                for h in range(g.n_kv_heads):
                    keys_per_head[h].append((pos, [float(x) for x in k[i][h]],
                                             [float(x) for x in vv[i][h]]))
                pos += 1
    out = []
    for v in range(g.n_views):
        q = frame_q(v, t)
        for i in range(g.tok_per_frame):
            row = []
            for h in range(g.n_q_heads):
                row.append(_attend_one([float(x) for x in q[i][h]], qpos_of[(v, i)],
                                       keys_per_head[h // group], g.rope_theta))
            out.append(row)
    return out


def brute_verify(g, prefix_k, prefix_v, frame_kv, t, k_tail, v_tail, q_blk, k_blk, v_blk):
    """Verify outputs [B][Hq][D]: block queries over window ++ tail ++ block, causal."""
    group = g.n_q_heads // g.n_kv_heads
    keys_per_head = [[] for _ in range(g.n_kv_heads)]
    pos = g.pos_base

    def add(k, vv, n):
        nonlocal pos
        for i in range(n):
            for h in range(g.n_kv_heads):
                keys_per_head[h].append((pos, [float(x) for x in k[i][h]],
                                         [float(x) for x in vv[i][h]]))
            pos += 1

    add(prefix_k, prefix_v, g.prefix_len)
    for v in range(g.n_views):
        for fid in range(t - g.n_frames + 1, t + 1):
            k, vv = frame_kv(v, fid)
            add(k, vv, g.tok_per_frame)
    add(k_tail, v_tail, len(k_tail))
    first_blk = pos
    add(k_blk, v_blk, len(k_blk))
    out = []
    for b in range(len(q_blk)):
        out.append([_attend_one([float(x) for x in q_blk[b][h]], first_blk + b,
                                keys_per_head[h // group], g.rope_theta)
                    for h in range(g.n_q_heads)])
    return out
