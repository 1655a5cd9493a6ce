"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each `pin_*` function raises AssertionError when the oracle disagrees with
  * a closed form (RoPE values, constant-V rows, a dominant logit),
  * brute force on tiny inputs (`brute_force.py`, independent scalar code),
  * a library routine in a special case (torch SDPA in fp64, plain causal
    attention when there is one view or when every token is a query),
  * an invariant (RoPE shift invariance, mask leak, norm preservation),
  * an explicit simulation (ring-slot occupancy after in-order inserts).
They look the oracle up at call time (`fd_oracle.<name>`), so the mutation
test can plant a mistake in the oracle and check that some pin fails.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle.fd_oracle as fd_oracle
from streaming_kv_cache_view_amd import synth
from streaming_kv_cache_view_amd.synth import Geometry, Workload

try:
    from . import brute_force
except ImportError:  # collected as a top-level module
    import brute_force


# Small geometries: several views / frames / heads, ragged sizes, both GQA groupings.
TINY = Workload(101, "tiny pin", Geometry(3, 3, 5, 3, 4, 2, 8, 16, 100.0, dtype=synth.F32),
                first_t=4)
TINY_G4 = Workload(102, "tiny pin G=4", Geometry(2, 2, 3, 2, 4, 1, 4, 8, 10.0, dtype=synth.F32),
                   first_t=3)


def _window_at(w, t, layer=0):
    g = w.geom
    pk, pv = synth.prefix_kv(w, layer)
    win = fd_oracle.StreamWindow(g, pk, pv)
    for fid in range(t + 1):
        for v in range(g.n_views):
            k, vv = synth.frame_kv(w, layer, v, fid)
            win.push(v, fid, k, vv)
    return win


def _q_new(w, t, layer=0):
    return np.concatenate([synth.frame_q(w, layer, v, t) for v in range(w.geom.n_views)])


def _stream(w, t, layer=0):
    return fd_oracle.oracle_stream(w.geom, _window_at(w, t, layer), _q_new(w, t, layer))


# ----------------------------------------------------------------------------
def pin_rope_closed_form():
    """D=4, theta=100: inverse frequencies 1 and 0.1; unit vectors rotate by p and 0.1 p."""
    x = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0], [0.0, 0.0, 1.0, 0.0]])
    y = fd_oracle.rope(x, np.array([1, 2, 1]), 100.0)
    c1, s1 = 0.5403023058681398, 0.8414709848078965      # cos 1, sin 1
    c2, s2 = 0.9800665778412416, 0.19866933079506122     # cos 0.2, sin 0.2
    want = np.array([[c1, 0.0, s1, 0.0], [0.0, c2, 0.0, s2], [-s1, 0.0, c1, 0.0]])
    assert np.allclose(y, want, rtol=0, atol=1e-15), (y, want)


def pin_rope_group_properties():
    """R_0 = I, |R_p x| = |x|, and <R_a x, R_b y> = <x, R_(b-a) y>."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 16))
    y = rng.standard_normal((5, 16))
    assert np.array_equal(fd_oracle.rope(x, np.zeros(5, np.int64), 1e4), x)
    p = np.array([0, 3, 17, 1000, 2 ** 20])
    assert np.allclose(np.linalg.norm(fd_oracle.rope(x, p, 1e4), axis=1),
                       np.linalg.norm(x, axis=1), rtol=1e-14)
    a = np.array([5, 9, 123, 4000, 77])
    b = np.array([2, 30, 123, 4100, 2 ** 20])
    lhs = np.sum(fd_oracle.rope(x, a, 1e4) * fd_oracle.rope(y, b, 1e4), axis=1)
    rhs = np.sum(x * fd_oracle.rope(y, b - a, 1e4), axis=1)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-9), (lhs, rhs)


def pin_brute_force_stream():
    """Oracle streaming output equals scalar brute force (config-1 and two tiny geometries)."""
    for w in (synth.CONFIGS[1], TINY, TINY_G4):
        g, t = w.geom, w.first_t
        pk, pv = synth.prefix_kv(w, 0)
        bf = brute_force.brute_stream(
            g, pk, pv, lambda v, f: synth.frame_kv(w, 0, v, f),
            lambda v, f: synth.frame_q(w, 0, v, f), t)
        got = _stream(w, t)
        err = np.max(np.abs(got - np.array(bf)))
        assert err <= 1e-12, (w.name, err)


def pin_brute_force_verify():
    """Oracle verify output equals scalar brute force."""
    for w, r, b in ((TINY, 4, 3), (TINY_G4, 0, 2), (synth.CONFIGS[1], 5, 8)):
        g, t = w.geom, w.first_t
        pk, pv = synth.prefix_kv(w, 0)
        kt, vt = synth.tail_kv(w, 0, r)
        qb, kb, vb = synth.block_qkv(w, 0, b)
        bf = brute_force.brute_verify(g, pk, pv, lambda v, f: synth.frame_kv(w, 0, v, f), t,
                                      kt, vt, qb, kb, vb)
        got = fd_oracle.oracle_verify(g, _window_at(w, t), kt, vt, qb, kb, vb)
        err = np.max(np.abs(got - np.array(bf)))
        assert err <= 1e-12, (w.name, err)


def pin_shift_invariance():
    """Shifting every position by the same amount leaves the output unchanged.

    Up to 2^20 the fp64 angles are exact to ~1e-10 rad, so the bound is 1e-9.  At the largest
    base the C ABI admits (last cache row at 2^31 - 1) an fp64 angle pos * inv_freq carries an
    absolute rounding error up to 2^31 * 2^-53 = 2^-22 rad, which moves each rotated element by
    at most that relative amount; 1e-5 bounds the resulting output change with a wide margin.
    """
    w = TINY
    ref = _stream(w, w.first_t)
    top = 2 ** 31 - w.geom.cache_rows - 1
    for c, bound in ((1, 1e-9), (1000, 1e-9), (2 ** 20, 1e-9), (top, 1e-5)):
        w2 = Workload(w.cfg_id, w.name, w.geom.replace(pos_base=c), first_t=w.first_t)
        err = np.max(np.abs(_stream(w2, w.first_t) - ref))
        assert err <= bound, (c, err)


def _sdpa(qr, kr, v, mask=None, causal=False):
    """torch SDPA in fp64 on CPU; q/k/v [N][H][D] with K/V heads repeated for GQA."""
    hq, hkv = qr.shape[1], kr.shape[1]
    k = np.repeat(kr, hq // hkv, axis=1)
    vv = np.repeat(v, hq // hkv, axis=1)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(np.transpose(a, (1, 0, 2))))
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(t(qr), t(k), t(vv), attn_mask=m,
                                                         is_causal=causal)
    return np.transpose(o.numpy(), (1, 0, 2))


def pin_sdpa_special_case():
    """Rotate in fp64, then torch SDPA (fp64, CPU) with the explicit view-major causal mask."""
    for w in (synth.CONFIGS[1], TINY):
        g, t = w.geom, w.first_t
        win = _window_at(w, t)
        k, v = win.kv()
        kpos = g.pos_base + np.arange(k.shape[0])
        qpos = []
        for vi in range(g.n_views):
            for i in range(g.tok_per_frame):
                qpos.append(g.pos_base + g.prefix_len + (vi * g.n_frames + g.n_frames - 1)
                            * g.tok_per_frame + i)
        qpos = np.array(qpos)
        mask = kpos[None, :] <= qpos[:, None]
        want = _sdpa(fd_oracle.rope(_q_new(w, t), qpos, g.rope_theta),
                     fd_oracle.rope(k, kpos, g.rope_theta), v, mask=mask)
        err = np.max(np.abs(_stream(w, t) - want))
        assert err <= 1e-12, (w.name, err)


def _full_window_direct(w, t, layer=0):
    """K, V and per-token Q of the window at t, built straight from frame ids."""
    g = w.geom
    pk, pv = synth.prefix_kv(w, layer)
    ks, vs, qs = [pk], [pv], [synth.prefix_q(w, layer)]
    for v in range(g.n_views):
        for fid in range(t - g.n_frames + 1, t + 1):
            k, vv = synth.frame_kv(w, layer, v, fid)
            ks.append(k)
            vs.append(vv)
            qs.append(synth.frame_q(w, layer, v, fid))
    return (np.concatenate(ks).astype(np.float64), np.concatenate(vs).astype(np.float64),
            np.concatenate(qs).astype(np.float64))


def pin_streaming_equals_full_recompute():
    """Streaming output == the new-frame rows of plain causal attention over the whole window.

    The non-streaming side recomputes every token of the window as a query
    with torch SDPA (is_causal), from frames looked up by id; no deque, no mask
    construction, no query-position formula is shared with the oracle.
    """
    for w in (synth.CONFIGS[1], TINY, TINY_G4):
        g, t = w.geom, w.first_t
        k, v, q = _full_window_direct(w, t)
        pos = g.pos_base + np.arange(k.shape[0])
        full = _sdpa(fd_oracle.rope(q, pos, g.rope_theta), fd_oracle.rope(k, pos, g.rope_theta),
                     v, causal=True)
        rows = []
        for vi in range(g.n_views):
            start = g.prefix_len + (vi * g.n_frames + g.n_frames - 1) * g.tok_per_frame
            rows.extend(range(start, start + g.tok_per_frame))
        err = np.max(np.abs(_stream(w, t) - full[rows]))
        assert err <= 1e-12, (w.name, err)


def pin_full_window_is_sdpa_causal():
    """Cold-start prefill == torch SDPA (is_causal) over the whole window, every row; and its
    newest-frame rows are the streaming output.  The window and its queries are built
    straight from frame ids (no deque), the positions are 0..N-1 + pos_base."""
    for w in (synth.CONFIGS[1], TINY, TINY_G4):
        g, t = w.geom, w.first_t
        k, v, q = _full_window_direct(w, t)
        got = fd_oracle.oracle_full_window(g, _window_at(w, t), q)
        pos = g.pos_base + np.arange(k.shape[0])
        full = _sdpa(fd_oracle.rope(q, pos, g.rope_theta), fd_oracle.rope(k, pos, g.rope_theta),
                     v, causal=True)
        assert np.max(np.abs(got - full)) <= 1e-12, w.name
        rows = []
        for vi in range(g.n_views):
            start = g.prefix_len + (vi * g.n_frames + g.n_frames - 1) * g.tok_per_frame
            rows.extend(range(start, start + g.tok_per_frame))
        assert np.max(np.abs(got[rows] - _stream(w, t))) <= 1e-12, w.name
        # the prefix rows only see the prefix: causal attention over the prefix alone
        P = g.prefix_len
        if P:
            pre = _sdpa(fd_oracle.rope(q[:P], pos[:P], g.rope_theta), fd_oracle.rope(k[:P], pos[:P], g.rope_theta),
                        v[:P], causal=True)
            assert np.max(np.abs(got[:P] - pre)) <= 1e-12, w.name


def pin_single_view_is_plain_causal():
    """With one view the streaming mask is plain causal attention; queries are the last T tokens."""
    w = Workload(103, "one view", Geometry(1, 3, 6, 4, 2, 1, 8, 8, 50.0, dtype=synth.F32),
                 first_t=5)
    g, t = w.geom, w.first_t
    k, v, q = _full_window_direct(w, t)
    pos = g.pos_base + np.arange(k.shape[0])
    full = _sdpa(fd_oracle.rope(q, pos, g.rope_theta), fd_oracle.rope(k, pos, g.rope_theta),
                 v, causal=True)
    err = np.max(np.abs(_stream(w, t) - full[-g.tok_per_frame:]))
    assert err <= 1e-12, err


def pin_closed_forms():
    """Constant V rows give that row; one dominant logit gives that key's V row."""
    g = TINY.geom
    n = g.window
    rng = np.random.default_rng(3)
    q = rng.standard_normal((g.n_new, g.n_q_heads, g.head_dim))
    k = rng.standard_normal((n, g.n_kv_heads, g.head_dim))
    row = rng.standard_normal((g.n_kv_heads, g.head_dim))
    v = np.broadcast_to(row, (n, g.n_kv_heads, g.head_dim)).copy()
    qpos = fd_oracle.new_query_positions(g)
    kpos = fd_oracle.window_positions(g, n)
    out = fd_oracle.attend(q, k, v, qpos, kpos, g.rope_theta)
    group = g.n_q_heads // g.n_kv_heads
    for h in range(g.n_q_heads):
        assert np.allclose(out[:, h, :], row[h // group], rtol=0, atol=1e-13)
    # dominant logit: the prefix key 0 is visible to every query; make it the only large score
    k = np.zeros((n, g.n_kv_heads, g.head_dim))
    v = rng.standard_normal((n, g.n_kv_heads, g.head_dim))
    e0 = np.zeros(g.head_dim)
    e0[0] = 1.0
    k[0, :, :] = 60.0 * e0
    # pre-rotate q so that R_{p_q} q = R_{p_0} e0 (score = 60*|e0|^2/sqrt(D))
    qv = fd_oracle.rope(np.broadcast_to(e0, (g.n_new, g.head_dim)).copy(),
                        kpos[0] - qpos, g.rope_theta)
    q = np.repeat(qv[:, None, :], g.n_q_heads, axis=1) * 10.0
    out = fd_oracle.attend(q, k, v, qpos, kpos, g.rope_theta)
    for h in range(g.n_q_heads):
        assert np.allclose(out[:, h, :], v[0, h // group], rtol=0, atol=1e-12)


def pin_mask_leak():
    """Keys after a query's position (later views) do not affect it: bit-identical output."""
    w = TINY
    g, t = w.geom, w.first_t
    win = _window_at(w, t)
    k, v = win.kv()
    q = _q_new(w, t)
    qpos = fd_oracle.new_query_positions(g)
    kpos = fd_oracle.window_positions(g, k.shape[0])
    base = fd_oracle.attend(q, k, v, qpos, kpos, g.rope_theta)
    last_view_start = g.prefix_len + (g.n_views - 1) * g.n_frames * g.tok_per_frame
    k2, v2 = k.copy(), v.copy()
    k2[last_view_start:] += 5.0
    v2[last_view_start:] -= 3.0
    out = fd_oracle.attend(q, k2, v2, qpos, kpos, g.rope_theta)
    rows = slice(0, (g.n_views - 1) * g.tok_per_frame)          # every view but the last
    assert np.array_equal(out[rows], base[rows])
    assert not np.allclose(out[rows.stop:], base[rows.stop:])   # and the last view does see them


def pin_ring_slots():
    """Slot occupancy equals an explicit simulation of in-order inserts into F slots."""
    for f in (1, 2, 4, 8):
        g = Geometry(2, f, 4, 0, 2, 1, 8, 0, 1e4)
        ring = [None] * f
        for t in range(3 * f + 3):
            ring[t % f] = t
            if t >= f - 1:
                assert fd_oracle.expected_ring_rows(g, t) == ring, (f, t)
                # read by age (oldest first) the slots give the logical window order
                ages = sorted(range(f), key=lambda s: ring[s])
                assert [ring[s] for s in ages] == list(range(t - f + 1, t + 1))


def pin_expected_cache_layout():
    """Cache rows hold prefix then, per view, the frame of each slot, token-major -> head-major."""
    w = TINY
    g, t = w.geom, 7
    pk, _ = synth.prefix_kv(w, 0)
    img = fd_oracle.expected_cache(g, pk, lambda v, f: synth.frame_kv(w, 0, v, f)[0], t)
    for h in range(g.n_kv_heads):
        for r in range(g.prefix_len):
            assert np.array_equal(img[h, r], pk[r, h])
        for v in range(g.n_views):
            for fid in range(t - g.n_frames + 1, t + 1):
                s = fid % g.n_frames
                k = synth.frame_kv(w, 0, v, fid)[0]
                for i in range(g.tok_per_frame):
                    row = g.prefix_len + (v * g.n_frames + s) * g.tok_per_frame + i
                    assert np.array_equal(img[h, row], k[i, h])
    assert np.isnan(img[:, g.window:, :]).all()


def pin_verify_sdpa():
    """Verify == torch SDPA over window ++ tail ++ block with block-causal mask."""
    w = TINY
    g, t = w.geom, w.first_t
    win = _window_at(w, t)
    k, v = win.kv()
    r, b = 5, 4
    kt, vt = synth.tail_kv(w, 0, r)
    qb, kb, vb = synth.block_qkv(w, 0, b)
    ka = np.concatenate([k, kt, kb]).astype(np.float64)
    va = np.concatenate([v, vt, vb]).astype(np.float64)
    pos = g.pos_base + np.arange(ka.shape[0])
    qpos = pos[-b:]
    mask = np.ones((b, ka.shape[0]), bool)
    mask[:, -b:] = np.tril(np.ones((b, b), bool))
    want = _sdpa(fd_oracle.rope(qb, qpos, g.rope_theta), fd_oracle.rope(ka, pos, g.rope_theta),
                 va, mask=mask)
    got = fd_oracle.oracle_verify(g, win, kt, vt, qb, kb, vb)
    err = np.max(np.abs(got - want))
    assert err <= 1e-12, err


def pin_stream_workload_rolling():
    """The whole-workload driver (which frames are pushed, which query frame is used at each t,
    which layer's draws) against scalar brute force at every window of a rolling stream.

    Over 2F+1 consecutive windows of a tiny geometry (the ring wraps twice) and at a layer
    other than 0, every yielded output equals `brute_force.brute_stream`, which builds the
    window at t from frame ids t-F+1..t and the queries of frame t by itself.
    """
    for w, layer in ((TINY, 2), (TINY_G4, 1)):
        g = w.geom
        ts = list(range(g.n_frames - 1, g.n_frames - 1 + 2 * g.n_frames + 1))
        got = dict(fd_oracle.run_stream_workload(w, layer, ts, synth))
        assert sorted(got) == ts, (w.name, sorted(got))
        pk, pv = synth.prefix_kv(w, layer)
        for t in ts:
            bf = brute_force.brute_stream(
                g, pk, pv, lambda v, f: synth.frame_kv(w, layer, v, f),
                lambda v, f: synth.frame_q(w, layer, v, f), t)
            err = np.max(np.abs(got[t] - np.array(bf)))
            assert err <= 1e-12, (w.name, layer, t, err)


def pin_kv_projection():
    """Brute-force sums on a tiny case; one-hot hidden states pick out weight columns; the
    head / dimension split of the output features."""
    rng = np.random.default_rng(21)
    t, hidden, hkv, d = 3, 5, 2, 4
    x = rng.standard_normal((t, hidden))
    w = rng.standard_normal((2 * hkv * d, hidden))
    k, v = fd_oracle.oracle_kv_projection(x, w, hkv, d)
    for i in range(t):
        for h in range(hkv):
            for e in range(d):
                sk = sum(x[i, j] * w[h * d + e, j] for j in range(hidden))
                sv = sum(x[i, j] * w[hkv * d + h * d + e, j] for j in range(hidden))
                assert abs(k[i, h, e] - sk) <= 1e-12 and abs(v[i, h, e] - sv) <= 1e-12
    eye = np.eye(hidden)[:t]
    k, v = fd_oracle.oracle_kv_projection(eye, w, hkv, d)
    for i in range(t):
        assert np.array_equal(k[i].reshape(-1), w[: hkv * d, i])
        assert np.array_equal(v[i].reshape(-1), w[hkv * d:, i])


ALL_PINS = [
    pin_rope_closed_form,
    pin_rope_group_properties,
    pin_brute_force_stream,
    pin_brute_force_verify,
    pin_shift_invariance,
    pin_sdpa_special_case,
    pin_streaming_equals_full_recompute,
    pin_full_window_is_sdpa_causal,
    pin_single_view_is_plain_causal,
    pin_closed_forms,
    pin_mask_leak,
    pin_ring_slots,
    pin_expected_cache_layout,
    pin_verify_sdpa,
    pin_kv_projection,
    pin_stream_workload_rolling,
]
