"""CPU tests: the oracle against its pins, and planted oracle mistakes caught by them."""
from __future__ import annotations

import numpy as np
import pytest

import oracle.fd_oracle as fd_oracle

try:
    from . import oracle_pins as P
except ImportError:
    import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# Mutation check: plant a plausible mistake in the oracle (on the CPU) and make
# sure at least one pin fails.  Each mutant replaces one oracle function.
# ----------------------------------------------------------------------------
_rope = fd_oracle.rope
_inv_freq = fd_oracle.inv_freq
_attend = fd_oracle.attend
_nqp = fd_oracle.new_query_positions
_ring = fd_oracle.expected_ring_rows


def _rope_wrong_sign(x, pos, theta):
    return _rope(x, -np.asarray(pos), theta)


def _rope_interleaved(x, pos, theta):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    perm = np.stack([np.arange(d // 2), np.arange(d // 2) + d // 2], axis=1).reshape(-1)
    inv = np.argsort(perm)
    return _rope(x[..., perm], pos, theta)[..., inv]


def _rope_dropped_term(x, pos, theta):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    y = _rope(x, pos, theta)
    ang = np.asarray(pos, np.float64)[:, None] * _inv_freq(d, theta)[None, :]
    s = np.sin(ang)
    if x.ndim == 3:
        s = s[:, None, :]
    y[..., d // 2:] -= x[..., : d // 2] * s          # y2 loses its x1*sin term
    return y


def _inv_freq_off(d, theta):
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -1.0 * i / d)


def _attend_variant(strict=False, modulo=False, scale=True):
    """A copy of the oracle's attention with one planted mistake switched on."""
    def attend(q, k, v, q_pos, k_pos, theta):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        nq, hq, d = q.shape
        hkv = k.shape[1]
        qr = fd_oracle.rope(q, q_pos, theta)
        kr = fd_oracle.rope(k, k_pos, theta)
        kp, qp = np.asarray(k_pos)[None, :], np.asarray(q_pos)[:, None]
        mask = (kp < qp) if strict else (kp <= qp)
        out = np.empty((nq, hq, d))
        for h in range(hq):
            kv = (h % hkv) if modulo else h // (hq // hkv)
            s = qr[:, h, :] @ kr[:, kv, :].T
            if scale:
                s = s / np.sqrt(d)
            s = np.where(mask, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[:, h, :] = (p / p.sum(axis=1, keepdims=True)) @ v[:, kv, :]
        return out
    return attend


def _nqp_off_by_one_frame(g):
    return _nqp(g) - g.tok_per_frame


def _nqp_off_by_one_token(g):
    return _nqp(g) + 1


def _ring_off(g, t):
    return _ring(g, t - 1)


def _window_newest_first(self):
    ks = [self.prefix_k] + [k for d in self.frames for (k, _) in reversed(d)]
    vs = [self.prefix_v] + [v for d in self.frames for (_, v) in reversed(d)]
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def _kv_proj_swapped(x, w_kv, n_kv_heads, head_dim):
    k, v = _KV_PROJ(x, w_kv, n_kv_heads, head_dim)
    return v, k


def _kv_proj_head_dim_transposed(x, w_kv, n_kv_heads, head_dim):
    k, v = _KV_PROJ(x, w_kv, n_kv_heads, head_dim)
    t = k.shape[0]
    fix = lambda a: a.reshape(t, head_dim, n_kv_heads).transpose(0, 2, 1)
    return fix(k), fix(v)


def _kv_proj_weight_layout(x, w_kv, n_kv_heads, head_dim):
    # the weights' memory read as [hidden][2*Hkv*D] (input-major) instead of one feature per row
    x = np.asarray(x, np.float64)
    n = n_kv_heads * head_dim
    w = np.asarray(w_kv, np.float64).reshape(-1, 2 * n)
    t = x.shape[0]
    return (x @ w[:, :n]).reshape(t, n_kv_heads, head_dim), (x @ w[:, n:]).reshape(t, n_kv_heads, head_dim)


def _full_window_stream_positions(geom, window, q_window):
    # every query rotated at the newest frame's positions, as a streaming-only oracle would
    k, v = window.kv()
    pos = fd_oracle.window_positions(geom, k.shape[0])
    qpos = np.minimum(pos + geom.tok_per_frame, pos[-1])
    return fd_oracle.attend(q_window, k, v, qpos, pos, geom.rope_theta)


def _workload_variant(q_lag=0, skip_last_push=False, frame_layer=None):
    """A copy of the oracle's workload driver with one planted mistake switched on: queries
    taken from frame t - q_lag, the last view's newest frame pushed only after attention,
    or the frames drawn from another layer's seeds."""
    def run(workload, layer, t_values, synth):
        g = workload.geom
        pk, pv = synth.prefix_kv(workload, layer)
        win = fd_oracle.StreamWindow(g, pk, pv)
        t_values = list(t_values)
        fl = layer if frame_layer is None else frame_layer
        for t in range(max(t_values) + 1):
            for v in range(g.n_views):
                if skip_last_push and v == g.n_views - 1 and t in t_values:
                    continue
                k, vv = synth.frame_kv(workload, fl, v, t)
                win.push(v, t, k, vv)
            if t in t_values:
                if not win.full():
                    raise AssertionError("window not full")
                q = np.concatenate([synth.frame_q(workload, layer, v, max(t - q_lag, 0))
                                    for v in range(g.n_views)])
                yield t, fd_oracle.oracle_stream(g, win, q)
            if skip_last_push and t in t_values:
                k, vv = synth.frame_kv(workload, fl, g.n_views - 1, t)
                win.push(g.n_views - 1, t, k, vv)
    return run


_KV_PROJ = fd_oracle.oracle_kv_projection

MUTANTS = {
    "rope_wrong_sign": ("rope", _rope_wrong_sign),
    "rope_interleaved_pairs": ("rope", _rope_interleaved),
    "rope_dropped_term": ("rope", _rope_dropped_term),
    "inv_freq_exponent": ("inv_freq", _inv_freq_off),
    "mask_strict": ("attend", _attend_variant(strict=True)),
    "gqa_modulo": ("attend", _attend_variant(modulo=True)),
    "missing_scale": ("attend", _attend_variant(scale=False)),
    "query_pos_frame": ("new_query_positions", _nqp_off_by_one_frame),
    "query_pos_token": ("new_query_positions", _nqp_off_by_one_token),
    "ring_off_by_one": ("expected_ring_rows", _ring_off),
    "kv_proj_swapped": ("oracle_kv_projection", _kv_proj_swapped),
    "kv_proj_head_dim_transposed": ("oracle_kv_projection", _kv_proj_head_dim_transposed),
    "kv_proj_weight_layout": ("oracle_kv_projection", _kv_proj_weight_layout),
    "full_window_query_positions": ("oracle_full_window", _full_window_stream_positions),
    "workload_query_frame_lag": ("run_stream_workload", _workload_variant(q_lag=1)),
    "workload_missing_last_push": ("run_stream_workload", _workload_variant(skip_last_push=True)),
    "workload_wrong_layer_seed": ("run_stream_workload", _workload_variant(frame_layer=0)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS) + ["window_newest_first"])
def test_pins_catch_planted_mistake(name, monkeypatch):
    if name == "window_newest_first":
        monkeypatch.setattr(fd_oracle.StreamWindow, "kv", _window_newest_first)
    else:
        attr, fn = MUTANTS[name]
        monkeypatch.setattr(fd_oracle, attr, fn)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, KeyError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} slipped through every pin"
