"""Helpers for the GPU tests: build device inputs from the seeded generator and drive the
HIP path through the C ABI (streaming_kv_cache_view_amd.fd).  Test infrastructure."""
from __future__ import annotations

import sys

import numpy as np
import torch

from streaming_kv_cache_view_amd import fd, synth

DEV = "cuda"
TOL = {synth.F32: 1e-5, synth.BF16: 2e-2}   # max-abs vs the fp64 oracle
SENTINEL = -7.5                              # exactly representable in bf16 and fp32


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tdtype(g):
    return torch.bfloat16 if g.dtype == synth.BF16 else torch.float32


def dev(a, g):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(tdtype(g)).contiguous()


def new_cache(g, fill=SENTINEL):
    shape = (g.n_kv_heads, g.cache_rows, g.head_dim)
    return (torch.full(shape, fill, dtype=tdtype(g), device=DEV),
            torch.full(shape, fill, dtype=tdtype(g), device=DEV))


def write_prefix(w, layer, kc, vc):
    """The caller places the static prefix rows [0, P) directly (head-major)."""
    g = w.geom
    if g.prefix_len == 0:
        return
    pk, pv = synth.prefix_kv(w, layer)
    kc[:, : g.prefix_len, :] = dev(np.transpose(pk, (1, 0, 2)), g)
    vc[:, : g.prefix_len, :] = dev(np.transpose(pv, (1, 0, 2)), g)


def insert(w, layer, kc, vc, t, frame_src=None):
    g = w.geom
    src = frame_src if frame_src is not None else t
    k, v, _ = synth.new_frames(w, layer, src)
    fd.kv_insert_frame(g, kc, vc, dev(k, g), dev(v, g), t)


def q_new(w, layer, t):
    g = w.geom
    return dev(np.concatenate([synth.frame_q(w, layer, v, t) for v in range(g.n_views)]), g)


def stream_out(w, layer, kc, vc, t, out_dtype="f32", q=None):
    g = w.geom
    out = torch.empty((g.n_new, g.n_q_heads, g.head_dim),
                      dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16, device=DEV)
    ws = torch.empty(fd.stream_workspace_bytes(g), dtype=torch.uint8, device=DEV)
    fd.stream_attn(g, q if q is not None else q_new(w, layer, t), kc, vc, t, out, ws, out_dtype=out_dtype)
    return out


def run_stream(w, layer, t_values, out_dtype="f32"):
    """Insert frames 0..max(t) and run attention at each t; yields (t, output on host, fp64)."""
    g = w.geom
    kc, vc = new_cache(g)
    write_prefix(w, layer, kc, vc)
    t_values = sorted(t_values)
    for t in range(t_values[-1] + 1):
        insert(w, layer, kc, vc, t)
        if t in t_values:
            out = stream_out(w, layer, kc, vc, t, out_dtype)
            yield t, out.float().cpu().numpy().astype(np.float64)


def window_caches(w, layer, t):
    g = w.geom
    kc, vc = new_cache(g)
    write_prefix(w, layer, kc, vc)
    for f in range(t + 1):
        insert(w, layer, kc, vc, f)
    return kc, vc


def run_verify(w, layer, t, n_tail, blk_len, kc=None, vc=None, out_dtype="f32"):
    """Verify on a window at t with n_tail reasoning rows; returns (out, kc, vc)."""
    g = w.geom
    if kc is None:
        kc, vc = window_caches(w, layer, t)
    if n_tail:
        kt, vt = synth.tail_kv(w, layer, n_tail)
        kc[:, g.window: g.window + n_tail, :] = dev(np.transpose(kt, (1, 0, 2)), g)
        vc[:, g.window: g.window + n_tail, :] = dev(np.transpose(vt, (1, 0, 2)), g)
    qb, kb, vb = synth.block_qkv(w, layer, blk_len)
    ws = torch.empty(fd.verify_workspace_bytes(g, blk_len), dtype=torch.uint8, device=DEV)
    out = torch.empty((blk_len, g.n_q_heads, g.head_dim),
                      dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16, device=DEV)
    fd.verify_attn(g, dev(qb, g), dev(kb, g), dev(vb, g), kc, vc, t, n_tail, blk_len, out, ws,
                   out_dtype=out_dtype)
    return out, kc, vc


def bf16_half_ulp(x):
    """Half a bfloat16 ulp at magnitude |x| (8 significant bits): 2^(e-8) for |x| in [2^e, 2^(e+1))."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, (np.floor(np.log2(a)) - 8).astype(np.int64))


def out_bound(want, g, out_dtype):
    """Per-element bound against the fp64 oracle: the input dtype's tolerance, plus for bf16
    outputs the half ulp that rounding the fp32 result to bf16 adds (at the magnitude the fp32
    result can reach, |ref| + tolerance)."""
    tol = TOL[g.dtype]
    if out_dtype != "bf16":
        return np.full(np.shape(want), tol)
    return tol + bf16_half_ulp(np.abs(want) + tol)


def check_out(got, want, g, out_dtype, what=""):
    """Assert |got - want| <= out_bound elementwise; returns the max-abs error."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), what
    err = np.abs(got - want)
    excess = err - out_bound(want, g, out_dtype)
    worst = int(np.argmax(excess))
    assert excess.flat[worst] <= 0, (what, float(err.flat[worst]), float(want.flat[worst]))
    return float(err.max())


def check_bf16_rounding(got_bf16, got_f32, what=""):
    """A bf16 output is the fp32 output of the same call rounded: within half a bf16 ulp of it
    (plus 2^-20 relative for fp32 reassociation)."""
    b = np.asarray(got_bf16, np.float64)
    f = np.asarray(got_f32, np.float64)
    err = np.abs(b - f)
    assert np.all(err <= bf16_half_ulp(f) * (1 + 2.0 ** -20) + 1e-30), (what, float(err.max()))


def max_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.isfinite(a).all()
    return float(np.max(np.abs(a - b)))
