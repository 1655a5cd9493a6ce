"""GPU parity tests: the HIP path, called through the C ABI, against the fp64 oracle.

Tolerances (max-abs vs fp64): 1e-5 for fp32 inputs, 2e-2 for bf16 inputs with fp32
accumulation; cache insertion and the verify tail copy are compared bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.fd_oracle as fd_oracle
from streaming_kv_cache_view_amd import fd, synth
from streaming_kv_cache_view_amd.synth import Geometry, Workload

try:
    from . import gpu_harness as H
except ImportError:
    import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fd.lib()   # raises if the HIP library is missing: no fallback


def oracle_outputs(w, layer, t_values):
    return dict(fd_oracle.run_stream_workload(w, layer, t_values, synth))


def check_stream(w, layer, t_values, out_dtype="f32"):
    want = oracle_outputs(w, layer, t_values)
    tol = H.TOL[w.geom.dtype] + (0.02 if out_dtype == "bf16" else 0.0)
    for t, got in H.run_stream(w, layer, t_values, out_dtype):
        err = H.max_err(got, want[t])
        H.say(f"  cfg {w.cfg_id} layer {layer} t {t}: max-abs {err:.3e} (tol {tol})")
        assert err <= tol, (w.name, layer, t, err)


# ---------------------------------------------------------------------------- insert
@pytest.mark.parametrize("cid,t_last", [(1, 4), (1, 9), (2, 6), (5, 19)])
def test_insert_bit_exact(cid, t_last):
    w = synth.CONFIGS[cid]
    g = w.geom
    H.say(f"insert cfg {cid} frames 0..{t_last}")
    kc, vc = H.window_caches(w, 0, t_last)
    torch.cuda.synchronize()
    pk, pv = synth.prefix_kv(w, 0)
    for cache, pre, idx in ((kc, pk, 0), (vc, pv, 1)):
        want = fd_oracle.expected_cache(g, pre, lambda v, f: synth.frame_kv(w, 0, v, f)[idx], t_last,
                                         fill=H.SENTINEL)
        got = cache.float().cpu().numpy()
        assert np.array_equal(got, want.astype(np.float32)), "cache image differs"
        # bit-level: re-encode the expectation in the cache dtype and compare raw bits
        want_t = torch.from_numpy(want.astype(np.float32)).to(H.tdtype(g))
        bits = torch.int16 if g.dtype == synth.BF16 else torch.int32
        assert torch.equal(cache.cpu().view(bits), want_t.view(bits))


# ---------------------------------------------------------------------------- streaming prefill
@pytest.mark.parametrize("cid", [1, 2])
def test_stream_small_configs(cid):
    w = synth.CONFIGS[cid]
    check_stream(w, 0, [w.first_t, w.first_t + 3])


def test_stream_backbone_layers():
    w = synth.CONFIGS[3]
    for layer in (0, 35):
        check_stream(w, layer, [w.first_t])


def test_stream_rolling_100_windows():
    """Config 5: all 100 windows on the GPU (the ring wraps 12.5 times); every window is
    checked on a sample of query rows, five windows on every row."""
    w = synth.CONFIGS[5]
    g = w.geom
    ts = list(range(w.first_t, w.first_t + w.windows))
    full_t = {ts[0], ts[1], ts[8], ts[49], ts[-1]}
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(g.n_new, 48, replace=False))
    pk, pv = synth.prefix_kv(w, 0)
    win = fd_oracle.StreamWindow(g, pk, pv)
    kc, vc = H.new_cache(g)
    H.write_prefix(w, 0, kc, vc)
    worst = 0.0
    for t in range(ts[-1] + 1):
        k, v, q = synth.new_frames(w, 0, t)
        for vi in range(g.n_views):
            win.push(vi, t, k[vi], v[vi])
        H.insert(w, 0, kc, vc, t)
        if t < ts[0]:
            continue
        got = H.stream_out(w, 0, kc, vc, t).cpu().numpy().astype(np.float64)
        kw, vw = win.kv()
        qpos = fd_oracle.new_query_positions(g)
        kpos = fd_oracle.window_positions(g, kw.shape[0])
        sel = slice(None) if t in full_t else rows
        want = fd_oracle.attend(q[sel], kw, vw, qpos[sel], kpos, g.rope_theta)
        err = H.max_err(got[sel], want)
        worst = max(worst, err)
        if t in full_t:
            H.say(f"  cfg 5 window t={t} (all rows): max-abs {err:.3e}")
        assert err <= H.TOL[g.dtype], (t, err)
    H.say(f"  cfg 5 worst over 100 windows: {worst:.3e}")


def test_stream_bf16_output():
    check_stream(synth.CONFIGS[2], 0, [4], out_dtype="bf16")


EXTRA = [
    Workload(201, "bf16 D=64", Geometry(3, 4, 40, 24, 4, 2, 64, 16, 1e4, dtype=synth.BF16), first_t=5),
    Workload(202, "fp32 D=128", Geometry(2, 3, 48, 16, 8, 2, 128, 16, 1e6, dtype=synth.F32), first_t=4),
    Workload(203, "G=1 ragged", Geometry(2, 2, 37, 5, 3, 3, 128, 40, 1e6, dtype=synth.BF16), first_t=3),
    Workload(204, "G=8", Geometry(2, 4, 64, 64, 16, 2, 128, 8, 1e6, dtype=synth.BF16), first_t=6),
    Workload(205, "F=1 no prefix", Geometry(3, 1, 100, 0, 4, 1, 128, 8, 1e6, dtype=synth.BF16), first_t=2),
    Workload(206, "one view", Geometry(1, 4, 130, 70, 8, 4, 64, 8, 1e4, dtype=synth.F32), first_t=7),
    Workload(207, "G=2 T=1", Geometry(4, 3, 1, 3, 2, 1, 64, 8, 1e4, dtype=synth.F32), first_t=2),
]


@pytest.mark.parametrize("w", EXTRA, ids=lambda w: w.name)
def test_stream_edge_geometries(w):
    check_stream(w, 0, [w.first_t])


# ---------------------------------------------------------------------------- invariants on the GPU
def test_mask_leak_bit_identical():
    """Rows that may not see a key are bit-identical when that key's K/V change."""
    w = synth.CONFIGS[2]
    g = w.geom
    t = 5
    kc, vc = H.window_caches(w, 0, t)
    base = H.stream_out(w, 0, kc, vc, t).cpu()
    # later views: perturb every row of the last view
    lv0 = g.prefix_len + (g.n_views - 1) * g.n_frames * g.tok_per_frame
    kc2, vc2 = kc.clone(), vc.clone()
    kc2[:, lv0: g.window] += 3.0
    vc2[:, lv0: g.window] -= 2.0
    out = H.stream_out(w, 0, kc2, vc2, t).cpu()
    n_prev = (g.n_views - 1) * g.tok_per_frame
    assert torch.equal(out[:n_prev], base[:n_prev])
    assert not torch.allclose(out[n_prev:], base[n_prev:])
    # the newest frame of view 1: token 40 and later may only be seen by tokens >= 40
    s_new = t % g.n_frames
    r0 = g.prefix_len + (1 * g.n_frames + s_new) * g.tok_per_frame
    kc3, vc3 = kc.clone(), vc.clone()
    kc3[:, r0 + 40: r0 + g.tok_per_frame] *= -1.0
    vc3[:, r0 + 40: r0 + g.tok_per_frame] += 1.0
    out = H.stream_out(w, 0, kc3, vc3, t).cpu()
    T = g.tok_per_frame
    assert torch.equal(out[:T + 40], base[:T + 40])
    assert not torch.allclose(out[T + 40: 2 * T], base[T + 40: 2 * T])
    assert not torch.allclose(out[2 * T:], base[2 * T:])      # later views see all of view 1


def test_ring_phase_invariance():
    """The same logical window stored at two ring phases gives the same output."""
    w = synth.CONFIGS[2]
    g = w.geom
    t = 6
    kc, vc = H.window_caches(w, 0, t)
    a = H.stream_out(w, 0, kc, vc, t).cpu().numpy()
    # same frame contents, inserted one index later: every frame sits one slot further on
    kc2, vc2 = H.new_cache(g)
    H.write_prefix(w, 0, kc2, vc2)
    for f in range(t + 1):
        H.insert(w, 0, kc2, vc2, f + 1, frame_src=f)
    b = H.stream_out(w, 0, kc2, vc2, t + 1, q=H.q_new(w, 0, t)).cpu().numpy()
    assert not torch.equal(kc, kc2)
    err = H.max_err(a, b)
    H.say(f"  ring phase t={t} vs t={t + 1}: max-abs {err:.3e}")
    assert err <= 2e-3
    want = oracle_outputs(w, 0, [t])[t]
    assert H.max_err(b, want) <= H.TOL[g.dtype]


def test_shift_invariance_pos_base():
    w = synth.CONFIGS[1]
    ref = oracle_outputs(w, 0, [4])[4]
    for c in (0, 1000, 2 ** 20):
        w2 = Workload(w.cfg_id, w.name, w.geom.replace(pos_base=c), first_t=4)
        (t, got), = list(H.run_stream(w2, 0, [4]))
        err = H.max_err(got, ref)
        H.say(f"  pos_base {c}: max-abs vs oracle {err:.3e}")
        assert err <= H.TOL[w.geom.dtype]


def test_deterministic():
    w = synth.CONFIGS[3]
    kc, vc = H.window_caches(w, 1, 4)
    q = H.q_new(w, 1, 4)
    a = H.stream_out(w, 1, kc, vc, 4, q=q)
    b = H.stream_out(w, 1, kc, vc, 4, q=q)
    assert torch.equal(a, b)


# ---------------------------------------------------------------------------- verify
def check_verify(w, layer, t, n_tail, blk_len, out_dtype="f32"):
    g = w.geom
    H.say(f"verify cfg {w.cfg_id} layer {layer} t {t} n_tail {n_tail} B {blk_len}")
    out, kc, vc = H.run_verify(w, layer, t, n_tail, blk_len, out_dtype=out_dtype)
    pk, pv = synth.prefix_kv(w, layer)
    win = fd_oracle.StreamWindow(g, pk, pv)
    for f in range(t + 1):
        for v in range(g.n_views):
            k, vv = synth.frame_kv(w, layer, v, f)
            win.push(v, f, k, vv)
    kt, vt = synth.tail_kv(w, layer, n_tail)
    qb, kb, vb = synth.block_qkv(w, layer, blk_len)
    want = fd_oracle.oracle_verify(g, win, kt, vt, qb, kb, vb)
    err = H.max_err(out.float().cpu().numpy(), want)
    tol = H.TOL[g.dtype] + (0.02 if out_dtype == "bf16" else 0.0)
    H.say(f"  max-abs {err:.3e} (tol {tol})")
    assert err <= tol
    # the block's K/V landed bit-exactly in the tail rows; the rest of the tail is untouched
    r0 = g.window + n_tail
    kbt = H.dev(np.transpose(kb, (1, 0, 2)), g)
    vbt = H.dev(np.transpose(vb, (1, 0, 2)), g)
    assert torch.equal(kc[:, r0: r0 + blk_len], kbt) and torch.equal(vc[:, r0: r0 + blk_len], vbt)
    rest = kc[:, r0 + blk_len:]
    assert bool((rest == H.SENTINEL).all())


@pytest.mark.parametrize("n_tail,blk_len", [(5, 8), (0, 1), (13, 3), (24, 8)])
def test_verify_small(n_tail, blk_len):
    check_verify(synth.CONFIGS[1], 0, 4, n_tail, blk_len)


def test_verify_small_bf16():
    check_verify(synth.CONFIGS[2], 0, 5, 40, 8)
    check_verify(synth.CONFIGS[2], 0, 5, 7, 8, out_dtype="bf16")


def test_verify_config4_layers():
    w = synth.CONFIGS[4]
    for layer in (0, 35):
        check_verify(w, layer, w.first_t, w.n_tail, w.blk_len)


# Larger draft blocks: G*B query rows per kv head in several 32-row blocks, two per workgroup
# (G = 4: B = 16 is 64 rows, B = 12 is 48 rows with a partial second block, B = 24 is three
# blocks (the second workgroup of a split has one), B = 32 four; config 1 has G = 2).
@pytest.mark.parametrize("cid,n_tail,blk_len", [(2, 40, 16), (2, 3, 12), (2, 17, 24), (2, 0, 32), (1, 8, 24),
                                                (1, 0, 16)])
def test_verify_block_rows(cid, n_tail, blk_len):
    check_verify(synth.CONFIGS[cid], 0, 5 if cid == 2 else 4, n_tail, blk_len)


def test_verify_config4_block16():
    w = synth.CONFIGS[4]
    check_verify(w, 0, w.first_t, w.n_tail, 16)
    check_verify(w, 7, w.first_t, w.n_tail, 16, out_dtype="bf16")


@pytest.mark.parametrize("w", EXTRA[:4], ids=lambda w: w.name)
def test_verify_edge_geometries(w):
    g = w.geom
    b = max(1, min(32 // (g.n_q_heads // g.n_kv_heads), g.tail_cap))
    check_verify(w, 0, w.first_t, max(0, g.tail_cap - b), b)


# ---------------------------------------------------------------------------- cold-start prefill
def window_queries(w, layer, t):
    """Queries of every window row in cache-row order [W][Hq][D], and the map cache row ->
    logical row (prefix, then view 0 oldest..newest, view 1, ...)."""
    g = w.geom
    P, T, F = g.prefix_len, g.tok_per_frame, g.n_frames
    q = np.empty((g.window, g.n_q_heads, g.head_dim), np.float64)
    logical = np.empty(g.window, np.int64)
    if P:
        q[:P] = synth.prefix_q(w, layer)
        logical[:P] = np.arange(P)
    slots = fd_oracle.expected_ring_rows(g, t)
    for v in range(g.n_views):
        for s, fid in enumerate(slots):
            r0 = P + (v * F + s) * T
            j = fid - (t - F + 1)                      # age of the frame (oldest = 0)
            q[r0: r0 + T] = synth.frame_q(w, layer, v, fid)
            logical[r0: r0 + T] = P + (v * F + j) * T + np.arange(T)
    return q, logical


def check_prefill(w, layer, t, rows=None, out_dtype="f32"):
    g = w.geom
    H.say(f"prefill cfg {w.cfg_id} ({w.name}) layer {layer} t {t}")
    kc, vc = H.window_caches(w, layer, t)
    q, logical = window_queries(w, layer, t)
    ws = torch.empty(fd.prefill_workspace_bytes(g), dtype=torch.uint8, device=H.DEV)
    out = torch.empty((g.window, g.n_q_heads, g.head_dim),
                      dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16, device=H.DEV)
    fd.prefill_attn(g, H.dev(q, g), kc, vc, t, out, ws, out_dtype=out_dtype)
    got = out.float().cpu().numpy().astype(np.float64)
    win = fd_oracle.StreamWindow(g, *synth.prefix_kv(w, layer))
    for f in range(t + 1):
        for v in range(g.n_views):
            win.push(v, f, *synth.frame_kv(w, layer, v, f))
    q_log = np.empty_like(q)
    q_log[logical] = q
    kw, vw = win.kv()
    pos = fd_oracle.window_positions(g, kw.shape[0])
    sel = np.arange(g.window) if rows is None else np.asarray(rows)
    want = fd_oracle.attend(q_log[logical[sel]], kw, vw, pos[logical[sel]], pos, g.rope_theta)
    tol = H.TOL[g.dtype] + (0.02 if out_dtype == "bf16" else 0.0)
    err = H.max_err(got[sel], want)
    H.say(f"  {len(sel)} rows: max-abs {err:.3e} (tol {tol})")
    assert err <= tol
    return got, kc, vc


@pytest.mark.parametrize("t", [3, 6])
def test_prefill_small(t):
    """Config 2 shapes: every window row (W = 1,088) against the oracle, at the first full
    window (slots in frame order) and at a later ring phase."""
    check_prefill(synth.CONFIGS[2], 0, t)


def test_prefill_matches_stream_rows():
    """The newest frames' rows of a cold-start prefill are the streaming call's output."""
    w = synth.CONFIGS[2]
    g = w.geom
    t = 6
    got, kc, vc = check_prefill(w, 0, t, rows=[0, 1, 500, 1087])
    st = H.stream_out(w, 0, kc, vc, t).cpu().numpy()
    s_new = t % g.n_frames
    for v in range(g.n_views):
        r0 = g.prefix_len + (v * g.n_frames + s_new) * g.tok_per_frame
        err = H.max_err(got[r0: r0 + g.tok_per_frame], st[v * g.tok_per_frame: (v + 1) * g.tok_per_frame])
        assert err <= 2e-3, (v, err)


def test_prefill_backbone_sampled():
    """Config 3 shapes (W = 4,608 queries over 4,608 keys): sampled rows of every segment."""
    w = synth.CONFIGS[3]
    g = w.geom
    rng = np.random.default_rng(11)
    rows = np.sort(np.concatenate([rng.choice(g.prefix_len, 24, replace=False),
                                   g.prefix_len + rng.choice(g.window - g.prefix_len, 104, replace=False),
                                   [0, g.prefix_len - 1, g.prefix_len, g.window - 1]]))
    check_prefill(w, 0, w.first_t + 1, rows=rows, out_dtype="bf16")


@pytest.mark.parametrize("w", [x for x in EXTRA if x.geom.dtype == synth.BF16], ids=lambda w: w.name)
def test_prefill_edge_geometries(w):
    check_prefill(w, 0, w.first_t)


# ---------------------------------------------------------------------------- K/V projection
def check_kv_project(w, layer, t, hidden):
    """Project every view's frame t and insert it: the slot rows against the oracle's
    projection (bf16 rounding of fp32 sums: |err| <= 2^-8 |ref| + 1e-4), every other row
    untouched."""
    g = w.geom
    H.say(f"kv projection cfg {w.cfg_id} ({w.name}) layer {layer} frame {t} hidden {hidden}")
    x = np.concatenate([synth.frame_hidden(w, layer, v, t, hidden) for v in range(g.n_views)])
    wk = synth.kv_weights(w, layer, hidden)
    kc, vc = H.new_cache(g)
    fd.kv_project_insert(g, H.dev(x, g), H.dev(wk, g), kc, vc, t)
    kc_h, vc_h = kc.float().cpu().numpy(), vc.float().cpu().numpy()
    s = t % g.n_frames
    worst = 0.0
    rows = np.zeros(g.cache_rows, bool)
    for v in range(g.n_views):
        xv = x[v * g.tok_per_frame: (v + 1) * g.tok_per_frame]
        k_ref, v_ref = fd_oracle.oracle_kv_projection(xv, wk, g.n_kv_heads, g.head_dim)
        r0 = g.prefix_len + (v * g.n_frames + s) * g.tok_per_frame
        rows[r0: r0 + g.tok_per_frame] = True
        for got, ref in ((kc_h, k_ref), (vc_h, v_ref)):
            seg = got[:, r0: r0 + g.tok_per_frame, :]                   # [Hkv][T][D]
            want = np.transpose(ref, (1, 0, 2))
            err = np.abs(seg - want)
            assert np.all(err <= 2.0 ** -8 * np.abs(want) + 1e-4), float(err.max())
            worst = max(worst, float(err.max()))
    assert np.all(kc_h[:, ~rows, :] == H.SENTINEL) and np.all(vc_h[:, ~rows, :] == H.SENTINEL)
    H.say(f"  max-abs {worst:.3e}; other rows untouched")


@pytest.mark.parametrize("cid,t,hidden", [(2, 5, 256), (2, 2, 1024), (3, 4, 4096)])
def test_kv_project_insert(cid, t, hidden):
    check_kv_project(synth.CONFIGS[cid], 0, t, hidden)


@pytest.mark.parametrize("w", [x for x in EXTRA if x.geom.dtype == synth.BF16], ids=lambda w: w.name)
def test_kv_project_edge_geometries(w):
    check_kv_project(w, 0, w.first_t, 192)


# ---------------------------------------------------------------------------- insert fused into the stream call
def check_stream_insert(w, layer, t, out_dtype="f32"):
    """fd_stream_attn_insert against fd_kv_insert_frame followed by fd_stream_attn on an identical
    copy of the caches: output and both caches bit-identical (the separate calls are checked
    against the oracle elsewhere; this one also against the oracle directly)."""
    g = w.geom
    H.say(f"stream+insert cfg {w.cfg_id} ({w.name}) layer {layer} t {t} out {out_dtype}")
    kc, vc = H.window_caches(w, layer, t - 1)   # frames 0 .. t-1 inserted
    kc2, vc2 = kc.clone(), vc.clone()
    k, v, _ = synth.new_frames(w, layer, t)
    kn, vn = H.dev(k, g), H.dev(v, g)
    q = H.q_new(w, layer, t)
    fd.kv_insert_frame(g, kc, vc, kn, vn, t)
    ref = H.stream_out(w, layer, kc, vc, t, out_dtype, q=q)
    out = torch.empty_like(ref)
    ws = torch.empty(fd.stream_workspace_bytes(g), dtype=torch.uint8, device=H.DEV)
    fd.stream_attn_insert(g, kn, vn, q, kc2, vc2, t, out, ws, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(kc, kc2) and torch.equal(vc, vc2), "cache images differ"
    assert torch.equal(out, ref), float((out.float() - ref.float()).abs().max())
    err = H.max_err(out.float().cpu().numpy().astype(np.float64), oracle_outputs(w, layer, [t])[t])
    tol = H.TOL[g.dtype] + (0.02 if out_dtype == "bf16" else 0.0)
    H.say(f"  bit-identical to insert + stream; max-abs vs oracle {err:.3e} (tol {tol})")
    assert err <= tol


@pytest.mark.parametrize("cid,dt", [(1, "f32"), (2, "f32"), (3, "f32"), (3, "bf16")])
def test_stream_insert_fused(cid, dt):
    w = synth.CONFIGS[cid]
    check_stream_insert(w, 0, w.first_t + 1, dt)


@pytest.mark.parametrize("w", EXTRA, ids=lambda w: w.name)
def test_stream_insert_fused_edge_geometries(w):
    check_stream_insert(w, 0, w.first_t + w.geom.n_frames)   # a later ring phase
