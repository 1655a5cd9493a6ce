"""GPU parity tests: the HIP path, called through the C ABI, against the fp64 oracle.

Tolerances (max-abs vs fp64): 1e-5 for fp32 inputs, 2e-2 for bf16 inputs with fp32
accumulation; cache insertion and the verify tail copy are compared bit for bit.
"""
from __future__ import annotations

import dataclasses

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
    """Streaming outputs against the oracle, element by element (out_bound: the input dtype's
    tolerance, plus half a bf16 ulp for bf16 outputs)."""
    want = oracle_outputs(w, layer, t_values)
    for t, got in H.run_stream(w, layer, t_values, out_dtype):
        err = H.check_out(got, want[t], w.geom, out_dtype, (w.name, layer, t))
        H.say(f"  cfg {w.cfg_id} layer {layer} t {t} out {out_dtype}: max-abs {err:.3e} "
              f"(tol {H.TOL[w.geom.dtype]}{' + half bf16 ulp' if out_dtype == 'bf16' else ''})")


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
    """bf16 output: against the oracle per element, and equal to the same call's fp32 output
    rounded to bf16 (within half an ulp), at configs 2 and 3."""
    for cid in (2, 3):
        w = synth.CONFIGS[cid]
        check_stream(w, 0, [w.first_t], out_dtype="bf16")
        kc, vc = H.window_caches(w, 0, w.first_t)
        q = H.q_new(w, 0, w.first_t)
        f32 = H.stream_out(w, 0, kc, vc, w.first_t, "f32", q=q).cpu().numpy()
        b16 = H.stream_out(w, 0, kc, vc, w.first_t, "bf16", q=q).float().cpu().numpy()
        H.check_bf16_rounding(b16, f32, ("stream", cid))


EXTRA = [
    Workload(201, "bf16 D=64", Geometry(3, 4, 40, 24, 4, 2, 64, 16, 1e4, dtype=synth.BF16), first_t=5),
    Workload(202, "fp32 D=128", Geometry(2, 3, 48, 16, 8, 2, 128, 16, 1e6, dtype=synth.F32), first_t=4),
    Workload(203, "G=1 ragged", Geometry(2, 2, 37, 5, 3, 3, 128, 40, 1e6, dtype=synth.BF16), first_t=3),
    Workload(204, "G=8", Geometry(2, 4, 64, 64, 16, 2, 128, 8, 1e6, dtype=synth.BF16), first_t=6),
    Workload(205, "F=1 no prefix", Geometry(3, 1, 100, 0, 4, 1, 128, 8, 1e6, dtype=synth.BF16), first_t=2),
    Workload(206, "one view", Geometry(1, 4, 130, 70, 8, 4, 64, 8, 1e4, dtype=synth.F32), first_t=7),
    Workload(207, "G=2 T=1", Geometry(4, 3, 1, 3, 2, 1, 64, 8, 1e4, dtype=synth.F32), first_t=2),
    # query-head groups that are not 1, 2 or a multiple of 4: the last four-head subset is ragged
    Workload(209, "G=3", Geometry(2, 3, 40, 12, 6, 2, 128, 16, 1e6, dtype=synth.BF16), first_t=4),
    Workload(210, "G=5", Geometry(2, 2, 64, 16, 5, 1, 128, 16, 1e6, dtype=synth.BF16), first_t=3),
    Workload(211, "G=6 D=64", Geometry(3, 2, 33, 8, 6, 1, 64, 24, 1e4, dtype=synth.BF16), first_t=3),
    Workload(212, "G=7 fp32", Geometry(2, 2, 29, 6, 14, 2, 128, 16, 1e6, dtype=synth.F32), first_t=3),
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


@pytest.mark.parametrize("cid", [1, 2])
def test_ring_phase_invariance(cid):
    """The same logical window stored at two ring phases gives the same output, bit for bit."""
    w = synth.CONFIGS[cid]
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
    # Bit-identical: a key's rotation depends on its logical position only (block base angle
    # times in-block offset, or the element's own angle, both from the logical layout), the
    # attention walks the key tiles in logical order (every frame by age) with the same work
    # split, so every operand and every sum is the same.
    H.say(f"  ring phase t={t} vs t={t + 1}: max-abs {H.max_err(a, b):.3e}")
    assert np.array_equal(a, b)
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


# pos_base up to the ABI's limit (positions < 2^31): the bf16 path's angle code (query angles
# from the hardware sin/cos on a revolution fraction, key angles as a block base angle times an
# in-block offset, verify's per-lane angles) at large positions
BIG_POS = [1000, 2 ** 20, 2 ** 30, None]   # None: 2^31 - S_cap - 1, the last row at 2^31 - 1


@pytest.mark.parametrize("c", BIG_POS, ids=lambda c: "max" if c is None else str(c))
def test_shift_invariance_bf16(c):
    """Config-2 shapes at a large pos_base: streaming, cold-start prefill (every row) and
    verify against the oracle at the same pos_base (and so, by the pinned shift invariance of
    the oracle, against the unshifted result)."""
    w = synth.CONFIGS[2]
    if c is None:
        c = 2 ** 31 - w.geom.cache_rows - 1
    w2 = Workload(w.cfg_id, w.name, w.geom.replace(pos_base=c), scale=w.scale, first_t=w.first_t)
    H.say(f"pos_base {c}")
    check_stream(w2, 0, [w.first_t + 1])
    check_prefill(w2, 0, w.first_t + 2)
    check_verify(w2, 0, w.first_t + 1, 40, 8)
    check_verify_batched(w2, 0, w.first_t + 1, [20, 3], 32, 8, "rotate")


def test_deterministic():
    w = synth.CONFIGS[3]
    kc, vc = H.window_caches(w, 1, 4)
    q = H.q_new(w, 1, 4)
    a = H.stream_out(w, 1, kc, vc, 4, q=q)
    b = H.stream_out(w, 1, kc, vc, 4, q=q)
    assert torch.equal(a, b)


# 512 attention workgroups (8 kv heads x 16 token blocks x 4 views), more than the GPU's CUs
MANY_WG = Workload(208, "512 workgroups", Geometry(4, 2, 512, 64, 32, 8, 128, 16, 1e6, dtype=synth.BF16), first_t=2)


@pytest.mark.parametrize("w", [synth.CONFIGS[2], synth.CONFIGS[3], synth.CONFIGS[5], MANY_WG]
                         + [x for x in EXTRA if x.cfg_id in (209, 210)], ids=lambda w: w.name)
def test_merge_modes_same_bits(w):
    """A view that two workgroups share is merged in the attention kernel by whichever piece
    finishes second (mode 1, the default), by the second piece (mode 2, which makes it finish
    second) or by the merge kernel (mode 0): fp32 and bf16 outputs must be the same bits in every
    mode, and match the oracle."""
    cid = w.cfg_id
    t = w.first_t + 1
    kc, vc = H.window_caches(w, 0, t)
    q = H.q_new(w, 0, t)
    got = {}
    prev = fd.stream_merge_mode()
    try:
        for mode in (1, 0, 2):
            assert fd.stream_merge_mode(mode) in (0, 1, 2) and fd.stream_merge_mode() == mode
            got[mode] = (H.stream_out(w, 0, kc, vc, t, q=q), H.stream_out(w, 0, kc, vc, t, out_dtype="bf16", q=q))
            if mode != 1:
                check_stream(w, 0, [t])
    finally:
        fd.stream_merge_mode(prev)
    assert fd.stream_merge_mode() == prev
    for mode in (0, 2):
        same = torch.equal(got[1][0], got[mode][0]) and torch.equal(got[1][1], got[mode][1])
        H.say(f"cfg {cid} t {t}: mode {mode} outputs equal to mode 1 (fp32 and bf16): {same}")
        assert same


def test_merge_in_kernel_repeat_bit_identical():
    """The in-kernel merge of split views over many calls: 12 config-3 layers (two ring phases each)
    and 6 config-5 windows, every output of the default mode the same bits as the merge kernel's
    (mode 0) on the same inputs."""
    prev = fd.stream_merge_mode()
    n = 0
    try:
        for cid, layers, ts in ((3, range(12), (4, 5)), (5, range(2), (8, 9, 10))):
            w = synth.CONFIGS[cid]
            for layer in layers:
                for t in ts:
                    kc, vc = H.window_caches(w, layer, t)
                    q = H.q_new(w, layer, t)
                    fd.stream_merge_mode(1)
                    a = H.stream_out(w, layer, kc, vc, t, q=q)
                    fd.stream_merge_mode(0)
                    b = H.stream_out(w, layer, kc, vc, t, q=q)
                    assert torch.equal(a, b), (cid, layer, t)
                    n += 1
    finally:
        fd.stream_merge_mode(prev)
    H.say(f"{n} calls: in-kernel merge bit-identical to the merge kernel")


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
    err = H.check_out(out.float().cpu().numpy(), want, g, out_dtype, ("verify", w.name, layer))
    H.say(f"  max-abs {err:.3e} (tol {H.TOL[g.dtype]}{' + half bf16 ulp' if out_dtype == 'bf16' else ''})")
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


GQA_ODD = [w for w in EXTRA if w.cfg_id in (209, 210, 211, 212)]   # G = 3, 5, 6, 7


@pytest.mark.parametrize("w", EXTRA[:4] + GQA_ODD, ids=lambda w: w.name)
def test_verify_edge_geometries(w):
    g = w.geom
    b = max(1, min(32 // (g.n_q_heads // g.n_kv_heads), g.tail_cap))
    check_verify(w, 0, w.first_t, max(0, g.tail_cap - b), b)


@pytest.mark.parametrize("w", GQA_ODD, ids=lambda w: w.name)
def test_verify_gqa_block8(w):
    """8-token blocks with G = 3, 5, 6, 7: G*8 = 24 .. 56 query rows per kv head, so the rows of
    the last 32-row block are ragged (rows past G*B idle)."""
    check_verify(w, 0, w.first_t, w.geom.tail_cap - 8, 8)


# ---------------------------------------------------------------------------- batched drafts, rotated view
def check_verify_batched(w, layer, t, n_tails, stride, blk, view=None, out_dtype="f32"):
    """S draft blocks over one window in one call: draft d's reasoning rows (seeded per draft)
    at cache rows N + d*stride, its block after them; every draft against oracle_verify with its
    own tail and block, block rows copied bit-exactly, other tail rows untouched.  view: None
    (keys rotated in the kernel), "rotate" (fd_rotate_window), "stream" (a streaming call's
    workspace start) or "persistent" (fd_stream_attn_view's key view, the verify's pos_base
    raised by fd_view_shift)."""
    g = w.geom
    S = len(n_tails)
    H.say(f"batched verify cfg {w.cfg_id} layer {layer} t {t} drafts {S} tails {n_tails} stride {stride} "
          f"B {blk} view {view}")
    kc, vc = H.window_caches(w, layer, t)
    drafts = []
    for d in range(S):
        kt, vt = synth.tail_kv(w, 100 + d, n_tails[d])     # each draft its own reasoning rows
        qb, kb, vb = synth.block_qkv(w, 100 + d, blk)
        r0 = g.window + d * stride
        kc[:, r0: r0 + n_tails[d]] = H.dev(np.transpose(kt, (1, 0, 2)), g)
        vc[:, r0: r0 + n_tails[d]] = H.dev(np.transpose(vt, (1, 0, 2)), g)
        drafts.append((kt, vt, qb, kb, vb))
    q = H.dev(np.stack([x[2] for x in drafts]), g)
    k = H.dev(np.stack([x[3] for x in drafts]), g)
    v = H.dev(np.stack([x[4] for x in drafts]), g)
    kview = None
    if view == "rotate":
        kview = torch.empty((g.n_kv_heads, g.window, g.head_dim), dtype=torch.float16, device=H.DEV)
        fd.rotate_window(g, kc, t, kview)
    elif view == "stream":
        sws = torch.empty(fd.stream_workspace_bytes(g), dtype=torch.uint8, device=H.DEV)
        o = torch.empty((g.n_new, g.n_q_heads, g.head_dim), device=H.DEV)
        fd.stream_attn(g, H.q_new(w, layer, t), kc, vc, t, o, sws)
        kview = sws
    gv = g
    if view == "persistent":   # a persistent view updated at t from the view of t-1, and the
        # verify's positions raised by the view's offset
        kc1, vc1 = H.window_caches(w, layer, t - 1)
        sws = torch.empty(fd.stream_workspace_bytes(g), dtype=torch.uint8, device=H.DEV)
        o = torch.empty((g.n_new, g.n_q_heads, g.head_dim), device=H.DEV)
        kview = torch.empty((g.n_kv_heads, g.window, g.head_dim), dtype=torch.float16, device=H.DEV)
        fd.stream_attn_view(g, H.q_new(w, layer, t - 1), kc1, vc1, t - 1, kview, -1, o, sws)
        H.insert(w, layer, kc1, vc1, t)
        fd.stream_attn_view(g, H.q_new(w, layer, t), kc1, vc1, t, kview, t - 1, o, sws)
        gv = dataclasses.replace(g, pos_base=g.pos_base + fd.view_shift(g, t))
        H.say(f"  persistent view, verify pos_base {gv.pos_base}")
    out = torch.empty((S, blk, g.n_q_heads, g.head_dim),
                      dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16, device=H.DEV)
    ws = torch.full((fd.verify_batched_workspace_bytes(g, S, blk),), 0xAB, dtype=torch.uint8, device=H.DEV)
    fd.verify_attn_batched(gv, q, k, v, kc, vc, t, n_tails, stride, blk, out, ws, k_view=kview,
                           out_dtype=out_dtype)
    got = out.float().cpu().numpy()
    win = fd_oracle.StreamWindow(g, *synth.prefix_kv(w, layer))
    for f in range(t + 1):
        for vv in range(g.n_views):
            win.push(vv, f, *synth.frame_kv(w, layer, vv, f))
    worst = 0.0
    for d, (kt, vt, qb, kb, vb) in enumerate(drafts):
        want = fd_oracle.oracle_verify(g, win, kt, vt, qb, kb, vb)
        worst = max(worst, H.check_out(got[d], want, g, out_dtype, ("batched", d)))
        r0 = g.window + d * stride + n_tails[d]
        assert torch.equal(kc[:, r0: r0 + blk], H.dev(np.transpose(kb, (1, 0, 2)), g))
        assert torch.equal(vc[:, r0: r0 + blk], H.dev(np.transpose(vb, (1, 0, 2)), g))
    end = g.window + (S - 1) * stride + n_tails[-1] + blk
    assert bool((kc[:, end:] == H.SENTINEL).all()) and bool((vc[:, end:] == H.SENTINEL).all())
    H.say(f"  max-abs {worst:.3e} over {S} drafts (tol {H.TOL[g.dtype]})")
    return got


@pytest.mark.parametrize("cid,n_tails,stride,view", [
    (4, [100, 37], 128, None), (4, [0, 5, 17, 33, 12, 30], 42, None), (4, [200], 0, "rotate"),
    (4, [0, 5, 17, 33, 12, 30], 42, "stream"), (2, [20, 3], 32, None), (2, [0, 1, 2, 0, 1, 2], 10, "rotate"),
    (4, [200], 0, "persistent"), (2, [20, 3], 32, "persistent")])
def test_verify_batched(cid, n_tails, stride, view):
    w = synth.CONFIGS[cid]
    check_verify_batched(w, 0, w.first_t + 1, n_tails, stride, 8, view)


def test_verify_batched_block16_and_bf16_out():
    """16-token drafts (two row blocks each) and a bf16 output."""
    w = synth.CONFIGS[4]
    check_verify_batched(w, 3, w.first_t, [40, 3], 100, 16, "rotate")
    check_verify_batched(w, 5, w.first_t, [60, 90, 0], 100, 8, None, out_dtype="bf16")


def test_verify_batched_more_row_blocks_than_resident():
    """Ten row blocks (five 16-token drafts, two 32-row blocks each): more than the kernel keeps
    resident at once, so a window unit reloads queries between its row blocks."""
    w = synth.CONFIGS[2]
    w2 = Workload(w.cfg_id, w.name, w.geom.replace(tail_cap=192), scale=w.scale, first_t=w.first_t)
    check_verify_batched(w2, 0, w.first_t + 1, [20, 3, 17, 0, 9], 40, 16, None)
    check_verify_batched(w2, 1, w.first_t + 2, [12, 3, 10, 0, 9, 1, 5, 2], 22, 8, "rotate")


def test_verify_repeat_bit_identical():
    """Consecutive calls on one workspace (its partial slots reused) give bit-identical outputs:
    single-draft config 4 and a three-draft call with a view."""
    w = synth.CONFIGS[4]
    g = w.geom
    t = w.first_t
    kc, vc = H.window_caches(w, 0, t)
    kt, vt = synth.tail_kv(w, 0, 200)
    kc[:, g.window: g.window + 200] = H.dev(np.transpose(kt, (1, 0, 2)), g)
    vc[:, g.window: g.window + 200] = H.dev(np.transpose(vt, (1, 0, 2)), g)
    qb, kb, vb = (H.dev(x, g) for x in synth.block_qkv(w, 0, 8))
    ws = torch.zeros(fd.verify_workspace_bytes(g, 8), dtype=torch.uint8, device=H.DEV)
    outs = []
    for _ in range(6):
        o = torch.empty((8, g.n_q_heads, g.head_dim), device=H.DEV)
        fd.verify_attn(g, qb, kb, vb, kc, vc, t, 200, 8, o, ws)
        outs.append(o)
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    kview = torch.empty((g.n_kv_heads, g.window, g.head_dim), dtype=torch.float16, device=H.DEV)
    fd.rotate_window(g, kc, t, kview)
    q3 = torch.stack([qb] * 3)
    k3, v3 = torch.stack([kb] * 3), torch.stack([vb] * 3)
    ws3 = torch.zeros(fd.verify_batched_workspace_bytes(g, 3, 8), dtype=torch.uint8, device=H.DEV)
    outs = []
    for _ in range(6):
        o = torch.empty((3, 8, g.n_q_heads, g.head_dim), device=H.DEV)
        fd.verify_attn_batched(g, q3, k3, v3, kc, vc, t, [50, 20, 0], 80, 8, o, ws3, k_view=kview)
        outs.append(o)
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    H.say("  six consecutive calls bit-identical (single draft; three drafts with a view)")


def test_rotate_window_matches_oracle_rotation():
    """fd_rotate_window: every window key rotated at its current position, as the oracle's fp64
    rotation rounded to fp16 (within half an fp16 ulp plus 2^-20 of the pair's input magnitude for
    the fp32 angle and rotation arithmetic); and the streaming call leaves the same bytes at its
    workspace start."""
    for cid in (2, 5):
        w = synth.CONFIGS[cid]
        g = w.geom
        t = w.first_t + 3
        kc, vc = H.window_caches(w, 0, t)
        kview = torch.empty((g.n_kv_heads, g.window, g.head_dim), dtype=torch.float16, device=H.DEV)
        fd.rotate_window(g, kc, t, kview)
        got = kview.float().cpu().numpy().astype(np.float64)
        kraw = kc[:, : g.window].float().cpu().numpy().astype(np.float64)      # [Hkv][W][D]
        pos = np.array([fd.key_position(g, t, x) for x in range(g.window)])
        want = np.transpose(fd_oracle.rope(np.transpose(kraw, (1, 0, 2)), pos, g.rope_theta), (1, 0, 2))
        a = np.maximum(np.abs(want), 2.0 ** -14)
        half_ulp = np.ldexp(1.0, (np.floor(np.log2(a)) - 11).astype(np.int64))
        # fp32 angle and rotation error scales with the pair's input magnitude (a rotated
        # element can cancel to near zero): 2^-20 of |x1| + |x2|
        pair = np.abs(kraw) + np.abs(np.concatenate([kraw[..., 64:], kraw[..., :64]], axis=-1))
        err = np.abs(got - want)
        excess = err - (half_ulp + 2.0 ** -20 * pair + 1e-7)
        i = np.unravel_index(int(np.argmax(excess)), excess.shape)
        assert excess[i] <= 0, ("worst", cid, i, float(got[i]), float(want[i]), float(kraw[i]),
                                float(kraw[i[0], i[1], (i[2] + 64) % 128]), int(pos[i[1]]))
        sws = torch.empty(fd.stream_workspace_bytes(g), dtype=torch.uint8, device=H.DEV)
        o = torch.empty((g.n_new, g.n_q_heads, g.head_dim), device=H.DEV)
        fd.stream_attn(g, H.q_new(w, 0, t), kc, vc, t, o, sws)
        torch.cuda.synchronize()
        assert torch.equal(sws[: kview.numel() * 2].view(torch.float16), kview.reshape(-1))
        H.say(f"  cfg {cid}: rotated window within half an fp16 ulp of the oracle's rotation; "
              f"equal to the streaming workspace's start")


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
    err = H.check_out(got[sel], want, g, out_dtype, ("prefill", w.name, layer))
    H.say(f"  {len(sel)} rows: max-abs {err:.3e} (tol {H.TOL[g.dtype]}"
          f"{' + half bf16 ulp' if out_dtype == 'bf16' else ''})")
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


def test_prefill_backbone_rows():
    """Config 3 shapes (W = 4,608 queries over 4,608 keys), fp32 output: every row of the prefix,
    every row of the segment with the longest key range (the newest frame of the last view) and
    sampled rows of every other segment.  Then the bf16 output of the same call: every row
    equals the fp32 output rounded to bf16 (within half an ulp)."""
    w = synth.CONFIGS[3]
    g = w.geom
    t = w.first_t + 1
    P, T, F = g.prefix_len, g.tok_per_frame, g.n_frames
    last = P + ((g.n_views - 1) * F + t % F) * T          # cache row of that segment's token 0
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([np.arange(P), np.arange(last, last + T),
                                     P + rng.choice(g.window - P, 96, replace=False), [g.window - 1]]))
    got, kc, vc = check_prefill(w, 0, t, rows=rows, out_dtype="f32")
    q, _ = window_queries(w, 0, t)
    ws = torch.empty(fd.prefill_workspace_bytes(g), dtype=torch.uint8, device=H.DEV)
    ob = torch.empty((g.window, g.n_q_heads, g.head_dim), dtype=torch.bfloat16, device=H.DEV)
    fd.prefill_attn(g, H.dev(q, g), kc, vc, t, ob, ws, out_dtype="bf16")
    H.check_bf16_rounding(ob.float().cpu().numpy(), got, "prefill config 3")


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
    err = H.check_out(out.float().cpu().numpy(), oracle_outputs(w, layer, [t])[t], g, out_dtype,
                      ("stream+insert", w.name))
    H.say(f"  bit-identical to insert + stream; max-abs vs oracle {err:.3e}")


@pytest.mark.parametrize("cid,dt", [(1, "f32"), (2, "f32"), (3, "f32"), (3, "bf16")])
def test_stream_insert_fused(cid, dt):
    w = synth.CONFIGS[cid]
    check_stream_insert(w, 0, w.first_t + 1, dt)


@pytest.mark.parametrize("w", EXTRA, ids=lambda w: w.name)
def test_stream_insert_fused_edge_geometries(w):
    check_stream_insert(w, 0, w.first_t + w.geom.n_frames)   # a later ring phase


# ---------------------------------------------------------------------------- persistent key view
def _key_view(g):
    return torch.empty((g.n_kv_heads, g.window, g.head_dim),
                       dtype=torch.float16 if g.dtype == synth.BF16 else torch.float32, device=H.DEV)


def check_view_rolling(w, n_win):
    """fd_stream_attn_insert_view over consecutive windows with the view kept between calls (after
    the first only the prefix and the new frames are rotated; the ring wraps), every row against the
    oracle.  Alongside, on a copy of the cache: the frames inserted separately and
    fd_stream_attn_view, and fd_stream_attn_insert_view rebuilding the whole view every window
    (view_frame -1).  Positions are integers, so a frame row's rotated value is the same whether
    it was rotated when the frame came in or again now: all three outputs are bit-identical."""
    cid = w.cfg_id
    g = w.geom
    ts = list(range(w.first_t, w.first_t + n_win))
    want = oracle_outputs(w, 0, ts)
    kc, vc = H.new_cache(g)
    H.write_prefix(w, 0, kc, vc)
    for t in range(ts[0]):
        H.insert(w, 0, kc, vc, t)
    kc2, vc2, kc3, vc3 = kc.clone(), vc.clone(), kc.clone(), vc.clone()
    views = [_key_view(g) for _ in range(3)]
    ws = torch.empty(fd.stream_workspace_bytes(g), dtype=torch.uint8, device=H.DEV)
    outs = [torch.empty((g.n_new, g.n_q_heads, g.head_dim), device=H.DEV) for _ in range(3)]
    vf = -1
    for t in ts:
        H.say(f"  cfg {cid} window t={t} (view of t={vf})")
        k, v, _ = synth.new_frames(w, 0, t)
        kn, vn, q = H.dev(k, g), H.dev(v, g), H.q_new(w, 0, t)
        fd.stream_attn_insert_view(g, kn, vn, q, kc, vc, t, views[0], vf, outs[0], ws)
        fd.kv_insert_frame(g, kc2, vc2, kn, vn, t)
        fd.stream_attn_view(g, q, kc2, vc2, t, views[1], vf, outs[1], ws)
        fd.stream_attn_insert_view(g, kn, vn, q, kc3, vc3, t, views[2], -1, outs[2], ws)
        vf = t
        torch.cuda.synchronize()
        assert torch.equal(kc, kc2) and torch.equal(vc, vc2) and torch.equal(kc, kc3), "cache images differ"
        assert torch.equal(views[0], views[1]) and torch.equal(views[0], views[2]), "views differ"
        assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2]), "outputs differ"
        err = H.check_out(outs[0].cpu().numpy().astype(np.float64), want[t], g, "f32", ("view", w.name, t))
        H.say(f"    max-abs vs oracle {err:.3e}")


@pytest.mark.parametrize("cid,n_win", [(1, 6), (2, 9), (5, 12)])
def test_stream_view_rolling(cid, n_win):
    check_view_rolling(synth.CONFIGS[cid], n_win)


@pytest.mark.parametrize("w", EXTRA, ids=lambda w: w.name)
def test_stream_view_edge_geometries(w):
    check_view_rolling(w, w.geom.n_frames + 2)


def test_stream_view_offset_wrap():
    """Around the end of an offset period (n = 2^24 / T frames): the window at n-1 (view of n-2),
    at n (the offset wraps to 0: the whole view is rebuilt) and at n+1 (view of n), each against
    the oracle on the window's F frames and bit-identical to a rebuild of the whole view."""
    w = synth.CONFIGS[2]
    g = w.geom
    per = max(1, (1 << 24) // g.tok_per_frame)
    assert fd.view_shift(g, per) == 0 and fd.view_shift(g, per - 1) == (per - 1) * g.tok_per_frame
    t0 = per - 2
    pk, pv = synth.prefix_kv(w, 0)
    win = fd_oracle.StreamWindow(g, pk, pv)
    kc, vc = H.new_cache(g)
    H.write_prefix(w, 0, kc, vc)
    for t in range(t0 - g.n_frames + 1, t0 + 1):   # the ring holds the last F frames
        k, v, _ = synth.new_frames(w, 0, t)
        for vi in range(g.n_views):
            win.push(vi, t, k[vi], v[vi])
        H.insert(w, 0, kc, vc, t)
    ws = torch.empty(fd.stream_workspace_bytes(g), dtype=torch.uint8, device=H.DEV)
    view, full = _key_view(g), _key_view(g)
    out, ref = (torch.empty((g.n_new, g.n_q_heads, g.head_dim), device=H.DEV) for _ in range(2))
    q0 = H.q_new(w, 0, t0)
    fd.stream_attn_view(g, q0, kc, vc, t0, view, -1, out, ws)   # the view of t0
    vf = t0
    qpos = fd_oracle.new_query_positions(g)
    for t in (per - 1, per, per + 1):
        k, v, q = synth.new_frames(w, 0, t)
        for vi in range(g.n_views):
            win.push(vi, t, k[vi], v[vi])
        kc2, vc2 = kc.clone(), vc.clone()
        kn, vn, qd = H.dev(k, g), H.dev(v, g), H.dev(q, g)
        fd.stream_attn_insert_view(g, kn, vn, qd, kc, vc, t, view, vf, out, ws)
        fd.stream_attn_insert_view(g, kn, vn, qd, kc2, vc2, t, full, -1, ref, ws)
        vf = t
        torch.cuda.synchronize()
        assert torch.equal(view, full) and torch.equal(out, ref), t
        kw, vw = win.kv()
        wnt = fd_oracle.attend(q, kw, vw, qpos, fd_oracle.window_positions(g, kw.shape[0]), g.rope_theta)
        err = H.check_out(out.cpu().numpy().astype(np.float64), wnt, g, "f32", ("view wrap", t))
        H.say(f"  t={t} (offset {fd.view_shift(g, t)}): max-abs vs oracle {err:.3e}")


# ---------------------------------------------------------------------------- fp16 operand range
# For bf16 inputs the rotated keys, and the rotated queries scaled by log2(e)/sqrt(D), are
# rounded to fp16 for the Q K^T matrix cores.  A rotated element is x cos - y sin (or
# x sin + y cos) of a stored pair (x, y), so its magnitude never exceeds sqrt(x^2 + y^2):
# stored key elements of +-45,056 (bf16-exact) give at most 63,718, below fp16's largest
# finite value 65,504.  The test puts such keys in one frequency pair of every key and
# queries of +-249,856 (scaled: at most 45,061) in another, with the other operand zero in
# each of those pairs, so the exact scores are those of the remaining pairs: any overflow to
# inf would show up as a NaN (inf * 0) in the outputs.
KBIG, QBIG = 45056.0, 249856.0
PK, PQ = 5, 9        # frequency pairs (i, i + D/2) carrying the large keys / the large queries


def _big_k(a, seed):
    a = np.array(a, np.float32, copy=True)
    h = a.shape[-1] // 2
    sg = np.random.default_rng(seed).choice([-1.0, 1.0], size=a.shape[:-1] + (2,)).astype(np.float32)
    a[..., PK], a[..., PK + h] = KBIG * sg[..., 0], KBIG * sg[..., 1]
    a[..., PQ] = a[..., PQ + h] = 0.0
    return a


def _big_q(a, seed):
    a = np.array(a, np.float32, copy=True)
    h = a.shape[-1] // 2
    sg = np.random.default_rng(seed).choice([-1.0, 1.0], size=a.shape[:-1] + (2,)).astype(np.float32)
    a[..., PQ], a[..., PQ + h] = QBIG * sg[..., 0], QBIG * sg[..., 1]
    a[..., PK] = a[..., PK + h] = 0.0
    return a


def test_rotation_overflow_report():
    """fd_stream_overflow / fd_prefill_overflow (config-2 shapes): 0 for ordinary inputs; a key
    (prefix row) or a query element beyond the fp16 operand bound is counted; a later call on
    the same workspace reports afresh, also a view call whose rotation pass launches fewer
    workgroups than the overflowing whole-window call before it (the last query workgroup of
    that call lies past the smaller grid); the prefill call likewise; a workspace no call has
    written is refused."""
    w = synth.CONFIGS[2]
    g = w.geom
    t = w.first_t
    kc, vc = H.window_caches(w, 0, t)
    q = H.q_new(w, 0, t)
    out = torch.empty((g.n_new, g.n_q_heads, g.head_dim), device=H.DEV)
    ws = torch.zeros(fd.stream_workspace_bytes(g), dtype=torch.uint8, device=H.DEV)
    with pytest.raises(fd.FdError):
        fd.stream_overflow(g, ws)                       # never written: no report
    fd.stream_attn(g, q, kc, vc, t, out, ws)
    assert fd.stream_overflow(g, ws) == 0
    kbig = kc.clone()
    kbig[1, 3, 5] = 1.0e5                               # prefix row 3 of kv head 1
    fd.stream_attn(g, q, kbig, vc, t, out, ws)
    assert fd.stream_overflow(g, ws) >= 1
    qbig = q.clone()
    qbig[g.n_new - 1, g.n_q_heads - 1, 9] = 4.0e6       # x log2(e)/sqrt(128): ~5e5 in fp16 units
    fd.stream_attn(g, qbig, kc, vc, t, out, ws)
    assert fd.stream_overflow(g, ws) >= 1
    fd.stream_attn(g, q, kc, vc, t, out, ws)
    assert fd.stream_overflow(g, ws) == 0
    view = _key_view(g)
    fd.stream_attn_view(g, qbig, kc, vc, t, view, -1, out, ws)      # whole window rotated
    assert fd.stream_overflow(g, ws) >= 1
    fd.stream_attn_view(g, q, kc, vc, t, view, t, out, ws)          # prefix and new frames only
    assert fd.stream_overflow(g, ws) == 0
    pws = torch.empty(fd.prefill_workspace_bytes(g), dtype=torch.uint8, device=H.DEV)
    gen = torch.Generator(device=H.DEV)
    gen.manual_seed(5)
    qw = torch.randn((g.window, g.n_q_heads, g.head_dim), generator=gen, device=H.DEV).to(torch.bfloat16)
    ow = torch.empty((g.window, g.n_q_heads, g.head_dim), device=H.DEV)
    fd.prefill_attn(g, qw, kc, vc, t, ow, pws)
    assert fd.prefill_overflow(g, pws) == 0
    fd.prefill_attn(g, qw, kbig, vc, t, ow, pws)
    assert fd.prefill_overflow(g, pws) >= 1
    fd.prefill_attn(g, qw, kc, vc, t, ow, pws)
    assert fd.prefill_overflow(g, pws) == 0


def test_fp16_operand_bound():
    """Streaming, batched verify with and without a rotated view, and single verify at the
    fp16 operand bound (config-2 shapes, two ring phases): finite and within the bf16
    tolerance of the oracle."""
    w = synth.CONFIGS[2]
    g = w.geom
    layer, t_last = 0, w.first_t + 1
    pk, pv = synth.prefix_kv(w, layer)
    pk = _big_k(pk, 1)
    win = fd_oracle.StreamWindow(g, pk, pv)
    kc, vc = H.new_cache(g)
    kc[:, : g.prefix_len, :] = H.dev(np.transpose(pk, (1, 0, 2)), g)
    vc[:, : g.prefix_len, :] = H.dev(np.transpose(pv, (1, 0, 2)), g)
    assert float(kc.abs().max()) == KBIG
    for t in range(t_last + 1):
        ks, vs = [], []
        for v in range(g.n_views):
            k, vv = synth.frame_kv(w, layer, v, t)
            k = _big_k(k, 100 + 8 * t + v)
            win.push(v, t, k, vv)
            ks.append(k)
            vs.append(vv)
        fd.kv_insert_frame(g, kc, vc, H.dev(np.stack(ks), g), H.dev(np.stack(vs), g), t)
        if t < t_last - 1:
            continue
        q = _big_q(np.concatenate([synth.frame_q(w, layer, v, t) for v in range(g.n_views)]), 7 + t)
        want = fd_oracle.oracle_stream(g, win, q)
        assert np.isfinite(want).all()
        got = H.stream_out(w, layer, kc, vc, t, q=H.dev(q, g))
        err = H.check_out(got.float().cpu().numpy(), want, g, "f32", ("fp16 bound stream", t))
        H.say(f"  fp16 bound: stream t {t} max-abs {err:.3e}")
    # verify: one draft through fd_verify_attn, two drafts through the batched call (rotated
    # view from fd_rotate_window), every tail and block at the bound too
    n_tails, stride, B = [12, 5], 32, 8
    kview = torch.empty((g.n_kv_heads, g.window, g.head_dim), dtype=torch.float16, device=H.DEV)
    fd.rotate_window(g, kc, t_last, kview)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(kview).all()) and float(kview.abs().max()) > 6.0e4
    qs, kbs, vbs, wants = [], [], [], []
    for d, nt in enumerate(n_tails):
        kt, vt = synth.tail_kv(w, 200 + d, nt)
        kt = _big_k(kt, 300 + d)
        qb, kb, vb = synth.block_qkv(w, 200 + d, B)
        qb, kb = _big_q(qb, 400 + d), _big_k(kb, 500 + d)
        r0 = g.window + d * stride
        kc[:, r0: r0 + nt] = H.dev(np.transpose(kt, (1, 0, 2)), g)
        vc[:, r0: r0 + nt] = H.dev(np.transpose(vt, (1, 0, 2)), g)
        wants.append(fd_oracle.oracle_verify(g, win, kt, vt, qb, kb, vb))
        qs.append(qb)
        kbs.append(kb)
        vbs.append(vb)
    for view in (None, kview):
        out = torch.empty((2, B, g.n_q_heads, g.head_dim), dtype=torch.float32, device=H.DEV)
        ws = torch.empty(fd.verify_batched_workspace_bytes(g, 2, B), dtype=torch.uint8, device=H.DEV)
        fd.verify_attn_batched(g, H.dev(np.stack(qs), g), H.dev(np.stack(kbs), g), H.dev(np.stack(vbs), g), kc, vc,
                               t_last, n_tails, stride, B, out, ws, k_view=view)
        for d in range(2):
            err = H.check_out(out[d].cpu().numpy(), wants[d], g, "f32", ("fp16 bound batched", d))
            H.say(f"  fp16 bound: batched verify draft {d} view {view is not None} max-abs {err:.3e}")
    out = torch.empty((B, g.n_q_heads, g.head_dim), dtype=torch.float32, device=H.DEV)
    ws = torch.empty(fd.verify_workspace_bytes(g, B), dtype=torch.uint8, device=H.DEV)
    fd.verify_attn(g, H.dev(qs[0], g), H.dev(kbs[0], g), H.dev(vbs[0], g), kc, vc, t_last, n_tails[0], B, out, ws)
    err = H.check_out(out.cpu().numpy(), wants[0], g, "f32", "fp16 bound verify")
    H.say(f"  fp16 bound: verify max-abs {err:.3e}")
