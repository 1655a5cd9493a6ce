"""The per-window loop captured in HIP graphs.

A window step is, per layer: insert the new frame of every view, streaming-prefill attention
of the new frames, and an 8-token verify.  Every kernel argument depends on the newest frame
index t only through t mod F (ring slot and ages), so F graphs, one per ring phase, replay any
stream.  The library allocates nothing and synchronises nothing inside a call, so the calls
capture as they are.  These tests replay the graphs over a rolling sequence of windows, with
the program's own eager work and synchronisations between replays, and compare every replay
bit for bit with the same calls launched eagerly on an identical copy of the caches, and (on
seeded inputs) with the fp64 oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.fd_oracle as fd_oracle
from streaming_kv_cache_view_amd import fd, synth

try:
    from . import gpu_harness as H
except ImportError:
    import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fd.lib()


class Window:
    """Static device buffers of one window step over `layers` layers (a graph reads and
    writes these same buffers on every replay)."""

    def __init__(self, g, layers, n_tail, blk, gen, fused=False):
        rnd = lambda *s: torch.randn(*s, generator=gen, device=H.DEV).to(torch.bfloat16)
        self.g, self.L, self.n_tail, self.blk, self.fused = g, layers, n_tail, blk, fused
        self.kc = [rnd(g.n_kv_heads, g.cache_rows, g.head_dim) for _ in range(layers)]
        self.vc = [rnd(g.n_kv_heads, g.cache_rows, g.head_dim) for _ in range(layers)]
        self.kn = [torch.empty(g.n_views, g.tok_per_frame, g.n_kv_heads, g.head_dim, dtype=torch.bfloat16,
                               device=H.DEV) for _ in range(layers)]
        self.vn = [torch.empty_like(x) for x in self.kn]
        self.qn = [torch.empty(g.n_new, g.n_q_heads, g.head_dim, dtype=torch.bfloat16, device=H.DEV)
                   for _ in range(layers)]
        self.qb = [torch.empty(blk, g.n_q_heads, g.head_dim, dtype=torch.bfloat16, device=H.DEV)
                   for _ in range(layers)]
        self.kb = [torch.empty(blk, g.n_kv_heads, g.head_dim, dtype=torch.bfloat16, device=H.DEV)
                   for _ in range(layers)]
        self.vb = [torch.empty_like(x) for x in self.kb]
        self.out = [torch.empty(g.n_new, g.n_q_heads, g.head_dim, device=H.DEV) for _ in range(layers)]
        self.vout = [torch.empty(blk, g.n_q_heads, g.head_dim, device=H.DEV) for _ in range(layers)]
        self.sws = torch.empty(fd.stream_workspace_bytes(g), dtype=torch.uint8, device=H.DEV)
        self.vws = torch.empty(fd.verify_workspace_bytes(g, blk), dtype=torch.uint8, device=H.DEV)

    def clone_caches_from(self, other):
        for a, b in zip(self.kc + self.vc, other.kc + other.vc):
            a.copy_(b)

    def load_inputs(self, src):
        """Copy one window's frame, query and block inputs (lists per layer) into the buffers."""
        for name in ("kn", "vn", "qn", "qb", "kb", "vb"):
            for dst, x in zip(getattr(self, name), src[name]):
                dst.copy_(x)

    def step(self, t):
        g = self.g
        for l in range(self.L):
            if self.fused:   # insert + attention in one launch sequence
                fd.stream_attn_insert(g, self.kn[l], self.vn[l], self.qn[l], self.kc[l], self.vc[l], t,
                                      self.out[l], self.sws)
            else:
                fd.kv_insert_frame(g, self.kc[l], self.vc[l], self.kn[l], self.vn[l], t)
                fd.stream_attn(g, self.qn[l], self.kc[l], self.vc[l], t, self.out[l], self.sws)
            fd.verify_attn(g, self.qb[l], self.kb[l], self.vb[l], self.kc[l], self.vc[l], t, self.n_tail,
                           self.blk, self.vout[l], self.vws)


def window_inputs(g, layers, blk, gen):
    rnd = lambda *s: torch.randn(*s, generator=gen, device=H.DEV).to(torch.bfloat16)
    return {
        "kn": [rnd(g.n_views, g.tok_per_frame, g.n_kv_heads, g.head_dim) for _ in range(layers)],
        "vn": [rnd(g.n_views, g.tok_per_frame, g.n_kv_heads, g.head_dim) for _ in range(layers)],
        "qn": [rnd(g.n_new, g.n_q_heads, g.head_dim) for _ in range(layers)],
        "qb": [rnd(blk, g.n_q_heads, g.head_dim) for _ in range(layers)],
        "kb": [rnd(blk, g.n_kv_heads, g.head_dim) for _ in range(layers)],
        "vb": [rnd(blk, g.n_kv_heads, g.head_dim) for _ in range(layers)],
    }


@pytest.mark.parametrize("cid,layers,fused", [(3, 3, False), (5, 2, False), (3, 2, True)])
def test_graph_rolling_windows_match_eager(cid, layers, fused):
    w = synth.CONFIGS[cid]
    g = w.geom
    F, blk, n_tail = g.n_frames, 8, min(200, g.tail_cap - 8)
    gen = torch.Generator(device=H.DEV)
    gen.manual_seed(20 + cid)
    eager = Window(g, layers, n_tail, blk, gen)   # eager: the separate insert and attention calls
    graphed = Window(g, layers, n_tail, blk, gen, fused)
    graphed.clone_caches_from(eager)
    t0 = F   # window full
    # one graph per ring phase, captured on a side stream (capture does not run the kernels)
    graphs = {}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for t in range(t0, t0 + F):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=side):
                graphed.step(t)
            graphs[t % F] = gr
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    n_windows = 2 * F + 1
    for i in range(n_windows):
        t = t0 + i
        src = window_inputs(g, layers, blk, gen)
        eager.load_inputs(src)
        eager.step(t)
        graphed.load_inputs(src)
        graphs[t % F].replay()
        torch.cuda.synchronize()
        for l in range(layers):
            assert torch.equal(eager.out[l], graphed.out[l]), (cid, t, l, "stream")
            assert torch.equal(eager.vout[l], graphed.vout[l]), (cid, t, l, "verify")
        H.say(f"  cfg {cid} window t={t} (graph phase {t % F}): stream and verify outputs bit-identical")
    for a, b in zip(eager.kc + eager.vc, graphed.kc + graphed.vc):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------- replays against the oracle
def _oracle_window(w, layer, upto):
    """The oracle's logical window after frames 0..upto of every view (seeded inputs)."""
    g = w.geom
    win = fd_oracle.StreamWindow(g, *synth.prefix_kv(w, layer))
    for f in range(upto + 1):
        for v in range(g.n_views):
            win.push(v, f, *synth.frame_kv(w, layer, v, f))
    return win


class SeededStep:
    """One layer's window step on static device buffers, fed from the seeded generator: insert
    the new frame of every view (or the fused insert + attention call), streaming-prefill
    attention, and the verify of a fixed draft block after n_tail fixed reasoning rows."""

    def __init__(self, w, layer, n_tail, blk, fused):
        g = self.g = w.geom
        self.w, self.layer, self.n_tail, self.blk, self.fused = w, layer, n_tail, blk, fused
        self.kc, self.vc = H.new_cache(g)
        H.write_prefix(w, layer, self.kc, self.vc)
        self.kt, self.vt = synth.tail_kv(w, layer, n_tail)
        self.kc[:, g.window: g.window + n_tail] = H.dev(np.transpose(self.kt, (1, 0, 2)), g)
        self.vc[:, g.window: g.window + n_tail] = H.dev(np.transpose(self.vt, (1, 0, 2)), g)
        self.qb_h, self.kb_h, self.vb_h = synth.block_qkv(w, layer, blk)
        self.qb, self.kb, self.vb = H.dev(self.qb_h, g), H.dev(self.kb_h, g), H.dev(self.vb_h, g)
        td = H.tdtype(g)
        self.kn = torch.empty((g.n_views, g.tok_per_frame, g.n_kv_heads, g.head_dim), dtype=td, device=H.DEV)
        self.vn = torch.empty_like(self.kn)
        self.qn = torch.empty((g.n_new, g.n_q_heads, g.head_dim), dtype=td, device=H.DEV)
        self.out = torch.empty((g.n_new, g.n_q_heads, g.head_dim), device=H.DEV)
        self.vout = torch.empty((blk, g.n_q_heads, g.head_dim), device=H.DEV)
        self.sws = torch.empty(fd.stream_workspace_bytes(g), dtype=torch.uint8, device=H.DEV)
        self.vws = torch.empty(fd.verify_workspace_bytes(g, blk), dtype=torch.uint8, device=H.DEV)

    def load(self, t):
        """Frame t's K, V and queries of every view into the static input buffers."""
        k, v, q = synth.new_frames(self.w, self.layer, t)
        self.kn.copy_(H.dev(k, self.g))
        self.vn.copy_(H.dev(v, self.g))
        self.qn.copy_(H.dev(q, self.g))
        return q

    def step(self, t):
        g = self.g
        if self.fused:
            fd.stream_attn_insert(g, self.kn, self.vn, self.qn, self.kc, self.vc, t, self.out, self.sws)
        else:
            fd.kv_insert_frame(g, self.kc, self.vc, self.kn, self.vn, t)
            fd.stream_attn(g, self.qn, self.kc, self.vc, t, self.out, self.sws)
        fd.verify_attn(g, self.qb, self.kb, self.vb, self.kc, self.vc, t, self.n_tail, self.blk, self.vout,
                       self.vws)


def _capture(st, ts):
    graphs = {}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for t in ts:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=side):
                st.step(t)
            graphs[t % st.g.n_frames] = gr
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return graphs


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replays_match_oracle_config2(fused):
    """Config-2 shapes (bf16), seeded inputs: F graphs (one per ring phase) replayed over 2F+1
    consecutive windows; every replay's streaming and verify outputs against the fp64 oracle."""
    w = synth.CONFIGS[2]
    g = w.geom
    F, layer, n_tail, blk = g.n_frames, 0, 40, 8
    st = SeededStep(w, layer, n_tail, blk, fused)
    for f in range(F - 1):   # warm-up inserts, eager
        H.insert(w, layer, st.kc, st.vc, f)
    graphs = _capture(st, range(F - 1, 2 * F - 1))
    win = _oracle_window(w, layer, F - 2)
    worst = 0.0
    for t in range(F - 1, F - 1 + 2 * F + 1):
        q = st.load(t)
        torch.cuda.synchronize()
        graphs[t % F].replay()
        torch.cuda.synchronize()
        for v in range(g.n_views):
            win.push(v, t, *synth.frame_kv(w, layer, v, t))
        err = H.max_err(st.out.cpu().numpy(), fd_oracle.oracle_stream(g, win, q))
        verr = H.max_err(st.vout.cpu().numpy(),
                         fd_oracle.oracle_verify(g, win, st.kt, st.vt, st.qb_h, st.kb_h, st.vb_h))
        worst = max(worst, err, verr)
        H.say(f"  cfg 2 replay t={t} (phase {t % F}): stream {err:.3e}, verify {verr:.3e}")
        assert err <= H.TOL[g.dtype] and verr <= H.TOL[g.dtype], (t, err, verr)
    H.say(f"  worst over {2 * F + 1} replays: {worst:.3e}")


def test_graph_replay_matches_oracle_config5():
    """One config-5 window (8,704 keys, 1 % 8-sigma K/V outliers) replayed from a graph: sampled
    streaming rows and the whole verify output against the fp64 oracle."""
    w = synth.CONFIGS[5]
    g = w.geom
    F, layer, n_tail, blk = g.n_frames, 0, 200, 8
    st = SeededStep(w, layer, n_tail, blk, fused=True)
    for f in range(F):
        H.insert(w, layer, st.kc, st.vc, f)
    t = F
    graphs = _capture(st, [t])
    q = st.load(t)
    torch.cuda.synchronize()
    graphs[t % F].replay()
    torch.cuda.synchronize()
    win = _oracle_window(w, layer, t)
    rows = np.sort(np.random.default_rng(9).choice(g.n_new, 64, replace=False))
    kw, vw = win.kv()
    want = fd_oracle.attend(q[rows], kw, vw, fd_oracle.new_query_positions(g)[rows],
                            fd_oracle.window_positions(g, kw.shape[0]), g.rope_theta)
    err = H.max_err(st.out.cpu().numpy()[rows], want)
    verr = H.max_err(st.vout.cpu().numpy(),
                     fd_oracle.oracle_verify(g, win, st.kt, st.vt, st.qb_h, st.kb_h, st.vb_h))
    H.say(f"  cfg 5 replay t={t}: stream (64 rows) {err:.3e}, verify {verr:.3e}")
    assert err <= H.TOL[g.dtype] and verr <= H.TOL[g.dtype]
