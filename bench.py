"""Benchmark of the streaming-prefill attention hot path on one MI355X.

One step = one window of the 36-layer backbone, for every layer:
    insert               new frame of 4 views -> ring slot
    streaming prefill    1,024 new-frame queries over 4,608 keys      (config 3)
        (the two through fd_stream_attn_insert_view, which copies the frame in the rotation pass
        and keeps the layer's keys rotated in a persistent view: after the first window only the
        prefix and the new frames are rotated)
    fd_verify_attn       8-token block over 4,608 + 200 + 8 keys      (config 4)
with 36 independent per-layer caches (717 MB of K/V, beyond the 256 MB Infinity Cache),
the ring advancing one frame per step.  Inputs are synthetic, seeded, resident in HBM.

Prints one JSON line.  `value` is the streaming-prefill attention throughput over the
whole step (algorithmic FLOPs = 4*D*Hq*unmasked (q,k) pairs, divided by the step time);
`roofline` is the streaming-prefill call (its kernels timed together with HIP events on
the stream they run on); `roofline_verify` the verify call (its two kernels).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "streaming-prefill attn TFLOP/s + verify KV GB/s, % of MI355X roofline"
KERNEL_SOURCES = ("streaming_kv_cache_view_amd/csrc/fd_kernels.hip",
                  "streaming_kv_cache_view_amd/csrc/fd_internal.h",
                  "streaming_kv_cache_view_amd/csrc/fd_api.cpp")
COPY_MIB = 512


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(profile: str):
    """HBM bytes per call from a committed counter summary under profiles/, or None.

    The summary records the hash of the kernel sources its counters were taken on
    (`source_sha256:`) and the copy-calibrated bytes per call (`traffic_bytes_per_call:`);
    once the sources have changed the figure no longer describes the kernel and None is
    returned."""
    try:
        with open(os.path.join(ROOT, "profiles", profile)) as f:
            text = f.read()
    except OSError:
        return None
    h = re.search(r"^source_sha256: ([0-9a-f]{64})\s*$", text, re.M)
    t = re.search(r"^traffic_bytes_per_call: (\d+)\s*$", text, re.M)
    if not (h and t) or h.group(1) != kernel_source_hash():
        return None
    return int(t.group(1))


def calibrate_copy():
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters:
    each dispatch reads and writes COPY_MIB MiB exactly once."""
    import torch
    n = COPY_MIB << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "dispatches": 4}), flush=True)


def stream_pairs(g) -> int:
    """Unmasked (query, key) pairs per head: token i of view v sees P + v*F*T + (F-1)*T + i + 1 keys."""
    tot = 0
    for v in range(g.n_views):
        base = g.prefix_len + v * g.n_frames * g.tok_per_frame + (g.n_frames - 1) * g.tok_per_frame
        tot += g.tok_per_frame * base + g.tok_per_frame * (g.tok_per_frame + 1) // 2
    return tot


def verify_pairs(g, n_tail, blk) -> int:
    return blk * (g.window + n_tail) + blk * (blk + 1) // 2


def verify_bytes(g, n_tail, blk, esz=2) -> int:
    """Algorithmic bytes of one verify call: the window's, the tail's and the block's K and V
    read once, the block's queries read and the fp32 outputs written."""
    return ((g.window + n_tail + blk) * g.n_kv_heads * g.head_dim * esz * 2
            + blk * g.n_q_heads * g.head_dim * esz + blk * g.n_q_heads * g.head_dim * 4)


def cpu_baseline(seconds: float = 24.0):
    """The fp64 oracle (as it stands) on bounded samples of the same workloads, each leg given
    about a third of `seconds` (whole units only, at least one): config-3 streaming-prefill
    layers, config-4 verify layers (of 36) and consecutive config-5 rolling windows.  Inputs
    are generated outside the timed region; only the oracle's attention calls (full window
    re-rotation, explicit mask) are timed.  Rates use the GPU legs' algorithmic FLOP and byte
    counts."""
    import oracle.fd_oracle as fd_oracle
    from streaming_kv_cache_view_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    leg = seconds / 3

    def window(w, layer, t):
        g = w.geom
        pk, pv = synth.prefix_kv(w, layer)
        win = fd_oracle.StreamWindow(g, pk, pv)
        for f in range(t + 1):
            for v in range(g.n_views):
                k, vv = synth.frame_kv(w, layer, v, f)
                win.push(v, f, k, vv)
        return win

    # config 3: streaming prefill, one layer after another
    w3 = synth.CONFIGS[3]
    g3 = w3.geom
    t_s, n_s = 0.0, 0
    while n_s < 36 and (n_s == 0 or t_s < leg):
        win = window(w3, n_s, w3.first_t)
        q = np.concatenate([synth.frame_q(w3, n_s, v, w3.first_t) for v in range(g3.n_views)])
        t0 = time.perf_counter()
        fd_oracle.oracle_stream(g3, win, q)
        t_s += time.perf_counter() - t0
        n_s += 1
    stream_tf = 4 * g3.head_dim * g3.n_q_heads * stream_pairs(g3) * n_s / t_s / 1e12
    # config 4: the 8-token verify, one layer after another (all 36 when they fit)
    w4 = synth.CONFIGS[4]
    g4 = w4.geom
    t_v, n_v = 0.0, 0
    while n_v < 36 and (n_v == 0 or t_v < leg):
        win = window(w4, n_v, w4.first_t)
        kt, vt = synth.tail_kv(w4, n_v, w4.n_tail)
        qb, kb, vb = synth.block_qkv(w4, n_v, w4.blk_len)
        t0 = time.perf_counter()
        fd_oracle.oracle_verify(g4, win, kt, vt, qb, kb, vb)
        t_v += time.perf_counter() - t0
        n_v += 1
    ver_gbs = verify_bytes(g4, w4.n_tail, w4.blk_len) * n_v / t_v / 1e9
    # config 5: consecutive rolling windows of layer 0 from the first full one
    w5 = synth.CONFIGS[5]
    g5 = w5.geom
    pk, pv = synth.prefix_kv(w5, 0)
    win = fd_oracle.StreamWindow(g5, pk, pv)
    t_5, n_5, t = 0.0, 0, 0
    while n_5 < w5.windows and (n_5 == 0 or t_5 < leg):
        for v in range(g5.n_views):
            k, vv = synth.frame_kv(w5, 0, v, t)
            win.push(v, t, k, vv)
        if t >= w5.first_t:
            q = np.concatenate([synth.frame_q(w5, 0, v, t) for v in range(g5.n_views)])
            t0 = time.perf_counter()
            fd_oracle.oracle_stream(g5, win, q)
            t_5 += time.perf_counter() - t0
            n_5 += 1
        t += 1
    c5_tf = 4 * g5.head_dim * g5.n_q_heads * stream_pairs(g5) * n_5 / t_5 / 1e12
    return {
        "value": round(stream_tf, 5),
        "unit": "TFLOP/s",
        "cores": min(cores, blas_threads),
        "cores_visible": cores,
        "blas_threads": blas_threads,
        "kind": "oracle",
        "sample": f"fp64 oracle, inputs generated untimed: streaming prefill of config 3, layers 0..{n_s - 1} "
                  f"of 36 ({t_s:.1f} s); value is this leg",
        "verify": {"value": round(ver_gbs, 4), "unit": "GB/s",
                   "sample": f"config-4 verify (8-token block over 4608+{w4.n_tail}+{w4.blk_len} keys), "
                             f"layers 0..{n_v - 1} of 36 ({t_v:.1f} s)"},
        "config5": {"value": round(c5_tf, 5), "unit": "TFLOP/s",
                    "sample": f"config-5 rolling windows 0..{n_5 - 1} of 100, layer 0 ({t_5:.1f} s)"},
    }


def rolling_windows(g, n_windows, gen, host_ahead):
    """Times n_windows consecutive windows of one layer: per window the fused insert + streaming
    attention call (fd_stream_attn_insert), back to back behind a queued GPU spin, HIP events
    around the sweep; and the same sweep of the attention call alone over the same windows."""
    import torch
    from streaming_kv_cache_view_amd import fd
    dev = "cuda"
    rnd = lambda *s: torch.randn(*s, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    kc = rnd(g.n_kv_heads, g.cache_rows, g.head_dim)
    vc = rnd(g.n_kv_heads, g.cache_rows, g.head_dim)
    n_in = 8   # distinct input sets, used in turn
    kn = [rnd(g.n_views, g.tok_per_frame, g.n_kv_heads, g.head_dim) for _ in range(n_in)]
    vn = [rnd(g.n_views, g.tok_per_frame, g.n_kv_heads, g.head_dim) for _ in range(n_in)]
    qn = [rnd(g.n_new, g.n_q_heads, g.head_dim) for _ in range(n_in)]
    out = torch.empty(g.n_new, g.n_q_heads, g.head_dim, device=dev)
    sws = torch.empty(fd.stream_workspace_bytes(g), dtype=torch.uint8, device=dev)
    t0 = g.n_frames   # frames 0 .. F-1 are in the cache

    def sweep(fused):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        host_ahead()
        e0.record()
        for w in range(n_windows):
            t = t0 + w
            if fused:
                fd.stream_attn_insert(g, kn[w % n_in], vn[w % n_in], qn[w % n_in], kc, vc, t, out, sws)
            else:
                fd.stream_attn(g, qn[w % n_in], kc, vc, t, out, sws)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n_windows * 1e3

    kview = torch.empty(g.n_kv_heads, g.window, g.head_dim, dtype=torch.float16, device=dev)

    def sweep_view(fused):
        # the persistent key view carried from window to window (the first one builds it whole)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        host_ahead()
        e0.record()
        for w in range(n_windows):
            t = t0 + w
            if fused:
                fd.stream_attn_insert_view(g, kn[w % n_in], vn[w % n_in], qn[w % n_in], kc, vc, t, kview, t - 1,
                                           out, sws)
            else:
                fd.stream_attn_view(g, qn[w % n_in], kc, vc, t, kview, t - 1, out, sws)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n_windows * 1e3

    sweep(True)   # warm-up
    fused_us = min(sweep(True) for _ in range(2))
    att_us = min(sweep(False) for _ in range(2))
    fd.stream_attn_view(g, qn[0], kc, vc, t0 - 1, kview, -1, out, sws)   # the view of the window before
    sweep_view(True)
    fused_view_us = min(sweep_view(True) for _ in range(2))
    att_view_us = min(sweep_view(False) for _ in range(2))
    flops = 4 * g.head_dim * g.n_q_heads * stream_pairs(g)
    tf = flops / (att_view_us * 1e-6) / 1e12
    return {
        "windows": n_windows,
        "stream_view_us_per_window": round(att_view_us, 2),
        "stream_insert_view_us_per_window": round(fused_view_us, 2),
        "stream_us_per_window": round(att_us, 2),
        "stream_insert_us_per_window": round(fused_us, 2),
        "gflop_per_window": round(flops / 1e9, 2),
        "achieved_tflops": round(tf, 2),
        "frac": round(tf / PEAK_BF16_TFLOPS, 4),
        "note": "100 rolling windows of one layer at 8,704 keys (V=4, F=8, T=256, P=512, 32/8 heads, D=128); "
                "fd_stream_attn_view per window with the persistent key view carried between windows (the "
                "attention alone, rate and frac) and fd_stream_attn_insert_view (the window step with its "
                "insert); beside them the same without a view (fd_stream_attn, fd_stream_attn_insert: the "
                "whole window rotated every call); HIP events around each 100-window sweep; timing inputs "
                "N(0,1) bf16",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=24.0,
                    help="oracle sample length over its three legs (config-3 layers, config-4 verify "
                         "layers, config-5 windows; whole units)")
    ap.add_argument("--core-only", action="store_true",
                    help="only the window step and its per-call timing (no block-16 verify, no graph "
                         "replay): the per-kernel averages of a profiled run then cover one call type each")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this path has no multi-GPU leg (heads would shard "
              "across GPUs with no exchange inside attention); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    import torch
    from streaming_kv_cache_view_amd import fd, synth

    dev = "cuda"
    w3, w4 = synth.CONFIGS[3], synth.CONFIGS[4]
    g = w3.geom
    assert w4.geom == g
    L = args.layers
    n_tail, blk = w4.n_tail, w4.blk_len
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    rnd = lambda *s: torch.randn(*s, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    kc = [rnd(g.n_kv_heads, g.cache_rows, g.head_dim) for _ in range(L)]
    vc = [rnd(g.n_kv_heads, g.cache_rows, g.head_dim) for _ in range(L)]
    kn = [rnd(g.n_views, g.tok_per_frame, g.n_kv_heads, g.head_dim) for _ in range(L)]
    vn = [rnd(g.n_views, g.tok_per_frame, g.n_kv_heads, g.head_dim) for _ in range(L)]
    qn = [rnd(g.n_new, g.n_q_heads, g.head_dim) for _ in range(L)]
    out = [torch.empty(g.n_new, g.n_q_heads, g.head_dim, device=dev) for _ in range(L)]
    qb = [rnd(blk, g.n_q_heads, g.head_dim) for _ in range(L)]
    kb = [rnd(blk, g.n_kv_heads, g.head_dim) for _ in range(L)]
    vb = [rnd(blk, g.n_kv_heads, g.head_dim) for _ in range(L)]
    vout = [torch.empty(blk, g.n_q_heads, g.head_dim, device=dev) for _ in range(L)]
    ws = torch.empty(max(fd.verify_workspace_bytes(g, blk), fd.verify_batched_workspace_bytes(g, 1, blk)),
                     dtype=torch.uint8, device=dev)
    sws = torch.empty(fd.stream_workspace_bytes(g), dtype=torch.uint8, device=dev)   # shared by layers
    kview = [torch.empty(g.n_kv_heads, g.window, g.head_dim, dtype=torch.float16, device=dev) for _ in range(L)]
    vframe = [-1] * L   # the frame each layer's key view reflects (-1: none yet)
    torch.cuda.synchronize()

    frame = [g.n_frames]   # newest frame index; the window starts full

    def host_ahead():
        """Queue a spin of some milliseconds on the GPU before a per-call timing sweep: the host
        enqueues the sweep's calls while it runs, so they execute back to back and an event
        pair brackets one call's kernels, not the host's time to issue the next call."""
        torch.cuda._sleep(12_000_000)

    def view_geom(t):
        """The geometry whose positions carry the key views' offset at frame t: a verify over a
        view reads its window keys from it and rotates its own rows at these positions."""
        return g.replace(pos_base=g.pos_base + fd.view_shift(g, t))

    def step():
        """One window: per layer the new frames' insert fused with the streaming-prefill call over
        the layer's persistent key view (after the first window only the prefix and the new frames
        are rotated), then the verify with its window keys read from that view."""
        t = frame[0]
        gv = view_geom(t)
        for l in range(L):
            fd.stream_attn_insert_view(g, kn[l], vn[l], qn[l], kc[l], vc[l], t, kview[l], vframe[l], out[l], sws)
            vframe[l] = t
            fd.verify_attn_batched(gv, qb[l], kb[l], vb[l], kc[l], vc[l], t, [n_tail], 0, blk, vout[l], ws,
                                   k_view=kview[l])
        frame[0] += 1

    def step_plain():
        """The same window without a key view: every call rotates the whole window."""
        t = frame[0]
        for l in range(L):
            fd.stream_attn_insert(g, kn[l], vn[l], qn[l], kc[l], vc[l], t, out[l], sws)
            fd.verify_attn(g, qb[l], kb[l], vb[l], kc[l], vc[l], t, n_tail, blk, vout[l], ws)
        frame[0] += 1

    def timed_steps(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # whole-step timing
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    ms_per_step = timed_steps(step, args.steps)
    plain_ms_per_step = None
    if not args.core_only:
        step_plain()
        plain_ms_per_step = timed_steps(step_plain, max(2, args.steps // 2))
        for l in range(L):
            vframe[l] = -1   # the plain steps left the views behind

    # per-call timing: each call type swept over the layers back to back behind a queued GPU spin,
    # two HIP events (on the stream the kernels are launched on) around each sweep, so a figure is
    # the average time per call with its launch gaps but no event packets between calls
    def sweep(call, reps):
        ms = []
        for rep_i in range(1 + reps):   # the first sweep is a warm-up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            host_ahead()
            e0.record()
            for l in range(L):
                call(l)
            e1.record()
            torch.cuda.synchronize()
            if rep_i > 0:
                ms.append(e0.elapsed_time(e1) / L)
        return ms

    t_pc = frame[0]
    reps = max(2, args.steps // 4)
    ins_ms = sweep(lambda l: fd.kv_insert_frame(g, kc[l], vc[l], kn[l], vn[l], t_pc), reps)
    plain = not args.core_only   # core-only (profiled runs): the view calls only, so that every
    # rotation-pass launch in a trace covers the same rows
    att_ms = sweep(lambda l: fd.stream_attn(g, qn[l], kc[l], vc[l], t_pc, out[l], sws), reps) if plain else None
    ver_ms = sweep(lambda l: fd.verify_attn(g, qb[l], kb[l], vb[l], kc[l], vc[l], t_pc, n_tail, blk, vout[l], ws),
                   reps)
    si_ms = (sweep(lambda l: fd.stream_attn_insert(g, kn[l], vn[l], qn[l], kc[l], vc[l], t_pc, out[l], sws), reps)
             if plain else None)
    for l in range(L):   # each layer's view of t_pc (the insert sweeps above put frame t_pc in the cache):
        # from the view of the last step (t_pc - 1), or rebuilt whole after the plain steps
        fd.stream_attn_view(g, qn[l], kc[l], vc[l], t_pc, kview[l], vframe[l], out[l], sws)
        vframe[l] = t_pc
    # with the view of t_pc: a call rotates the prefix and the newest slot, as one from the view of t_pc - 1
    attv_ms = sweep(lambda l: fd.stream_attn_view(g, qn[l], kc[l], vc[l], t_pc, kview[l], t_pc, out[l], sws), reps)
    siv_ms = sweep(lambda l: fd.stream_attn_insert_view(g, kn[l], vn[l], qn[l], kc[l], vc[l], t_pc, kview[l], t_pc,
                                                        out[l], sws), reps)
    gv_pc = view_geom(t_pc)
    verv_ms = sweep(lambda l: fd.verify_attn_batched(gv_pc, qb[l], kb[l], vb[l], kc[l], vc[l], t_pc, [n_tail], 0, blk,
                                                     vout[l], ws, k_view=kview[l]), reps)
    mean = lambda a: sum(a) / len(a)
    med = lambda a: sorted(a)[len(a) // 2]
    att_us = mean(att_ms) * 1e3 if plain else None
    ver_us, ins_us = mean(ver_ms) * 1e3, mean(ins_ms) * 1e3
    attv_us, verv_us = mean(attv_ms) * 1e3, mean(verv_ms) * 1e3

    v16_us = graph_ms_per_step = prefill_us = kvproj_us = c5 = vgraph_us = batched = None
    esz_in = 2
    F = g.n_frames
    if not args.core_only:
        # verify with 16-token draft blocks (64 query rows per kv head)
        b16 = 16
        qb16 = [rnd(b16, g.n_q_heads, g.head_dim) for _ in range(L)]
        kb16 = [rnd(b16, g.n_kv_heads, g.head_dim) for _ in range(L)]
        vb16 = [rnd(b16, g.n_kv_heads, g.head_dim) for _ in range(L)]
        vout16 = [torch.empty(b16, g.n_q_heads, g.head_dim, device=dev) for _ in range(L)]
        ws16 = torch.empty(fd.verify_workspace_bytes(g, b16), dtype=torch.uint8, device=dev)
        t16 = frame[0]
        v16_ms = sweep(lambda l: fd.verify_attn(g, qb16[l], kb16[l], vb16[l], kc[l], vc[l], t16, n_tail, b16,
                                                vout16[l], ws16), reps)
        v16_us = mean(v16_ms) * 1e3

        # batched verify: S independent 8-token drafts with their own reasoning tails over one
        # window in one call, with and without the rotated window a streaming call leaves in its
        # workspace (here from fd_rotate_window); tails in a cache with room for six of them
        gb = g.replace(tail_cap=6 * (n_tail + blk))
        kcb = [rnd(g.n_kv_heads, gb.cache_rows, g.head_dim) for _ in range(L)]
        vcb = [rnd(g.n_kv_heads, gb.cache_rows, g.head_dim) for _ in range(L)]
        kview = [torch.empty(g.n_kv_heads, g.window, g.head_dim, dtype=torch.float16, device=dev) for _ in range(L)]
        for l in range(L):
            fd.rotate_window(gb, kcb[l], t16, kview[l])
        batched = {}
        for tails in ((200, 120), (200, 150, 100, 175, 125, 50)):
            S = len(tails)
            qs = [rnd(S, blk, g.n_q_heads, g.head_dim) for _ in range(L)]
            ks = [rnd(S, blk, g.n_kv_heads, g.head_dim) for _ in range(L)]
            vs = [rnd(S, blk, g.n_kv_heads, g.head_dim) for _ in range(L)]
            ob = torch.empty(S, blk, g.n_q_heads, g.head_dim, device=dev)
            wsb = torch.empty(fd.verify_batched_workspace_bytes(gb, S, blk), dtype=torch.uint8, device=dev)
            nbytes = ((g.window + sum(tails) + S * blk) * g.n_kv_heads * g.head_dim * esz_in * 2
                      + S * blk * g.n_q_heads * g.head_dim * (esz_in + 4))
            for use_view in (False, True):
                b_ms = sweep(lambda l: fd.verify_attn_batched(gb, qs[l], ks[l], vs[l], kcb[l], vcb[l], t16, tails,
                                                              n_tail + blk, blk, ob, wsb,
                                                              k_view=kview[l] if use_view else None), reps)
                us = mean(b_ms) * 1e3
                gbs = nbytes / (us * 1e-6) / 1e9
                batched[f"S{S}{'_view' if use_view else ''}"] = {
                    "us_per_call": round(us, 2), "gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
                    "drafts": S, "n_tails": list(tails), "k_view": use_view,
                    "bytes_per_call": nbytes}
            del qs, ks, vs, ob, wsb
        del kcb, vcb, kview

        # cold-start (non-streaming) prefill: every window row a query, same mask
        pws = torch.empty(fd.prefill_workspace_bytes(g), dtype=torch.uint8, device=dev)
        qw = [rnd(g.window, g.n_q_heads, g.head_dim) for _ in range(L)]
        ow = [torch.empty(g.window, g.n_q_heads, g.head_dim, device=dev) for _ in range(L)]
        pf_ms = sweep(lambda l: fd.prefill_attn(g, qw[l], kc[l], vc[l], t16, ow[l], pws), 1)
        prefill_us = mean(pf_ms) * 1e3
        del qw, ow, pws

        # K/V projection of the new frames with the ring-slot insert as its epilogue
        hidden = g.n_q_heads * g.head_dim
        xs = [rnd(g.n_new, hidden) for _ in range(L)]
        wkv = [(torch.randn(2 * g.n_kv_heads * g.head_dim, hidden, generator=gen, device=dev)
                / hidden ** 0.5).to(torch.bfloat16) for _ in range(L)]
        kp_ms = sweep(lambda l: fd.kv_project_insert(g, xs[l], wkv[l], kc[l], vc[l], t16), 1)
        kvproj_us = mean(kp_ms) * 1e3
        kvproj_flops = 2 * g.n_new * (2 * g.n_kv_heads * g.head_dim) * hidden
        del xs, wkv

        # the 36 verify calls of a step captured in one HIP graph: wall time of the sequence
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        tv = frame[0]
        with torch.cuda.stream(side):
            vgr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(vgr, stream=side):
                for l in range(L):
                    fd.verify_attn(g, qb[l], kb[l], vb[l], kc[l], vc[l], tv, n_tail, blk, vout[l], ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        vgr.replay()
        torch.cuda.synchronize()
        vg_ms = []
        for _ in range(max(2, args.steps // 2)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            vgr.replay()
            e1.record()
            torch.cuda.synchronize()
            vg_ms.append(e0.elapsed_time(e1))
        vgraph_us = sorted(vg_ms)[len(vg_ms) // 2] * 1e3 / L
        del vgr

        # config 5 shapes: 100 rolling windows of one layer (V=4, F=8, T=256, P=512: 8,704 keys),
        # each an insert of the new frames and a streaming-prefill call; timing inputs N(0,1)
        c5 = rolling_windows(synth.CONFIGS[5].geom, 100, gen, host_ahead)

        # the same window step replayed from HIP graphs: one graph per ring phase (t mod F), every
        # kernel argument depending on the newest frame only through it
        F = g.n_frames
        graphs = {}
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(F):
                gr = torch.cuda.CUDAGraph()
                frame[0] = g.n_frames + i
                with torch.cuda.graph(gr, stream=side):
                    step_plain()   # a graph fixes the view offset, which moves with the frame index
                graphs[(g.n_frames + i) % F] = gr
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for i in range(F):
            graphs[i].replay()
        torch.cuda.synchronize()
        t_start.record()
        for i in range(args.steps):
            graphs[i % F].replay()
        t_end.record()
        torch.cuda.synchronize()
        graph_ms_per_step = t_start.elapsed_time(t_end) / args.steps

    esz = 2
    flops_layer = 4 * g.head_dim * g.n_q_heads * stream_pairs(g)
    vbytes_layer = verify_bytes(g, n_tail, blk, esz)
    flops_prefill = 4 * g.head_dim * g.n_q_heads * (g.window * (g.window + 1) // 2)
    b16 = 16
    v16bytes_layer = verify_bytes(g, n_tail, b16, esz)
    ibytes_layer = 2 * 2 * g.n_views * g.tok_per_frame * g.n_kv_heads * g.head_dim * esz
    value = flops_layer * L / (ms_per_step * 1e-3) / 1e12
    att_tflops = flops_layer / (attv_us * 1e-6) / 1e12
    att_plain_tflops = flops_layer / (att_us * 1e-6) / 1e12 if plain else None
    ver_gbs = vbytes_layer / (verv_us * 1e-6) / 1e9
    ver_plain_gbs = vbytes_layer / (ver_us * 1e-6) / 1e9

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16, resident in HBM)",
        "config": {
            "workload": f"backbone window step: {L} layers x (insert 4x256-token frame + streaming-prefill "
                        f"attention over the layer's persistent key view, 1024 queries over 4608 keys, 32/8 "
                        f"heads, D=128 + 8-token verify over 4608+{n_tail}+{blk} keys)",
            "layers": L, "views": g.n_views, "frames": g.n_frames, "tok_per_frame": g.tok_per_frame,
            "prefix": g.prefix_len, "heads_q_kv": [g.n_q_heads, g.n_kv_heads], "head_dim": g.head_dim,
            "parallelism": "1 GPU",
        },
        "roofline": {
            "kernel": "fd_stream_attn_view (rope_window_kernel + stream_pp_kernel; at this geometry no view is cut twice, so no merge launch)",
            "bound": "mfma",
            "achieved": round(att_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": committed_traffic("stream_attn_config3_traffic.md"),
        },
        "roofline_verify": {
            "kernel": "fd_verify_attn_batched, one draft, window keys from the key view (verify_dma_kernel + "
                      "verify_merge_dma_kernel)",
            "bound": "hbm",
            "achieved": round(ver_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(ver_gbs / PEAK_HBM_GBS, 4),
            "traffic": committed_traffic("verify_attn_config4_traffic.md"),
        },
        "per_call_us": {"insert": round(ins_us, 2), "stream_attn_view": round(attv_us, 2),
                        "stream_attn_insert_view": round(mean(siv_ms) * 1e3, 2),
                        "verify_attn_view": round(verv_us, 2), "verify_attn": round(ver_us, 2),
                        "stream_attn": plain and round(att_us, 2),
                        "stream_attn_insert": plain and round(mean(si_ms) * 1e3, 2)},
        "stream_attn_plain_tflops": plain and round(att_plain_tflops, 2),
        "verify_attn_plain_gbs": round(ver_plain_gbs, 1),
        "per_call_us_median": {k: round(med(x) * 1e3, 2) for k, x in
                               (("insert", ins_ms), ("stream_attn_view", attv_ms), ("stream_attn", att_ms),
                                ("verify_attn_view", verv_ms), ("verify_attn", ver_ms)) if x},
        "per_call_us_min": {k: round(min(x) * 1e3, 2) for k, x in
                            (("insert", ins_ms), ("stream_attn_view", attv_ms), ("stream_attn", att_ms),
                             ("verify_attn_view", verv_ms), ("verify_attn", ver_ms)) if x},
        "per_call_note": "each call type swept over the 36 layers back to back; HIP events around each sweep; "
                         "_view: with the layer's persistent key view (the prefix and the new frames rotated), "
                         "without: the whole window rotated every call",
        "plain_ms_per_step": None if plain_ms_per_step is None else round(plain_ms_per_step, 4),
        "verify_graph": None if vgraph_us is None else {
            "us_per_call": round(vgraph_us, 2),
            "gbs": round(vbytes_layer / (vgraph_us * 1e-6) / 1e9, 1),
            "frac": round(vbytes_layer / (vgraph_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "note": f"the {L} verify calls of a step captured in one HIP graph, median replay / {L}"},
        "verify_batched": None if batched is None else dict(batched, note=(
            "fd_verify_attn_batched: S 8-token drafts with their own reasoning tails over one window per "
            "call; algorithmic bytes = window K/V once + every draft's tail and block K/V + queries + fp32 "
            "outputs; _view: window keys read from the rotated fp16 view")),
        "config5": c5,
        "insert_gbs": round(ibytes_layer / (ins_us * 1e-6) / 1e9, 1),
        "verify_block16": None if v16_us is None else {
            "us_per_call": round(v16_us, 2),
            "gbs": round(v16bytes_layer / (v16_us * 1e-6) / 1e9, 1),
            "frac": round(v16bytes_layer / (v16_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "note": "16-token draft block, 64 query rows per kv head"},
        "prefill": None if prefill_us is None else {
            "us_per_call": round(prefill_us, 2),
            "achieved_tflops": round(flops_prefill / (prefill_us * 1e-6) / 1e12, 2),
            "frac": round(flops_prefill / (prefill_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "stream_over_prefill_time": round(att_us / prefill_us, 4),
            "stream_over_prefill_flops": round(flops_layer / flops_prefill, 4),
            "note": "cold-start prefill of all 4,608 window rows (fd_prefill_attn) beside the streaming call"},
        "kv_projection": None if kvproj_us is None else {
            "us_per_call": round(kvproj_us, 2),
            "achieved_tflops": round(kvproj_flops / (kvproj_us * 1e-6) / 1e12, 2),
            "frac": round(kvproj_flops / (kvproj_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "note": "fd_kv_project_insert: 1,024 tokens x hidden 4,096 -> K and V (8 heads x 128), "
                    "written into the ring slot"},
        "graph": None if graph_ms_per_step is None else {
            "ms_per_step": round(graph_ms_per_step, 4), "eager_ms_per_step": plain_ms_per_step and round(plain_ms_per_step, 4),
            "graphs": F, "launches_per_step": L * 5,
            "note": "the step without key views (fd_stream_attn_insert + fd_verify_attn per layer) replayed from "
                    "one HIP graph per ring phase (t mod F), beside the same step run eagerly; a key view's "
                    "offset follows the frame index, which a replayed graph cannot"},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
