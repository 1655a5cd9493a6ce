"""Benchmark of the streaming-prefill attention hot path on one MI355X.

One step = one window of the 36-layer backbone, for every layer:
    insert               new frame of 4 views -> ring slot
    streaming prefill    1,024 new-frame queries over 4,608 keys      (config 3)
        (the two through fd_stream_attn_insert, which copies the frame in the rotation pass)
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


def cpu_baseline(min_seconds: float = 12.0, max_layers: int = 36):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload: config-3
    streaming-prefill layers, one after another, until min_seconds have elapsed (or all
    max_layers are done).  Returns its algorithmic TFLOP/s (same FLOP count as the GPU)."""
    import oracle.fd_oracle as fd_oracle
    from streaming_kv_cache_view_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    w3 = synth.CONFIGS[3]
    g = w3.geom
    flops, layers = 0, 0
    t0 = time.perf_counter()
    while layers < max_layers and time.perf_counter() - t0 < min_seconds:
        for _t, _out in fd_oracle.run_stream_workload(w3, layers, [w3.first_t], synth):
            flops += 4 * g.head_dim * g.n_q_heads * stream_pairs(g)
        layers += 1
    t_stream = time.perf_counter() - t0
    return {
        "value": flops / t_stream / 1e12,
        "unit": "TFLOP/s",
        "cores": min(cores, blas_threads),
        "kind": "oracle",
        "sample": f"fp64 oracle streaming prefill of config 3, layers 0..{layers - 1} of 36 "
                  f"(window build + full re-rotation + explicit mask), {t_stream:.1f} s; "
                  f"host cores visible {cores}, BLAS threads {blas_threads}",
    }


def rolling_windows(g, n_windows, gen, host_ahead):
    """Times n_windows consecutive windows of one layer (insert + streaming-prefill attention,
    each call bracketed by its own events, back to back behind a queued GPU spin)."""
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
    ins_ms, att_ms = [], []
    for rep_i in range(2):   # the first sweep is a warm-up
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_windows + 1)]
        host_ahead()
        ev[0].record()
        for w in range(n_windows):
            t = t0 + w
            fd.kv_insert_frame(g, kc, vc, kn[w % n_in], vn[w % n_in], t)
            ev[2 * w + 1].record()
            fd.stream_attn(g, qn[w % n_in], kc, vc, t, out, sws)
            ev[2 * w + 2].record()
        torch.cuda.synchronize()
        if rep_i > 0:
            ins_ms = [ev[2 * w].elapsed_time(ev[2 * w + 1]) for w in range(n_windows)]
            att_ms = [ev[2 * w + 1].elapsed_time(ev[2 * w + 2]) for w in range(n_windows)]
    flops = 4 * g.head_dim * g.n_q_heads * stream_pairs(g)
    att_us = sum(att_ms) / len(att_ms) * 1e3
    tf = flops / (att_us * 1e-6) / 1e12
    return {
        "windows": n_windows,
        "stream_us_per_window": round(att_us, 2),
        "stream_us_median": round(sorted(att_ms)[len(att_ms) // 2] * 1e3, 2),
        "stream_us_min": round(min(att_ms) * 1e3, 2),
        "insert_us_per_window": round(sum(ins_ms) / len(ins_ms) * 1e3, 2),
        "gflop_per_window": round(flops / 1e9, 2),
        "achieved_tflops": round(tf, 2),
        "frac": round(tf / PEAK_BF16_TFLOPS, 4),
        "note": "100 rolling windows of one layer at 8,704 keys (V=4, F=8, T=256, P=512, 32/8 heads, D=128); "
                "inserts timed separately; timing inputs N(0,1) bf16",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle sample length (whole config-3 layers until this many seconds)")
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
    ws = torch.empty(fd.verify_workspace_bytes(g, blk), dtype=torch.uint8, device=dev)
    sws = torch.empty(fd.stream_workspace_bytes(g), dtype=torch.uint8, device=dev)   # shared by layers
    torch.cuda.synchronize()

    frame = [g.n_frames]   # newest frame index; the window starts full

    def host_ahead():
        """Queue a spin of some milliseconds on the GPU before a per-call timing sweep: the host
        enqueues the sweep's calls while it runs, so they execute back to back and an event
        pair brackets one call's kernels, not the host's time to issue the next call."""
        torch.cuda._sleep(12_000_000)

    def step(ev=None):
        """One window: per layer the insert of the new frames, the streaming-prefill call and the
        verify.  The timed step uses the fused insert + attention entry point; the per-call pass
        (ev given) times the three calls one by one."""
        t = frame[0]
        for l in range(L):
            if ev is None:
                fd.stream_attn_insert(g, kn[l], vn[l], qn[l], kc[l], vc[l], t, out[l], sws)
                fd.verify_attn(g, qb[l], kb[l], vb[l], kc[l], vc[l], t, n_tail, blk, vout[l], ws)
                continue
            ev[0][l].record()
            fd.kv_insert_frame(g, kc[l], vc[l], kn[l], vn[l], t)
            ev[1][l].record()
            fd.stream_attn(g, qn[l], kc[l], vc[l], t, out[l], sws)
            ev[2][l].record()
            fd.verify_attn(g, qb[l], kb[l], vb[l], kc[l], vc[l], t, n_tail, blk, vout[l], ws)
            ev[3][l].record()
            fd.stream_attn_insert(g, kn[l], vn[l], qn[l], kc[l], vc[l], t, out[l], sws)
            ev[4][l].record()
        frame[0] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # whole-step timing
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # per-call timing (events on the stream the kernels are launched on)
    ins_ms, att_ms, ver_ms, si_ms = [], [], [], []
    for _ in range(max(1, args.steps // 2)):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(L)] for _ in range(5)]
        host_ahead()
        step(ev)
        torch.cuda.synchronize()
        for l in range(L):
            ins_ms.append(ev[0][l].elapsed_time(ev[1][l]))
            att_ms.append(ev[1][l].elapsed_time(ev[2][l]))
            ver_ms.append(ev[2][l].elapsed_time(ev[3][l]))
            si_ms.append(ev[3][l].elapsed_time(ev[4][l]))
    mean = lambda a: sum(a) / len(a)
    med = lambda a: sorted(a)[len(a) // 2]
    att_us, ver_us, ins_us = mean(att_ms) * 1e3, mean(ver_ms) * 1e3, mean(ins_ms) * 1e3

    v16_us = graph_ms_per_step = prefill_us = kvproj_us = c5 = vgraph_us = None
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
        v16_ms = []
        for rep_i in range(1 + max(1, args.steps // 4)):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(L + 1)]
            host_ahead()
            ev[0].record()
            for l in range(L):
                fd.verify_attn(g, qb16[l], kb16[l], vb16[l], kc[l], vc[l], t16, n_tail, b16, vout16[l], ws16)
                ev[l + 1].record()
            torch.cuda.synchronize()
            if rep_i > 0:   # the first sweep is a warm-up
                v16_ms += [ev[l].elapsed_time(ev[l + 1]) for l in range(L)]
        v16_us = sum(v16_ms) / len(v16_ms) * 1e3

        # cold-start (non-streaming) prefill: every window row a query, same mask
        pws = torch.empty(fd.prefill_workspace_bytes(g), dtype=torch.uint8, device=dev)
        qw = [rnd(g.window, g.n_q_heads, g.head_dim) for _ in range(L)]
        ow = [torch.empty(g.window, g.n_q_heads, g.head_dim, device=dev) for _ in range(L)]
        pf_ms = []
        for rep_i in range(2):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(L + 1)]
            host_ahead()
            ev[0].record()
            for l in range(L):
                fd.prefill_attn(g, qw[l], kc[l], vc[l], t16, ow[l], pws)
                ev[l + 1].record()
            torch.cuda.synchronize()
            if rep_i > 0:
                pf_ms += [ev[l].elapsed_time(ev[l + 1]) for l in range(L)]
        prefill_us = sum(pf_ms) / len(pf_ms) * 1e3
        del qw, ow, pws

        # K/V projection of the new frames with the ring-slot insert as its epilogue
        hidden = g.n_q_heads * g.head_dim
        xs = [rnd(g.n_new, hidden) for _ in range(L)]
        wkv = [(torch.randn(2 * g.n_kv_heads * g.head_dim, hidden, generator=gen, device=dev)
                / hidden ** 0.5).to(torch.bfloat16) for _ in range(L)]
        kp_ms = []
        for rep_i in range(2):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(L + 1)]
            host_ahead()
            ev[0].record()
            for l in range(L):
                fd.kv_project_insert(g, xs[l], wkv[l], kc[l], vc[l], t16)
                ev[l + 1].record()
            torch.cuda.synchronize()
            if rep_i > 0:
                kp_ms += [ev[l].elapsed_time(ev[l + 1]) for l in range(L)]
        kvproj_us = sum(kp_ms) / len(kp_ms) * 1e3
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
                    step()
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
    vbytes_layer = ((g.window + n_tail + blk) * g.n_kv_heads * g.head_dim * esz * 2
                    + blk * g.n_q_heads * g.head_dim * esz + blk * g.n_q_heads * g.head_dim * 4)
    flops_prefill = 4 * g.head_dim * g.n_q_heads * (g.window * (g.window + 1) // 2)
    b16 = 16
    v16bytes_layer = ((g.window + n_tail + b16) * g.n_kv_heads * g.head_dim * esz * 2
                      + b16 * g.n_q_heads * g.head_dim * esz + b16 * g.n_q_heads * g.head_dim * 4)
    ibytes_layer = 2 * 2 * g.n_views * g.tok_per_frame * g.n_kv_heads * g.head_dim * esz
    value = flops_layer * L / (ms_per_step * 1e-3) / 1e12
    att_tflops = flops_layer / (att_us * 1e-6) / 1e12
    ver_gbs = vbytes_layer / (ver_us * 1e-6) / 1e9

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
                        f"attention, 1024 queries over 4608 keys, 32/8 heads, D=128 + 8-token verify over "
                        f"4608+{n_tail}+{blk} keys)",
            "layers": L, "views": g.n_views, "frames": g.n_frames, "tok_per_frame": g.tok_per_frame,
            "prefix": g.prefix_len, "heads_q_kv": [g.n_q_heads, g.n_kv_heads], "head_dim": g.head_dim,
            "parallelism": "1 GPU",
        },
        "roofline": {
            "kernel": "fd_stream_attn (rope_window_kernel + stream_pp_kernel + stream_merge_kernel)",
            "bound": "mfma",
            "achieved": round(att_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": committed_traffic("stream_attn_config3_traffic.md"),
        },
        "roofline_verify": {
            "kernel": "fd_verify_attn (verify_dma_kernel + verify_merge_kernel)",
            "bound": "hbm",
            "achieved": round(ver_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(ver_gbs / PEAK_HBM_GBS, 4),
            "traffic": committed_traffic("verify_attn_config4_traffic.md"),
        },
        "per_call_us": {"insert": round(ins_us, 2), "stream_attn": round(att_us, 2),
                        "verify_attn": round(ver_us, 2), "stream_attn_insert": round(mean(si_ms) * 1e3, 2)},
        "per_call_us_median": {k: round(med(x) * 1e3, 2) for k, x in
                               (("insert", ins_ms), ("stream_attn", att_ms), ("verify_attn", ver_ms))},
        "per_call_us_min": {k: round(min(x) * 1e3, 2) for k, x in
                            (("insert", ins_ms), ("stream_attn", att_ms), ("verify_attn", ver_ms))},
        "verify_graph": None if vgraph_us is None else {
            "us_per_call": round(vgraph_us, 2),
            "gbs": round(vbytes_layer / (vgraph_us * 1e-6) / 1e9, 1),
            "frac": round(vbytes_layer / (vgraph_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "note": f"the {L} verify calls of a step captured in one HIP graph, median replay / {L}"},
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
            "ms_per_step": round(graph_ms_per_step, 4), "eager_ms_per_step": round(ms_per_step, 4),
            "graphs": F, "launches_per_step": L * 5,
            "note": "the same step replayed from one HIP graph per ring phase (t mod F)"},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
