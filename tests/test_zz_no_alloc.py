"""fd_verify_attn_noalloc, the allocation-free verify, through the C ABI.

Consecutive calls on one GPU share the library's static scratch array; each is checked against
fd_verify_attn (same kernels, caller workspace) on an identical copy of the caches -- outputs and
caches bit for bit -- and against the fp64 oracle.  The calls shrink one after another (backbone
shapes with a 16-token block, then config-2 shapes with an 8-token block, then fp32 config 1), so a
later call runs over scratch contents a larger call left behind.
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


CALLS = [(4, 3, 4, 200, 16), (2, 0, 5, 40, 8), (1, 0, 4, 5, 8)]   # (config, layer, t, n_tail, block)


def test_noalloc_verify_matches_workspace_call():
    for cid, layer, t, n_tail, blk in CALLS:
        w = synth.CONFIGS[cid]
        g = w.geom
        H.say(f"noalloc verify cfg {cid} layer {layer} t {t} n_tail {n_tail} B {blk}")
        kc, vc = H.window_caches(w, layer, t)
        kt, vt = synth.tail_kv(w, layer, n_tail)
        kc[:, g.window: g.window + n_tail] = H.dev(np.transpose(kt, (1, 0, 2)), g)
        vc[:, g.window: g.window + n_tail] = H.dev(np.transpose(vt, (1, 0, 2)), g)
        kc2, vc2 = kc.clone(), vc.clone()
        qb, kb, vb = synth.block_qkv(w, layer, blk)
        qd, kd, vd = H.dev(qb, g), H.dev(kb, g), H.dev(vb, g)
        ref = torch.empty((blk, g.n_q_heads, g.head_dim), dtype=torch.float32, device=H.DEV)
        ws = torch.empty(fd.verify_workspace_bytes(g, blk), dtype=torch.uint8, device=H.DEV)
        fd.verify_attn(g, qd, kd, vd, kc2, vc2, t, n_tail, blk, ref, ws)
        out = torch.full_like(ref, float("nan"))
        fd.verify_attn_noalloc(g, qd, kd, vd, kc, vc, t, n_tail, blk, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), float((out - ref).abs().max())
        assert torch.equal(kc, kc2) and torch.equal(vc, vc2)
        win = fd_oracle.StreamWindow(g, *synth.prefix_kv(w, layer))
        for f in range(t + 1):
            for v in range(g.n_views):
                win.push(v, f, *synth.frame_kv(w, layer, v, f))
        want = fd_oracle.oracle_verify(g, win, kt, vt, qb, kb, vb)
        err = H.check_out(out.cpu().numpy(), want, g, "f32", ("noalloc", cid))
        H.say(f"  bit-identical to fd_verify_attn; max-abs vs oracle {err:.3e} (tol {H.TOL[g.dtype]})")
