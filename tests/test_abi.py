"""CPU tests of the C ABI: exports, host-side position helper, and every validation error.

No compute call is made here (there is no GPU): every invalid call returns its
error before anything is enqueued, and no valid compute call is issued.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import oracle.fd_oracle as fd_oracle
from streaming_kv_cache_view_amd import fd, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fdattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fd.LIB_PATH), reason="libfdattn.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fd_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = fd.lib()
    names = declared_functions()
    assert set(names) == set(fd.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_struct_layout_matches_header():
    assert ctypes.sizeof(fd.FdGeom) == 56
    assert fd.FdGeom.rope_theta.offset == 32 and fd.FdGeom.pos_base.offset == 40
    assert fd.FdGeom.out_dtype.offset == 52


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_cache_rows(cid):
    g = synth.CONFIGS[cid].geom
    assert fd.cache_rows(g) == g.window + g.tail_cap


@pytest.mark.parametrize("cid,t", [(1, 3), (1, 4), (1, 9), (2, 6), (5, 8), (5, 19), (5, 107)])
def test_key_position_matches_oracle_ring_reading(cid, t):
    """Physical row -> logical position, against the oracle's slot occupancy and window order."""
    g = synth.CONFIGS[cid].geom.replace(pos_base=17)
    slots = fd_oracle.expected_ring_rows(g, t)
    want = np.empty(g.cache_rows, np.int64)
    want[: g.prefix_len] = g.pos_base + np.arange(g.prefix_len)
    for v in range(g.n_views):
        for s, fid in enumerate(slots):
            j = fid - (t - g.n_frames + 1)          # index of the frame inside its view (oldest = 0)
            r0 = g.prefix_len + (v * g.n_frames + s) * g.tok_per_frame
            p0 = g.pos_base + g.prefix_len + (v * g.n_frames + j) * g.tok_per_frame
            want[r0: r0 + g.tok_per_frame] = p0 + np.arange(g.tok_per_frame)
    want[g.window:] = g.pos_base + np.arange(g.window, g.cache_rows)
    rows = range(g.cache_rows) if g.cache_rows < 2000 else range(0, g.cache_rows, 7)
    got = [fd.key_position(g, t, r) for r in rows]
    assert got == [int(want[r]) for r in rows]
    # the rows of the newest frame sit at the new-query positions
    qpos = fd_oracle.new_query_positions(g)
    s_new = t % g.n_frames
    for v in range(g.n_views):
        r0 = g.prefix_len + (v * g.n_frames + s_new) * g.tok_per_frame
        assert fd.key_position(g, t, r0) == qpos[v * g.tok_per_frame]


FAKE = 0x10000          # never dereferenced: validation fails first
MISALIGNED = 0x10008


def _g(**kw):
    base = dict(n_views=2, n_frames=4, tok_per_frame=16, prefix_len=8, n_q_heads=4, n_kv_heads=2,
                head_dim=64, tail_cap=32, rope_theta=1e4, pos_base=0, in_dtype=fd.FD_BF16,
                out_dtype=fd.FD_F32)
    base.update(kw)
    return fd.FdGeom(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(n_views=0), -2), (dict(n_frames=0), -2), (dict(tok_per_frame=0), -2), (dict(prefix_len=-1), -2),
    (dict(n_q_heads=3), -2), (dict(n_q_heads=6, n_kv_heads=2), -2), (dict(head_dim=96), -2),
    (dict(rope_theta=float("nan")), -2), (dict(rope_theta=1.0), -2), (dict(pos_base=-1), -2),
    (dict(pos_base=1 << 31), -2), (dict(tail_cap=-1), -2), (dict(tok_per_frame=1 << 24), -2),
    (dict(in_dtype=7), -3), (dict(out_dtype=2), -3),
])
def test_geometry_errors(kw, code):
    L = fd.lib()
    g = _g(**kw)
    assert L.fd_cache_rows(ctypes.byref(g)) == -1
    assert L.fd_stream_attn(ctypes.byref(g), FAKE, FAKE, FAKE, 5, FAKE, FAKE, 1 << 40, None) == code
    assert L.fd_stream_workspace_bytes(ctypes.byref(g)) == 0
    assert L.fd_kv_insert_frame(ctypes.byref(g), FAKE, FAKE, FAKE, FAKE, 0, None) == code
    assert L.fd_verify_workspace_bytes(ctypes.byref(g), 8) == 0


def test_call_errors():
    L = fd.lib()
    g = _g()
    gp = ctypes.byref(g)
    sws = L.fd_stream_workspace_bytes(gp)
    # rotated keys (fp16), then for bf16 inputs the rotated, scaled queries (fp16, V*T*Hq*D) and
    # two fp32 partial slots (O[128][D], (m, l)[128]) per (row block, chunk); a row block is 128
    # query rows: min(G, 4) heads x (4 / min(G, 4)) 32-token blocks -> G=2: 2 heads, 64 tokens,
    # one block per kv head; between queries and partials, the attention kernel's tile table
    # (8 bytes per tile of each view's key sequence: view 0 prefix + 3 frames + diagonal,
    # view 1 prefix + 7 frames + diagonal)
    krot = g.n_kv_heads * (8 + 2 * 4 * 16) * 64 * 2
    qrot = 2 * 16 * 4 * 64 * 2
    n_rb = g.n_kv_heads * 1 * 1
    align = lambda x: (x + 255) // 256 * 256
    assert sws == align(krot) + align(qrot) + align((5 + 9) * 8) + n_rb * 2 * 2 * (128 * 64 + 256) * 4
    assert L.fd_stream_workspace_bytes(ctypes.byref(_g(in_dtype=fd.FD_F32))) == g.n_kv_heads * (8 + 2 * 4 * 16) * 64 * 4
    assert L.fd_stream_attn(None, FAKE, FAKE, FAKE, 5, FAKE, FAKE, sws, None) == -1
    assert L.fd_stream_attn(gp, None, FAKE, FAKE, 5, FAKE, FAKE, sws, None) == -1
    assert L.fd_stream_attn(gp, FAKE, FAKE, FAKE, 5, None, FAKE, sws, None) == -1
    assert L.fd_stream_attn(gp, FAKE, FAKE, FAKE, 2, FAKE, FAKE, sws, None) == -4     # window not full
    assert L.fd_stream_attn(gp, FAKE, FAKE, FAKE, 5, FAKE, None, sws, None) == -7     # no workspace
    assert L.fd_stream_attn(gp, FAKE, FAKE, FAKE, 5, FAKE, FAKE, sws - 1, None) == -7
    assert L.fd_stream_attn(gp, MISALIGNED, FAKE, FAKE, 5, FAKE, FAKE, sws, None) == -5
    assert L.fd_stream_attn(gp, FAKE, FAKE, FAKE, 5, FAKE, MISALIGNED, sws, None) == -5
    S = L.fd_stream_attn_insert
    assert S(None, FAKE, FAKE, FAKE, FAKE, FAKE, 5, FAKE, FAKE, sws, None) == -1
    assert S(gp, None, FAKE, FAKE, FAKE, FAKE, 5, FAKE, FAKE, sws, None) == -1          # no k_new
    assert S(gp, FAKE, None, FAKE, FAKE, FAKE, 5, FAKE, FAKE, sws, None) == -1          # no v_new
    assert S(gp, FAKE, FAKE, FAKE, FAKE, FAKE, 5, None, FAKE, sws, None) == -1          # no out
    assert S(gp, FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, sws, None) == -4          # window not full
    assert S(gp, FAKE, FAKE, FAKE, FAKE, FAKE, 5, FAKE, FAKE, sws - 1, None) == -7
    assert S(gp, MISALIGNED, FAKE, FAKE, FAKE, FAKE, 5, FAKE, FAKE, sws, None) == -5
    assert S(gp, FAKE, FAKE, FAKE, MISALIGNED, FAKE, 5, FAKE, FAKE, sws, None) == -5
    assert L.fd_kv_insert_frame(gp, FAKE, None, FAKE, FAKE, 0, None) == -1
    assert L.fd_kv_insert_frame(gp, FAKE, FAKE, FAKE, FAKE, -1, None) == -4
    assert L.fd_kv_insert_frame(gp, FAKE, FAKE, FAKE, MISALIGNED, 0, None) == -5
    ws = L.fd_verify_workspace_bytes(gp, 8)
    ws17 = L.fd_verify_workspace_bytes(gp, 17)                                 # G*B = 34: two row blocks
    assert ws > 0 and ws17 > ws and L.fd_verify_workspace_bytes(gp, 33) == 0   # B > 32 (and > tail_cap)
    g8 = _g(n_q_heads=16)                                                      # G = 8
    assert L.fd_verify_workspace_bytes(ctypes.byref(g8), 16) > 0               # 128 query rows
    assert L.fd_verify_workspace_bytes(ctypes.byref(g8), 17) == 0              # 136 > 128
    args = [FAKE, FAKE, FAKE, FAKE, FAKE]
    assert L.fd_verify_attn(gp, *args, 5, -1, 8, FAKE, FAKE, ws, None) == -6
    assert L.fd_verify_attn(gp, *args, 5, 30, 8, FAKE, FAKE, ws, None) == -6   # n_tail + B > tail_cap
    assert L.fd_verify_attn(gp, *args, 5, 0, 0, FAKE, FAKE, ws, None) == -6
    assert L.fd_verify_attn(gp, *args, 5, 0, 17, FAKE, FAKE, ws, None) == -7   # two row blocks: more workspace
    assert L.fd_verify_attn(ctypes.byref(g8), *args, 5, 0, 17, FAKE, FAKE, ws17, None) == -6   # G*B > 128
    assert L.fd_verify_attn(gp, *args, 5, 0, 8, FAKE, None, ws, None) == -7
    assert L.fd_verify_attn(gp, *args, 5, 0, 8, FAKE, FAKE, ws - 1, None) == -7
    assert L.fd_verify_attn(gp, *args, 2, 0, 8, FAKE, FAKE, ws, None) == -4
    assert L.fd_verify_attn(gp, *args, 5, 0, 8, MISALIGNED, FAKE, ws, None) == -5
    assert L.fd_verify_attn(gp, None, *args[1:], 5, 0, 8, FAKE, FAKE, ws, None) == -1
    for code in range(-8, 1):
        assert fd.lib().fd_status_str(code).decode() != "unknown status"


def test_prefill_call_errors():
    L = fd.lib()
    g = _g()                                   # bf16 inputs
    gp = ctypes.byref(g)
    pws = L.fd_prefill_workspace_bytes(gp)
    # rotated keys, every window row's rotated queries (W = 8 + 2*4*16 = 136 rows) and the tile
    # table (frame (v, j): prefix + v*F + j earlier frames + diagonal, one 64-key tile each here;
    # then the prefix segment); every segment is attended whole, so no partial slots
    W = 8 + 2 * 4 * 16
    align = lambda x: (x + 255) // 256 * 256
    n_tiles = sum(1 + sg + 1 for sg in range(2 * 4)) + 1
    assert pws == align(g.n_kv_heads * W * 64 * 2) + align(W * 4 * 64 * 2) + align(n_tiles * 8)
    assert L.fd_prefill_workspace_bytes(ctypes.byref(_g(in_dtype=fd.FD_F32))) == 0
    assert L.fd_prefill_attn(ctypes.byref(_g(in_dtype=fd.FD_F32)), FAKE, FAKE, FAKE, 5, FAKE, FAKE, pws,
                             None) == -3                                        # bf16 only
    assert L.fd_prefill_attn(gp, None, FAKE, FAKE, 5, FAKE, FAKE, pws, None) == -1
    assert L.fd_prefill_attn(gp, FAKE, FAKE, FAKE, 5, None, FAKE, pws, None) == -1
    assert L.fd_prefill_attn(gp, FAKE, FAKE, FAKE, 2, FAKE, FAKE, pws, None) == -4   # window not full
    assert L.fd_prefill_attn(gp, FAKE, FAKE, FAKE, 5, FAKE, FAKE, pws - 1, None) == -7
    assert L.fd_prefill_attn(gp, FAKE, FAKE, FAKE, 5, FAKE, None, pws, None) == -7
    assert L.fd_prefill_attn(gp, MISALIGNED, FAKE, FAKE, 5, FAKE, FAKE, pws, None) == -5


def test_kv_project_call_errors():
    L = fd.lib()
    gp = ctypes.byref(_g())                     # bf16 inputs; N = 2*Hkv*D = 256
    f = L.fd_kv_project_insert
    assert f(ctypes.byref(_g(in_dtype=fd.FD_F32)), FAKE, FAKE, 64, FAKE, FAKE, 0, None) == -3   # bf16 only
    assert f(gp, None, FAKE, 64, FAKE, FAKE, 0, None) == -1
    assert f(gp, FAKE, FAKE, 64, FAKE, None, 0, None) == -1
    assert f(gp, FAKE, FAKE, 96, FAKE, FAKE, 0, None) == -2      # hidden not a multiple of 64
    assert f(gp, FAKE, FAKE, 0, FAKE, FAKE, 0, None) == -2
    assert f(gp, FAKE, FAKE, 1 << 22, FAKE, FAKE, 0, None) == -2  # w would exceed 2 GiB
    assert f(gp, FAKE, FAKE, 64, FAKE, FAKE, -1, None) == -4
    assert f(gp, FAKE, MISALIGNED, 64, FAKE, FAKE, 0, None) == -5


def test_workspace_size_covers_largest_block():
    g = synth.CONFIGS[4].geom
    ws = fd.verify_workspace_bytes(g, 8)
    # the largest split count is reached when n_tail + B == tail_cap
    nblk = (-(-g.prefix_len // 32) + g.n_views * g.n_frames * -(-g.tok_per_frame // 32)
            + -(-g.tail_cap // 32))
    splits = -(-nblk // 4)
    assert ws >= g.n_kv_heads * splits * (32 * g.head_dim + 64) * 4
    # 16-token blocks: G*16 = 64 query rows per kv head, two 32-row blocks
    assert fd.verify_workspace_bytes(g, 16) >= 2 * g.n_kv_heads * splits * (32 * g.head_dim + 64) * 4
