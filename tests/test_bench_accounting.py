"""CPU tests of bench.py's algorithmic work accounting against the oracle's own mask.

The FLOP and byte counts that bench.py divides by time are closed forms; here they are checked
against a brute-force count of the unmasked (query, key) pairs built from the oracle's
positions (key position <= query position), for the configs the bench and the tests use.
"""
from __future__ import annotations

import numpy as np
import pytest

import bench
from oracle import fd_oracle
from streaming_kv_cache_view_amd import synth


def _pairs(q_pos, k_pos):
    k_sorted = np.sort(np.asarray(k_pos))
    return int(np.searchsorted(k_sorted, np.asarray(q_pos), side="right").sum())


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_stream_pairs_match_the_mask(cid):
    g = synth.CONFIGS[cid].geom
    q = fd_oracle.new_query_positions(g)
    k = fd_oracle.window_positions(g, g.window)
    assert bench.stream_pairs(g) == _pairs(q, k)


def test_stream_flops_config3():
    g = synth.CONFIGS[3].geom
    assert bench.stream_pairs(g) == 3_015_168
    assert 4 * g.head_dim * g.n_q_heads * bench.stream_pairs(g) == 49_400_512_512   # 49.40 GFLOP


def test_verify_pairs_match_the_mask():
    w = synth.CONFIGS[4]
    g = w.geom
    n_tail, blk = w.n_tail, w.blk_len
    k = fd_oracle.window_positions(g, g.window + n_tail + blk)
    q = np.int64(g.pos_base) + g.window + n_tail + np.arange(blk)
    assert bench.verify_pairs(g, n_tail, blk) == _pairs(q, k)


def test_full_window_pairs():
    g = synth.CONFIGS[3].geom
    pos = fd_oracle.window_positions(g, g.window)
    assert _pairs(pos, pos) == g.window * (g.window + 1) // 2
