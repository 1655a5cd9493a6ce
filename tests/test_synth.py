"""CPU tests of the seeded generator and the workload geometry it encodes."""
import json
import os

import numpy as np
import torch

from streaming_kv_cache_view_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -2.00390625, 3.0e-39, 65504.0], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(synth.round_bf16(x), want)


def test_draws_are_deterministic_and_independent():
    w = synth.CONFIGS[2]
    a = synth.draw(w, 0, "K", 1, 3, (4, 2, 8))
    b = synth.draw(w, 0, "K", 1, 3, (4, 2, 8))
    c = synth.draw(w, 0, "K", 1, 4, (4, 2, 8))
    d = synth.draw(w, 1, "K", 1, 3, (4, 2, 8))
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)
    assert np.array_equal(synth.round_bf16(a), a)          # bf16-exact values
    assert abs(np.std(synth.draw(w, 0, "V", 0, 0, (20000,))) - 0.5) < 0.02


def test_outliers_on_kv_only():
    w = synth.CONFIGS[5]
    k = synth.draw(w, 0, "K", 0, 0, (256, 8, 128))
    q = synth.draw(w, 0, "Q", 0, 0, (256, 8, 128))
    frac = np.mean(np.abs(k) == 8.0)
    assert 0.008 < frac < 0.012
    assert np.max(np.abs(q)) < 7.0


def test_config_geometry():
    g = synth.CONFIGS[3].geom
    assert g.window == 4608 and g.n_new == 1024
    assert synth.CONFIGS[5].geom.window == 8704
    assert synth.CONFIGS[1].geom.window == 136 and synth.CONFIGS[2].geom.window == 1088
    w4 = synth.CONFIGS[4]
    assert w4.geom.window + w4.n_tail + w4.blk_len == 4816


def test_streaming_cut_matches_pages():
    fig = json.load(open(GOLDEN))
    for cid in (1, 2, 3):
        g = synth.CONFIGS[cid].geom
        frame_tokens = g.n_views * g.n_frames * g.tok_per_frame
        assert g.n_new / frame_tokens == 1 - fig["effective_sequence_cut"]["value"]
    assert synth.CONFIGS[4].blk_len == fig["draft_block"]["value"]
