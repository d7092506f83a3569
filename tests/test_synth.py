"""Host-side checks of the seeded input generators."""
import numpy as np

import synth


def test_bf16_round_ties_to_even_and_idempotent():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], dtype=np.float32)
    r = synth.bf16_round(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                      # tie -> even mantissa
    assert r[2] == 1.0 + 2 ** -6            # tie -> even (rounds up)
    np.testing.assert_array_equal(synth.bf16_round(r), r)
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)


def test_config_shapes_and_candidates():
    cfg = synth.get_config(5).shrunk(B=3, lengths=("fixed", 40), num_candidates=8)
    inp = synth.make_inputs(cfg)
    assert np.all(inp.lengths == 48)
    assert inp.X.shape == (144, cfg.D)
    for b in range(3):
        t = inp.timestamps[inp.seq_offsets[b]:inp.seq_offsets[b + 1]]
        assert np.all(np.diff(t) >= 0)
        assert np.all(t[40:] == t[39])
    assert np.all((inp.X.view(np.uint32) & 0xFFFF) == 0)


def test_zipf_lengths_are_clipped():
    cfg = synth.get_config(3)
    n = synth.make_lengths(cfg, np.random.default_rng(cfg.seed))
    assert n.min() >= 32 and n.max() <= 2048 and len(n) == 64


def test_same_seed_same_values():
    cfg = synth.get_config(1)
    a, b = synth.make_inputs(cfg), synth.make_inputs(cfg)
    np.testing.assert_array_equal(a.X, b.X)
    np.testing.assert_array_equal(a.timestamps, b.timestamps)
