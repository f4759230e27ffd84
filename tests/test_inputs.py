"""The seeded input generator: rounding, shapes, determinism."""
import numpy as np

import gsa_inputs as gi


def test_bf16_rounding_known_values():
    vals = np.array([1.0, -2.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                     3.0e38, -0.0], np.float32)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6);
    # just above a tie rounds up; 3e38 stays finite.
    expect = [0x3F80, 0xC000, 0x3F80, 0x3F82, 0x3F81, 0x7F62, 0x8000]
    assert gi.bf16_bits(vals).tolist() == expect
    assert np.array_equal(gi.bf16_bits_to_f32(np.array(expect, np.uint16))[:2], [1.0, -2.0])


def test_shapes_and_sentinel():
    d = gi.make_inputs("c1", seed=0, rank=1)
    assert d["A"].shape == (1024, 512) and d["A"].dtype == np.uint16
    assert d["x"].shape == (1, 512)
    assert d["slots"].shape == (2, 1024, 1)
    assert np.isnan(d["slots"][1]).all() and np.isfinite(d["slots"][0]).all()


def test_deterministic_and_seed_sensitive():
    a = gi.make_inputs("c1", seed=3)
    b = gi.make_inputs("c1", seed=3)
    c = gi.make_inputs("c1", seed=4)
    assert np.array_equal(a["A"], b["A"]) and np.array_equal(a["x"], b["x"])
    assert not np.array_equal(a["A"], c["A"])


def test_distribution_roughly_as_stated():
    d = gi.make_inputs("c2")
    A = gi.bf16_bits_to_f32(d["A"])
    assert abs(A.std() - 0.02) < 5e-4 and abs(A.mean()) < 5e-4
    x = gi.bf16_bits_to_f32(d["x"])
    assert abs(x.std() - 1.0) < 0.1
