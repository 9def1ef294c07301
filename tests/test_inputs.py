"""The seeded input generator: determinism, shapes, dtype rounding, ranges."""
import numpy as np

from state_space_model_mamba2_amd import inputs


def test_deterministic_and_shapes():
    s = inputs.workload("tiny_fp32")
    a, b = inputs.generate(s, seed=0), inputs.generate(s, seed=0)
    for k in ["x", "dt", "A", "B", "C", "D", "dy"]:
        assert np.array_equal(getattr(a, k), getattr(b, k)), k
    assert a.x.shape == (1, 256, 2, 16) and a.dt.shape == (1, 256, 2)
    assert a.B.shape == (1, 256, 1, 16) and a.A.shape == (2,) and a.dy.shape == a.x.shape
    c = inputs.generate(s, seed=1)
    assert not np.array_equal(a.x, c.x)


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.14159], dtype=np.float32)
    bits = inputs.f32_to_bf16_bits(v)
    back = inputs.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.0 + 2 ** -6)
    assert back[3] == -2.5 and abs(back[4] - 3.140625) < 1e-7


def test_ranges_follow_recipe():
    s = inputs.workload("mamba2_370m", batch=1, seqlen=512)
    g = inputs.generate(s, seed=0)
    A = g.A
    assert np.all(A <= -1.0) and np.all(A >= -16.0)
    dt = g.as_f64("dt")
    assert np.all(dt > 0)
    assert 1e-3 < np.median(dt) < 1e-1
    x = g.as_f64("x")
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    lc = inputs.generate(inputs.workload("long_context", seqlen=1024), seed=0)
    assert np.median(lc.as_f64("dt")) < np.median(dt)
