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


def test_e4m3_codes_match_torch_and_known_values():
    torch = __import__("pytest").importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ours = inputs.E4M3_VALUES
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], theirs[fin])
    assert ours[0x38] == 1.0 and ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e4m3_rounding_is_nearest_even_and_saturating():
    torch = __import__("pytest").importorskip("torch")
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 3,
                        rng.uniform(-448, 448, 5000).astype(np.float32),
                        (rng.standard_normal(5000) * 2.0 ** -8).astype(np.float32)])
    ours = inputs.f32_to_e4m3_bits(v)
    theirs = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)
    # ties go to the even code: 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39)
    assert inputs.f32_to_e4m3_bits(np.array([1.0625, 1.1875, -1.0625]))[:3].tolist() == [0x38, 0x3A, 0xB8]
    assert inputs.f32_to_e4m3_bits(np.array([1000.0, -1e9]))[:2].tolist() == [0x7E, 0xFE]


def test_fp8_mode_rounds_x_b_c_only():
    s = inputs.workload("mamba2_370m", batch=1, seqlen=256, nheads=2, dtype="fp8")
    g = inputs.generate(s, seed=0)
    ref = inputs.generate(s.replace(dtype="bf16"), seed=0)
    assert g.x.dtype == np.uint8 and g.B.dtype == np.uint8 and g.C.dtype == np.uint8
    assert np.array_equal(g.dt, ref.dt) and np.array_equal(g.dy, ref.dy)
    assert np.max(np.abs(g.as_f64("x") - ref.as_f64("x"))) <= 448 * 2.0 ** -4
