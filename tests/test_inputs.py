"""The seeded input generator against published constants and distribution facts. CPU only."""

import numpy as np

from dropless_grouped_gemm_router_amd import inputs


def test_splitmix64_first_outputs_from_seed_zero():
    # Published SplitMix64 sequence for state 0 (reference implementation by S. Vigna).
    z = inputs._mix64(np.array([1, 2, 3], dtype=np.uint64) * inputs.GOLDEN)
    assert [int(v) for v in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20, 0.0, -0.0],
                 np.float32)
    b = inputs.f32_to_bf16_bits(f)
    assert [int(v) for v in b] == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81, 0x0000, 0x8000]
    assert np.array_equal(inputs.bf16_bits_to_f32(b)[:4], np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5], np.float32))


def test_normal_moments_and_determinism():
    z = inputs.standard_normal(0, 0, 1 << 18)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01
    assert abs(np.mean(z ** 4) - 3.0) < 0.05
    assert np.array_equal(z[:1000], inputs.standard_normal(0, 0, 1000))
    assert not np.array_equal(z[:1000], inputs.standard_normal(0, 1, 1000))
    assert not np.array_equal(z[:1000], inputs.standard_normal(1, 0, 1000))


def test_init_scales_and_storage():
    p = inputs.Problem(64, 4, 2, 256, 64, 128, "bf16")
    t = inputs.make_inputs(p, seed=0, with_grad_out=True)
    assert t["w_router"].stored.dtype == np.float32
    assert t["x"].stored.dtype == np.uint16
    assert abs(t["w_gate"].value.std() * np.sqrt(256) - 1) < 0.05
    assert abs(t["w_down"].value.std() * np.sqrt(64) - 1) < 0.05
    assert abs(t["ws_down"].value.std() * np.sqrt(128) - 1) < 0.05
    assert np.array_equal(inputs.bf16_bits_to_f32(t["x"].stored), t["x"].value)


def test_skew_zero_is_the_uniform_router_and_skew_scales_columns():
    p0 = inputs.Problem(256, 64, 8, 256, 64, 0, "bf16", 128)
    p9 = inputs.Problem(256, 64, 8, 256, 64, 0, "bf16", 128, skew=0.9)
    a = inputs.make_inputs(p0, seed=3)
    b = inputs.make_inputs(inputs.Problem(256, 64, 8, 256, 64, 0, "bf16", 128, skew=0.0), seed=3)
    c = inputs.make_inputs(p9, seed=3)
    for n in a:
        assert np.array_equal(a[n].stored, b[n].stored), n
        if n != "w_router":
            assert np.array_equal(a[n].stored, c[n].stored), n
    # column e scaled by 0.1^(e/63): expert 0 unchanged, expert 63 by 0.1
    ratio = c["w_router"].value / a["w_router"].value
    assert np.allclose(ratio[:, 0], 1.0) and np.allclose(ratio[:, 63], 0.1, rtol=1e-6)
    assert np.allclose(ratio[:, 21], 0.1 ** (21 / 63), rtol=1e-6)


def test_skewed_routing_loads_low_experts():
    """Plausibility: at skew 0.9 the busiest expert carries well over twice
    the mean load, at skew 0 it stays near the mean."""
    from oracle import oracle

    for skew, lo, hi in ((0.0, 1.0, 1.5), (0.9, 2.0, 4.0)):
        p = inputs.Problem(4096, 64, 8, 512, 64, 0, "fp32", 128, skew=skew)
        t = inputs.make_inputs(p, seed=0, names=["x", "w_router"])
        _, idx, _ = oracle.route(t["x"].value, t["w_router"].value, p.top_k)
        frac = np.bincount(idx.ravel(), minlength=64).max() / idx.size
        assert lo < frac * 64 < hi, (skew, frac * 64)
