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
