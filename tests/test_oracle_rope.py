"""Pins for the oracle's rotary embedding and storage rounding."""
import numpy as np
import pytest
import torch

from oracle import rope_rotate, round_to_bf16, round_to_dtype


def _complex_rope(x, pos, theta, begin, end):
    """Independent formulation: pair (x_i, x_{i+h}) as the complex number
    x_i + 1j x_{i+h} and multiply it by exp(1j * pos * theta**(-2i/d_rot))."""
    y = np.array(x, dtype=np.float64, copy=True)
    d_rot = end - begin
    h = d_rot // 2
    z = y[..., begin:begin + h] + 1j * y[..., begin + h:end]
    freq = np.array([theta ** (-2.0 * i / d_rot) for i in range(h)])
    z = z * np.exp(1j * pos * freq)
    y[..., begin:begin + h] = z.real
    y[..., begin + h:end] = z.imag
    return y


@pytest.mark.parametrize("pos", [0, 1, 77, 16383, 131071, 140000])
def test_rope_matches_complex_form(pos):
    # the angle pos * inv_freq carries one fp64 rounding (~pos * 2**-53 rad),
    # and the two formulations may compute inv_freq one ulp apart
    x = np.random.default_rng(pos).standard_normal((3, 128))
    np.testing.assert_allclose(rope_rotate(x, pos, 5e5, 0, 128),
                               _complex_rope(x, pos, 5e5, 0, 128), rtol=0,
                               atol=1e-13 + 2e-15 * pos)


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(0)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    np.testing.assert_array_equal(rope_rotate(q, 0, 1e4, 0, 64), q)
    r = rope_rotate(q, 9999, 1e4, 0, 64)
    assert abs(np.linalg.norm(r) - np.linalg.norm(q)) < 1e-12
    dots = [rope_rotate(q, a + s, 1e4, 0, 64) @ rope_rotate(k, b + s, 1e4, 0, 64)
            for a, b in [(10, 3)] for s in (0, 5, 1000)]
    np.testing.assert_allclose(dots, dots[0], rtol=0, atol=1e-11)
    assert abs(dots[0] - rope_rotate(q, 7, 1e4, 0, 64) @ k) < 1e-11


def test_partial_rope_range_and_off_switch():
    x = np.random.default_rng(1).standard_normal(576)
    y = rope_rotate(x, 1234, 1e4, 512, 576)
    np.testing.assert_array_equal(y[:512], x[:512])
    np.testing.assert_allclose(y, _complex_rope(x, 1234, 1e4, 512, 576), atol=1e-12, rtol=0)
    np.testing.assert_array_equal(rope_rotate(x, 1234, 0.0, 0, 576), x)


def test_bf16_rounding_matches_library_on_fp32_values():
    x32 = np.random.default_rng(2).standard_normal(10000).astype(np.float32) * 3
    lib = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_to_bf16(x32.astype(np.float64)), lib)


def test_bf16_rounding_ties_to_even_in_one_step():
    one = 1.0
    assert round_to_bf16(np.array(one + 2.0 ** -8))[()] == 1.0              # tie -> even
    assert round_to_bf16(np.array(one + 3 * 2.0 ** -8))[()] == 1.0 + 2.0 ** -6
    # just above the tie: rounds up when rounded once from float64 (an fp32
    # intermediate would first land on the tie and then go down to 1.0)
    assert round_to_bf16(np.array(one + 2.0 ** -8 + 2.0 ** -30))[()] == 1.0 + 2.0 ** -7
    assert round_to_bf16(np.array(-2.5e-39))[()] == np.round(-2.5e-39 * 2.0 ** 133) * 2.0 ** -133
    assert round_to_dtype(np.array(0.1), "f32")[()] == float(np.float32(0.1))
