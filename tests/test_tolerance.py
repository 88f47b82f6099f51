"""The 16-bit parity bar itself (tests/helpers.elementwise_tolerance), checked on the CPU.

A correctly rounded output must always pass it (whatever its magnitude), and an output one
full unit in the last place off must fail wherever the bar is wider than the flat 2e-3."""
import numpy as np
import pytest

from tests.helpers import FP32_MARGIN, TOL, elementwise_tolerance, half_ulp


def round_to_bits(x, dtype):
    """float64 -> nearest representable value of the 16-bit type (ties to even), as float64.
    bf16: float32 first (exact for these inputs), then the upper 16 bits with RNE."""
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float64)
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def ulp_at(x, dtype):
    return 2 * half_ulp(x, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_correctly_rounded_outputs_pass(dtype):
    rng = np.random.default_rng(0)
    # exact values over [1e-3, 20): below and above the points where the flat bar stops being
    # attainable (1 for bf16, 8 for f16)
    x = np.exp(rng.uniform(np.log(1e-3), np.log(20.0), 200000)) * rng.choice([-1, 1], 200000)
    got = round_to_bits(x, dtype)
    assert np.all(np.abs(got - x) <= elementwise_tolerance(x, dtype))
    # Where the bar is raised, a float32 error up to FP32_MARGIN before the rounding is
    # absorbed as well.
    tol = elementwise_tolerance(x, dtype)
    raised = tol > TOL[dtype]
    assert raised.any() and (~raised).any()
    got2 = round_to_bits(x + rng.uniform(-1, 1, x.shape) * FP32_MARGIN * 0.99, dtype)
    assert np.all(np.abs(got2 - x)[raised] <= tol[raised])


@pytest.mark.parametrize("dtype,lo", [("bf16", 1.0), ("f16", 8.0)])
def test_one_ulp_off_fails_where_the_bar_is_raised(dtype, lo):
    rng = np.random.default_rng(1)
    x = rng.uniform(lo, 4 * lo, 10000)
    got = round_to_bits(x, dtype)
    away = np.where(got >= x, 1.0, -1.0)
    wrong = got + away * ulp_at(x, dtype)   # one output step beyond the correctly rounded value
    tol = elementwise_tolerance(x, dtype)
    assert np.all(tol > TOL[dtype])
    assert np.all(np.abs(wrong - x) > tol)


def test_flat_bar_below_one_for_bf16():
    x = np.array([0.0, 1e-4, 0.3, 0.5, 0.75, 0.999])
    assert np.all(elementwise_tolerance(x, "bf16") == TOL["bf16"])
    assert np.all(elementwise_tolerance(x, "f32") == TOL["f32"])
    # exactly at 1 the half ulp (2^-8) exceeds the flat bar
    assert elementwise_tolerance(np.array([1.0]), "bf16")[0] == pytest.approx(2.0 ** -8 + FP32_MARGIN)
