"""Pins for the oracle's one-step rounding ``rho`` (CPU only).

``rho`` is checked against library conversions that round once (numpy fp64->fp32 and
fp64->fp16, torch fp32->bf16 on values that are exact in fp32) and against closed-form cases
chosen so that a double rounding, a wrong tie rule, a wrong subnormal floor or a wrong overflow
threshold each fail.
"""

import numpy as np
import pytest
import torch

from oracle import rho


def _spread(seed, n=200000):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n).astype(np.float64))
    # add exact ties and near-ties for the 16-bit formats
    base = rng.integers(1, 2**11, 2000).astype(np.float64)
    ties = np.concatenate([(base + 0.5) * 2.0**-11, (base + 0.5) * 2.0**-5, (base * 2 + 1) * 2.0**-9])
    return np.concatenate([v, ties, -ties])


@pytest.mark.parametrize("seed", [0, 1])
def test_f32_matches_numpy_cast(seed):
    v = _spread(seed)
    assert np.array_equal(rho(v, "f32"), v.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("seed", [2, 3])
def test_f16_matches_numpy_cast(seed):
    v = _spread(seed) * 1e-3
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(rho(v, "f16"), ref)


def test_bf16_matches_torch_on_fp32_exact_values():
    rng = np.random.default_rng(4)
    v32 = (rng.standard_normal(200000) * np.exp2(rng.integers(-60, 60, 200000))).astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(rho(v32.astype(np.float64), "bf16"), ref)


def test_closed_forms():
    # ties to even
    assert rho([1 + 2**-8], "bf16")[0] == 1.0
    assert rho([1 + 3 * 2**-8], "bf16")[0] == 1 + 2**-6
    assert rho([1 + 2**-11], "f16")[0] == 1.0
    # one step: just above a bf16 tie by less than an fp32 ulp must round up
    assert rho([1 + 2**-8 + 2**-30], "bf16")[0] == 1 + 2**-7
    assert rho([1 + 2**-11 + 2**-40], "f16")[0] == 1 + 2**-10
    # overflow: fp16 max is 65504; 65520 is the tie to 65536 and goes to infinity
    assert rho([65519.0], "f16")[0] == 65504.0
    assert rho([65520.0], "f16")[0] == np.inf
    assert rho([-70000.0], "f16")[0] == -np.inf
    bf16_max = (2 - 2**-7) * 2.0**127
    assert rho([bf16_max], "bf16")[0] == bf16_max
    assert rho([bf16_max + 2.0**119], "bf16")[0] == np.inf  # exact tie rounds to even = 2**128
    assert rho([bf16_max + 2.0**119 - 2.0**100], "bf16")[0] == bf16_max
    # subnormal floor: fp16 smallest subnormal is 2**-24; half of it ties to zero
    assert rho([2**-25], "f16")[0] == 0.0
    assert rho([1.5 * 2**-25], "f16")[0] == 2**-24
    assert rho([3 * 2**-25], "f16")[0] == 2 * 2**-24  # tie between 1 and 2 quanta -> even
    # bf16 subnormals exist below 2**-126 with quantum 2**-133
    assert rho([2**-133], "bf16")[0] == 2**-133
    assert rho([2**-134], "bf16")[0] == 0.0
    # specials
    out = rho([0.0, -0.0, np.inf, -np.inf, np.nan], "bf16")
    assert out[0] == 0 and not np.signbit(out[0])
    assert out[1] == 0 and np.signbit(out[1])
    assert out[2] == np.inf and out[3] == -np.inf and np.isnan(out[4])


def test_f64_is_identity():
    v = _spread(5)
    assert np.array_equal(rho(v, "f64"), v)
