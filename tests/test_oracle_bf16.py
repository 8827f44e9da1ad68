"""Pins for the oracle's bf16 conversions (CPU only).

f64_to_bf16 must be the single, direct round-to-nearest-even of an fp64 value
to bf16.  It is pinned against torch's fp32->bf16 conversion (a library
routine) on fp32-representable inputs, against hand-made double-rounding
traps where going through fp32 first gives the wrong answer, and against a
brute-force nearest-neighbour check.
"""

import numpy as np
import pytest
import torch

from oracle import bf16_to_f64, f64_to_bf16


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_every_bf16_value_is_a_fixed_point():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_to_f64(bits)
    finite = np.isfinite(vals)
    back = f64_to_bf16(vals[finite])
    assert np.array_equal(back, bits[finite])
    # infinities survive, NaNs stay NaNs
    inf_bits = bits[np.isinf(vals)]
    assert np.array_equal(f64_to_bf16(bf16_to_f64(inf_bits)), inf_bits)
    nan_back = f64_to_bf16(vals[np.isnan(vals)])
    assert np.all(np.isnan(bf16_to_f64(nan_back)))


def test_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(7)
    # wide exponent range, both signs, fp32 subnormals and near-overflow values
    mant = rng.uniform(1.0, 2.0, 200000)
    expo = rng.integers(-149, 128, 200000)
    sign = rng.choice([-1.0, 1.0], 200000)
    x32 = (sign * np.ldexp(mant, expo)).astype(np.float32)
    x32 = np.concatenate([x32, rng.standard_normal(100000).astype(np.float32),
                          np.array([0.0, -0.0, 3.3895e38, -3.3895e38, 1e-45], np.float32)])
    x32 = x32[np.isfinite(x32)]
    ours = f64_to_bf16(x32.astype(np.float64))
    assert np.array_equal(ours, _torch_bf16_bits(x32))


@pytest.mark.parametrize("x, expect", [
    # 1 + 2^-8 is the exact midpoint between 1 and 1 + 2^-7: ties to even -> 1
    (1.0 + 2.0**-8, 0x3F80),
    # a hair above the midpoint must round up; via fp32 the hair is lost and
    # the tie would go down to 1.0 (the double-rounding trap)
    (1.0 + 2.0**-8 + 2.0**-40, 0x3F81),
    (-(1.0 + 2.0**-8 + 2.0**-40), 0xBF81),
    # a hair below the midpoint rounds down
    (1.0 + 2.0**-8 - 2.0**-40, 0x3F80),
    # midpoint between 1+2^-7 (odd) and 1+2^-6 (even): ties to even -> up
    (1.0 + 3 * 2.0**-8, 0x3F82),
    # 2^-133 is the smallest bf16 subnormal; half of it ties to +0
    (2.0**-133, 0x0001),
    (2.0**-134, 0x0000),
    (2.0**-134 + 2.0**-160, 0x0001),
    # overflow: the largest bf16 is (2 - 2^-7) * 2^127; the midpoint above it goes to inf
    ((2 - 2.0**-7) * 2.0**127, 0x7F7F),
    ((2 - 2.0**-8) * 2.0**127, 0x7F80),
    (1e300, 0x7F80),
    (-1e300, 0xFF80),
])
def test_single_rounding_cases(x, expect):
    assert int(f64_to_bf16(np.array([x]))[0]) == expect


def test_nearest_by_brute_force():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(50000) * np.exp2(rng.integers(-20, 20, 50000))
    b = f64_to_bf16(x).astype(np.int64)
    here = bf16_to_f64(b.astype(np.uint16))
    # neighbours one bf16 step above and below in magnitude (same sign)
    up = bf16_to_f64((b + 1).astype(np.uint16))
    dn = bf16_to_f64((b - 1).astype(np.uint16))
    d0 = np.abs(x - here)
    assert np.all(d0 <= np.abs(x - up))
    assert np.all(d0 <= np.abs(x - dn))
    # exact ties must land on an even pattern
    tie = (d0 == np.abs(x - up)) | (d0 == np.abs(x - dn))
    assert np.all(b[tie] % 2 == 0)
