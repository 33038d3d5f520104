"""Pins of the FP8 (E4M3) cache oracle against things other than itself.

(a) torch's ``float8_e4m3fn`` dtype (a library implementation of OCP E4M3)
decodes every code and rounds float32 values in range; (b) values fixed by
the format itself (1.0, the largest finite value, the smallest subnormal,
NaN codes); (c) brute force: the chosen code is nearest over all 254 finite
codes, ties to an even mantissa; (d) saturation; (e) quantize/dequantize
round trip within half a step, which is what attention over the cache sees.
"""

import numpy as np
import pytest
import torch

import oracle.fp8 as fp8


ALL = np.arange(256, dtype=np.uint8)


def _torch_value(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_code(x32):
    t = torch.from_numpy(np.asarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_every_code_decodes_like_torch():
    got, want = fp8.e4m3_value(ALL), _torch_value(ALL)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def test_values_fixed_by_the_format():
    assert fp8.e4m3_value(0x38) == 1.0
    assert fp8.e4m3_value(0x7E) == 448.0 == fp8.E4M3_MAX
    assert fp8.e4m3_value(0xFE) == -448.0
    assert fp8.e4m3_value(0x01) == 2.0 ** -9            # smallest subnormal
    assert fp8.e4m3_value(0x08) == 2.0 ** -6            # smallest normal
    assert fp8.e4m3_value(0xC0) == -2.0
    assert np.isnan(fp8.e4m3_value(0x7F)) and np.isnan(fp8.e4m3_value(0xFF))
    # finite codes round-trip through the encoder
    finite = ALL[(ALL & 0x7F) != 0x7F]
    assert np.array_equal(fp8.e4m3_code(fp8.e4m3_value(finite)), finite)


def test_rounding_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * 3,
        rng.standard_normal(5000) * 100,
        rng.standard_normal(5000) * 2.0 ** -7,           # subnormal range
        rng.uniform(-448, 448, 5000),
    ]).astype(np.float32)
    # exact midpoints between neighbouring finite magnitudes, both signs
    mags = fp8.e4m3_value(np.arange(0x7F))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (mags[:-1] + mags[1:]) / 2)
    x = np.concatenate([x, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1000)])
    assert np.array_equal(fp8.e4m3_code(x.astype(np.float64)), _torch_code(x))


def test_nearest_by_brute_force_with_ties_to_even():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(400) * 10, rng.standard_normal(100) * 0.01])
    finite = ALL[(ALL & 0x7F) != 0x7F]
    vals = fp8.e4m3_value(finite)
    mags = fp8.e4m3_value(np.arange(0x7F))
    ties = (mags[:-1] + mags[1:]) / 2
    for xi in np.concatenate([x, ties, -ties]):
        c = int(fp8.e4m3_code(xi))
        d = np.abs(vals - xi)
        best = finite[d == d.min()]
        if len(best) == 1:
            assert c == int(best[0]) or (xi == 0 and c & 0x7F == 0)
        else:
            # a tie: the even mantissa wins, and the sign follows x
            even = [int(b) for b in best if int(b) % 2 == 0 and (int(b) >> 7) == (xi < 0)]
            assert c in even, (xi, c, best)


def test_saturation_and_signed_zero():
    assert np.array_equal(fp8.e4m3_code(np.array([448.0, 460.0, 1e6, 1e300])), [0x7E] * 4)
    assert np.array_equal(fp8.e4m3_code(np.array([-449.0, -1e9])), [0xFE] * 2)
    assert int(fp8.e4m3_code(0.0)) == 0x00
    assert int(fp8.e4m3_code(-0.0)) == 0x80
    assert int(fp8.e4m3_code(-2.0 ** -12)) == 0x80        # rounds to -0


@pytest.mark.parametrize("scale", [1.0, 0.0173, 3.5])
def test_round_trip_within_half_a_step(scale):
    rng = np.random.default_rng(2)
    x = rng.standard_normal(10000) * 40 * scale
    x = np.clip(x, -448 * scale, 448 * scale)
    back = fp8.dequantize(fp8.quantize(x, scale), scale)
    # spacing of E4M3 around |v|: 2^(floor(log2|v|) - 3), at least 2^-9
    v = np.abs(x) / scale
    step = np.exp2(np.floor(np.log2(np.maximum(v, 2.0 ** -6))) - 3) * scale
    assert (np.abs(back - x) <= step / 2 * (1 + 1e-12)).all()
