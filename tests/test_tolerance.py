"""The output-rounding allowance the GPU parity tests add to the stated tolerance: half a unit in
the last place of the output type, checked against numpy's own spacing of float16/float32 and
against bf16 spacing built from its 8-bit significand. CPU only."""
import numpy as np
import pytest

pytest.importorskip("torch")
from _gpu_cases import excess_error, half_ulp  # noqa: E402


@pytest.mark.parametrize("dtype,np_t", [("f16", np.float16), ("f32", np.float32)])
def test_half_ulp_matches_numpy_spacing(dtype, np_t):
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 3, 500), rng.normal(0, 1e-3, 100), [1.0, 2.0, -4.0, 65000.0]])
    x = x.astype(np_t)  # representable values: spacing is exact there
    want = np.spacing(np.abs(x)).astype(np.float64) / 2  # the binade of |x|, away from zero
    assert np.array_equal(half_ulp(x.astype(np.float64), dtype), want)


def test_half_ulp_bf16():
    # bf16 keeps 8 significant bits: the spacing in [2^e, 2^(e+1)) is 2^(e-7)
    for e in range(-20, 20):
        for frac in (1.0, 1.25, 1.9921875):
            x = frac * 2.0 ** e
            assert half_ulp(np.array([x, -x]), "bf16").tolist() == [2.0 ** (e - 8)] * 2


def test_excess_error():
    ref = np.array([0.5, 3.0, 5.0])
    got = ref + np.array([0.001, 0.009, -0.02])
    # bf16 half-ulps: 2^-9, 2^-7, 2^-6
    assert excess_error(got, ref, "bf16") == pytest.approx(max(0.001 - 2 ** -9, 0.009 - 2 ** -7,
                                                               0.02 - 2 ** -6))
    assert excess_error(np.zeros(0), np.zeros(0), "f16") == 0.0
