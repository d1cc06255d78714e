"""The per-element bars of the GPU parity tests, on the CPU: half a unit in the last place of the
output type (against numpy's own spacing of float16/float32 and bf16 spacing built from its 8-bit
significand); the stated tolerance, widened by that half unit only where it reaches the
tolerance itself; and the prefill arithmetic bound, against a direct simulation of the kernel's
documented arithmetic (weights rounded to 16 bits, the same rounded weights summed) on random
inputs."""
import numpy as np
import pytest

pytest.importorskip("torch")
from _gpu_cases import (TOL, excess_error, half_ulp, parity_bar,  # noqa: E402
                        prefill_bound)


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


def test_parity_bar_allowance_only_where_the_bar_is_unattainable():
    # bf16: half ulp 2^-7 at [2, 4) < 1e-2 (plain bar); 2^-6 at [4, 8) > 1e-2 (allowance)
    ref = np.array([0.3, 1.5, 3.99, 4.0, 6.0, -5.0])
    bar = parity_bar(ref, "bf16")
    assert bar.tolist() == [1e-2, 1e-2, 1e-2, 1e-2 + 2 ** -6, 1e-2 + 2 ** -6, 1e-2 + 2 ** -6]
    # fp16 reaches it from 32 on (half ulp 2^-6), fp32 from 256 on (2^-16)
    assert parity_bar(np.array([31.9, 32.0]), "f16").tolist() == [1e-2, 1e-2 + 2 ** -6]
    assert parity_bar(np.array([255.0, 256.0]), "f32").tolist() == [1e-5, 1e-5 + 2 ** -16]
    for dt in ("f32", "f16", "bf16"):
        x = np.linspace(-3, 3, 1001)
        assert (parity_bar(x, dt) == TOL[dt]).all()


def _rne(x, dtype):
    import torch
    t = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return torch.from_numpy(np.asarray(x, np.float32)).to(t).to(torch.float64).numpy()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_bound_covers_simulated_kernel_arithmetic(dtype):
    """Weights 2^(z - m) with m one of the scores (at most 2^8 above it), rounded to the 16-bit
    type; numerator and denominator from the same rounded weights in fp32; output rounded to the
    type. The bound must hold on every element, and be reasonably tight (not vacuous)."""
    rng = np.random.default_rng(3)
    worst, ratios = 0.0, []
    for n in (1, 2, 3, 5, 17, 64, 300, 2000):
        for _ in range(4):
            d = 32
            V = _rne(rng.standard_normal((n, d)) * rng.choice([0.5, 1, 3]), dtype)
            z = rng.standard_normal(n) * rng.choice([0.5, 2, 6])
            w = np.exp(z - z.max())
            w /= w.sum()
            o = w @ V
            m2 = w @ (V * V)
            m = z[rng.integers(n)] if n > 1 else z[0]
            m = max(m, z.max() - 8 * np.log(2))             # lazy maximum within 2^8
            p = np.exp2((z - m) / np.log(2)).astype(np.float32)
            pr = _rne(p, dtype).astype(np.float32)
            num = (pr[:, None] * V.astype(np.float32)).sum(0, dtype=np.float32)
            den = pr.sum(dtype=np.float32)
            got = _rne(num / den, dtype)
            vmax = float(np.abs(V).max())
            bound = prefill_bound(o, m2, n, vmax, dtype)
            err = np.abs(got - o)
            assert (err <= bound).all(), (n, float((err / bound).max()))
            worst = max(worst, float((err / bound).max()))
            ratios.append(float(np.median(bound)))
    assert worst > 0.05, worst              # the bound is not vacuously loose
