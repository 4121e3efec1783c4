"""The GELU of the GEMM epilogue (gemm.hip): its fitted constants, evaluated in
float32 as the kernel evaluates them, against the exact z * Phi(z).  Host-side
check of the kernel's constants; the kernel itself is compared with the oracle
in the GPU tests."""
import os
import re

import numpy as np
from scipy.special import ndtr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "protein_language_model_amd", "csrc", "gemm.hip")


def kernel_coefficients():
    found = dict(re.findall(r"constexpr float kGeluP(\d+) = ([-+0-9.e]+)f;", open(SRC).read()))
    return np.array([float(found[str(k)]) for k in range(len(found))], np.float32)


def f32(x):
    return np.asarray(x, np.float64).astype(np.float32)


def gelu_as_kernel(z):
    """Horner in t = min(|z|, 9) with one rounding per FMA, q = exp2 of it,
    then max(z, 0) - t q with one rounding (NaN propagating through the
    minimum and the maximum, as the kernel's IEEE 754-2019 forms do)."""
    z = f32(z)
    co = kernel_coefficients()
    with np.errstate(invalid="ignore", over="ignore"):
        t = np.minimum(np.abs(z), np.float32(9))
        p = np.full_like(t, co[-1])
        for ck in co[-2::-1]:
            p = f32(p.astype(np.float64) * t + np.float64(ck))
        q = f32(np.exp2(p.astype(np.float64)))
        relu = np.where(np.isnan(z), z, np.where(z > 0, z, np.float32(0)))
        return f32(relu.astype(np.float64) - t.astype(np.float64) * q.astype(np.float64))


def test_tail_probability_bounds():
    co = kernel_coefficients()
    assert len(co) == 7
    a = np.linspace(0.0, 9.0, 90001).astype(np.float32)
    p = np.full_like(a, co[-1])
    for ck in co[-2::-1]:
        p = f32(p.astype(np.float64) * a + np.float64(ck))
    q = np.exp2(p.astype(np.float64))
    phi = ndtr(-a.astype(np.float64))
    err = np.abs(q - phi)
    assert err.max() <= 7e-7
    assert (err / phi)[a < 4].max() <= 4e-5
    assert (err / phi)[a < 5].max() <= 7e-4
    assert q[-1] < 2.0 ** -57   # at |z| = 9, where the kernel switches to q = 0 (Phi(-9) ~ 1.1e-19)


def test_gelu_against_exact():
    z = np.concatenate([np.linspace(-12, 12, 240001), -np.logspace(-30, 1.1, 2000), np.logspace(-30, 1.1, 2000)])
    g = gelu_as_kernel(z).astype(np.float64)
    zz = f32(z).astype(np.float64)
    exact = zz * ndtr(zz)
    # q's error (absolute 7e-7, relative 4e-5 below |z| = 4) plus two fp32 roundings
    bound = 7e-7 * np.abs(zz) + 2.0 ** -23 * np.abs(exact)
    tail = np.abs(zz) < 4
    assert np.all(np.abs(g - exact)[tail] <= np.maximum(bound, 4e-5 * np.abs(exact) + 2.0 ** -23 * np.abs(exact))[tail])
    # below half a bf16 ulp of the result wherever the result is a normal float
    normal = np.abs(exact) > 1e-30
    assert np.all((np.abs(g - exact) <= 2.0 ** -9 * np.abs(exact))[normal & (np.abs(zz) < 5)])
    assert np.all(np.abs(g - exact) <= bound + 1e-30)
    # the sign of the result is the sign of z (no cancellation to +0 in the
    # tail); from z = -9 down the tail term is held at its value at 9: one
    # negative constant within 2.5e-18 of the exact value
    inner = (zz != 0) & (np.abs(zz) < 9) & (np.abs(exact) > 1e-37)
    assert np.all(np.sign(g[inner]) == np.sign(zz[inner]))
    far = zz <= -9
    assert np.all(g[far] == g[far][0]) and -2.5e-18 < g[far][0] < 0
    assert np.all(np.abs(g[far] - exact[far]) < 2.5e-18)


def test_gelu_special_values():
    g = gelu_as_kernel(np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e30, -1e30, -9.5, 9.5]))
    tail = gelu_as_kernel(np.array([-9.0]))[0]
    assert -2.5e-18 < tail < 0
    assert g[0] == 0 and g[1] == 0
    assert g[2] == np.inf
    assert g[3] == tail and np.isnan(g[4])   # -inf: the held tail value; NaN stays NaN
    assert g[5] == np.float32(1e30)
    assert g[6] == tail and g[7] == tail and g[8] == np.float32(9.5)
