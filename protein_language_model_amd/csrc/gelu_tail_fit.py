"""Coefficients of the GELU epilogue in gemm.hip (run once; prints C constants).

GELU(z) = z Phi(z), Phi the standard normal CDF.  The kernel evaluates
q = Phi(-a), a = min(|z|, 9), as 2^P(a) with P a degree-6 polynomial fitted to
log2 Phi(-a) on [0, 9], and GELU(z) = z (1 - q) for z >= 0, z q for z < 0.
The fit is a weighted least-squares Chebyshev fit, reweighted (Lawson) towards
the minimax of |2^P - Phi| / max(Phi, 1e-3): absolute error where Phi is
large, relative error in the tail, where z q is the result itself.  The
printed bounds evaluate P in float32 by Horner's rule, as the kernel does.
"""
import numpy as np
from scipy.special import log_ndtr, ndtr

DEGREE, A, TAU = 6, 9.0, 1e-3


def fit(degree=DEGREE, a_max=A, tau=TAU, n=40001, iters=60):
    a = np.linspace(0.0, a_max, n)
    t = a / a_max * 2.0 - 1.0
    f = log_ndtr(-a) / np.log(2.0)
    phi = ndtr(-a)
    scale = np.maximum(phi, tau)
    w = (phi / scale) ** 2
    for _ in range(iters):
        c = np.polynomial.chebyshev.chebfit(t, f, degree, w=np.sqrt(w))
        err = np.abs(np.exp2(np.polynomial.chebyshev.chebval(t, c)) - phi) / scale
        w = w * (err / err.max() + 1e-3)
        w /= w.max()
    # monomial coefficients in a (lowest order first), rounded to float32
    poly_t = np.polynomial.Polynomial(np.polynomial.chebyshev.cheb2poly(c))
    return poly_t(np.polynomial.Polynomial([-1.0, 2.0 / a_max])).coef.astype(np.float32)


def horner_f32(coef, a):
    a = np.asarray(a, np.float32)
    p = np.full_like(a, coef[-1])
    for ck in coef[-2::-1]:
        p = (p.astype(np.float64) * a + np.float64(ck)).astype(np.float32)  # one rounding, as an fma
    return p


if __name__ == "__main__":
    co = fit()
    a = np.linspace(0.0, A, 200001).astype(np.float32)
    phi = ndtr(-a.astype(np.float64))
    q = np.exp2(horner_f32(co, a).astype(np.float64))
    for k, ck in enumerate(co):
        print(f"constexpr float kGeluP{k} = {float(ck)!r}f;")
    print(f"// float32: max |q - Phi(-a)| = {np.abs(q - phi).max():.2e} on [0, {A}];", end="")
    for hi in (4.0, 5.0, 6.0):
        m = a < hi
        print(f" max rel a < {hi:g}: {(np.abs(q - phi) / phi)[m].max():.1e};", end="")
    print()
