"""Fit of the arctangent polynomial the triplet encoder uses (atan01 in
csrc/tq_octo.hip): atan(a) ~ a * P(a^2) on [0, 1], P of degree 7.

Lawson's iteratively reweighted least squares toward the minimax (equal
ripple) fit of the odd polynomial, on a dense Chebyshev grid in float64.
The coefficients are then rounded to fp32 and the error of the fp32 Horner
evaluation (one fused multiply-add per step, emulated exactly in float64) is
measured on a finer grid.

    python -m kv_cache_vector_encode_amd.fit_atan

prints the coefficients, highest degree first, and the largest error in
radians.  Build-time tool: the kernels do not import it.
"""

from __future__ import annotations

import numpy as np

DEGREE = 7      # P(s) = sum_k c_k s^k, k = 0 .. 7


def fit(degree: int = DEGREE, points: int = 4001, iters: int = 300) -> np.ndarray:
    """Coefficients c_0 .. c_degree (float64) of P."""
    t = np.cos(np.pi * (np.arange(points) + 0.5) / points)          # Chebyshev nodes on [-1, 1]
    a = 0.5 * (t + 1.0)                                               # on [0, 1]
    A = np.stack([a ** (2 * k + 1) for k in range(degree + 1)], axis=1)
    f = np.arctan(a)
    w = np.full(points, 1.0 / points)
    c = np.zeros(degree + 1)
    for _ in range(iters):
        sw = np.sqrt(w)
        c, *_ = np.linalg.lstsq(A * sw[:, None], f * sw, rcond=None)
        e = np.abs(A @ c - f)
        w = w * e
        w /= w.sum()
    return c


def horner_fp32(coeffs32: np.ndarray, a: np.ndarray) -> np.ndarray:
    """a * P(a^2) as the kernel evaluates it in fp32: s = a*a rounded, then
    p = fma(p, s, c) from the highest coefficient down (each fma exact in
    float64 and rounded once to fp32), then a * p rounded."""
    a32 = a.astype(np.float32)
    s = (a32.astype(np.float64) * a32).astype(np.float32)
    p = np.full_like(s, coeffs32[-1])
    for c in coeffs32[-2::-1]:
        p = (p.astype(np.float64) * s + np.float64(c)).astype(np.float32)
    return (a32.astype(np.float64) * p).astype(np.float32)


def max_error_fp32(coeffs32: np.ndarray, n: int = 1_000_001) -> float:
    a = np.linspace(0.0, 1.0, n)
    a32 = a.astype(np.float32)
    return float(np.max(np.abs(horner_fp32(coeffs32, a32).astype(np.float64) - np.arctan(a32.astype(np.float64)))))


def main() -> None:
    c32 = fit().astype(np.float32)
    for c in c32[::-1]:
        print(f"{float(c):.9e}f")
    print(f"max |a P(a^2) - atan(a)| in fp32 on [0, 1]: {max_error_fp32(c32):.3e} rad")


if __name__ == "__main__":
    main()
