"""Lloyd-Max scalar quantizer for the standard Gaussian, in fp64.

Source: "Closing - The Three-Step Summary", Step 2 (Quantize) and "The One-Slide
Version": once the rotation has made coordinates near-Gaussian, each coordinate is
quantized with the Lloyd-Max codebook that is MSE-optimal for a Gaussian, and the
centroids are scaled by 1/sqrt(d) for head dimension d. The same slide states the
result is within a factor 2.72 of the information-theoretic limit.

A Lloyd-Max quantizer satisfies two conditions (Lloyd 1957 / Max 1960):
  * centroid condition: each reconstruction level is the conditional mean of the
    density over its cell;
  * midpoint condition: each decision threshold is the midpoint of the two
    neighbouring levels.
The Gaussian is symmetric, so the solution is symmetric and, for an even number
of levels, the middle threshold is exactly 0. We solve for the positive half and
mirror it. Plain Lloyd iteration (alternate the two conditions) converges too
slowly at 256 levels, so after a few Lloyd sweeps the same two conditions are
solved with Newton's method; the tests check the conditions by independent
quadrature, not by re-evaluating these formulas.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import ndtr, ndtri

INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def phi(x):
    """Standard normal density; phi(+-inf) = 0."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        out = INV_SQRT_2PI * np.exp(-0.5 * x * x)
    return np.where(np.isinf(x), 0.0, out)


def upper_tail(x):
    """Q(x) = P[X > x] for X ~ N(0,1), accurate far into the upper tail."""
    return ndtr(-np.asarray(x, dtype=np.float64))


def _cells(p):
    """Cell edges (tau_k, tau_{k+1}) of the positive half: tau_0 = 0, tau_K = +inf."""
    K = len(p)
    tau = np.empty(K + 1)
    tau[0] = 0.0
    tau[1:K] = 0.5 * (p[:-1] + p[1:])
    tau[K] = np.inf
    return tau


def _residual(p):
    tau = _cells(p)
    a, b = tau[:-1], tau[1:]
    mass = upper_tail(a) - upper_tail(b)
    first_moment = phi(a) - phi(b)  # integral of x*phi(x) over [a, b]
    return p * mass - first_moment, tau, mass


def _jacobian(p, tau, mass):
    K = len(p)
    J = np.zeros((K, K))
    ft = phi(tau)
    for k in range(K):
        J[k, k] = mass[k]
        if k >= 1:  # dependence through the lower edge tau_k = (p_{k-1} + p_k)/2
            g = (tau[k] - p[k]) * ft[k]
            J[k, k] += 0.5 * g
            J[k, k - 1] += 0.5 * g
        if k <= K - 2:  # dependence through the upper edge tau_{k+1} = (p_k + p_{k+1})/2
            g = (p[k] - tau[k + 1]) * ft[k + 1]
            J[k, k] += 0.5 * g
            J[k, k + 1] += 0.5 * g
    return J


def positive_levels(bits: int, tol: float = 1e-15, max_newton: int = 200) -> np.ndarray:
    """Positive reconstruction levels p_0 < ... < p_{K-1} (K = 2**bits / 2) for N(0,1)."""
    if bits < 1:
        raise ValueError("bits >= 1")
    L = 1 << bits
    K = L // 2
    # start from the Gaussian quantiles of equiprobable cells (upper half)
    p = ndtri(0.5 + (np.arange(K) + 0.5) / L)
    # a few Lloyd sweeps: centroid of each cell given the midpoint thresholds
    for _ in range(50):
        tau = _cells(p)
        p = (phi(tau[:-1]) - phi(tau[1:])) / (upper_tail(tau[:-1]) - upper_tail(tau[1:]))
    # Newton on the centroid condition with midpoint thresholds, damped to keep order
    for _ in range(max_newton):
        F, tau, mass = _residual(p)
        step = np.linalg.solve(_jacobian(p, tau, mass), -F)
        lam = 1.0
        while True:
            cand = p + lam * step
            if cand[0] > 0 and np.all(np.diff(cand) > 0):
                break
            lam *= 0.5
        p = cand
        if np.max(np.abs(lam * step) / np.maximum(1.0, np.abs(p))) < tol:
            break
    # final exact Lloyd sweep removes the last Newton rounding
    tau = _cells(p)
    p = (phi(tau[:-1]) - phi(tau[1:])) / (upper_tail(tau[:-1]) - upper_tail(tau[1:]))
    return p


def levels(bits: int) -> np.ndarray:
    """All 2**bits Lloyd-Max levels for N(0,1), ascending, exactly symmetric (fp64)."""
    p = positive_levels(bits)
    return np.concatenate([-p[::-1], p])


def thresholds_of(levels_: np.ndarray) -> np.ndarray:
    """Midpoint decision thresholds of an ascending set of levels."""
    c = np.asarray(levels_, dtype=np.float64)
    return 0.5 * (c[:-1] + c[1:])


def distortion(levels_: np.ndarray, thresholds: np.ndarray) -> float:
    """E[(X - Q(X))^2] for X ~ N(0,1) and the quantizer with these levels and thresholds.

    Written cell by cell with the Gaussian partial moments
      int_a^b phi = Phi(b) - Phi(a),  int_a^b x phi = phi(a) - phi(b),
      int_a^b x^2 phi = Phi(b) - Phi(a) + a phi(a) - b phi(b).
    """
    c = np.asarray(levels_, dtype=np.float64)
    t = np.asarray(thresholds, dtype=np.float64)
    a = np.concatenate([[-np.inf], t])
    b = np.concatenate([t, [np.inf]])
    mass = ndtr(b) - ndtr(a)
    # use the upper tail on the positive side for accuracy
    pos = a >= 0
    mass[pos] = upper_tail(a[pos]) - upper_tail(b[pos])
    m1 = phi(a) - phi(b)
    with np.errstate(invalid="ignore"):
        aphi = np.where(np.isinf(a), 0.0, a * phi(a))
        bphi = np.where(np.isinf(b), 0.0, b * phi(b))
    m2 = mass + aphi - bphi
    return float(np.sum(m2 - 2.0 * c * m1 + c * c * mass))
