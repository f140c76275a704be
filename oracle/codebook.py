"""Lloyd-Max codebooks for rotated, L2-normalized coordinates (oracle; test infrastructure).

Follows [Spec] "Step 2: Lloyd-Max Scalar Quantization" and "Codebook Generation":
after a random orthogonal rotation each coordinate of a unit vector follows a
Beta(d/2, d/2) law (on [0, 1], centred at 1/2); the quantizer is the Lloyd-Max
quantizer of that law: start from uniform boundaries, set each centroid to the
conditional mean of its cell, set each boundary to the midpoint of its two
neighbouring centroids, repeat until converged.  [Spec] "As-Built Notes" fixes the
normalization to the vector L2 norm, so the quantizer acts on y = 2u - 1 in
[-1, 1], whose density is proportional to (1 - y^2)^m with m = d/2 - 1.

Readings where the pages leave a step open:

* the literal Beta(d/2, d/2) law is used (m = d/2 - 1); the exact marginal of a
  coordinate of a uniform point on the sphere has m' = (d - 3)/2, which is only
  used to state the expected round-trip MSE (``distortion(..., m=m_sphere(d))``);
* the pages say "~20 iterations"; that does not converge from a uniform start, so
  the iteration runs until the largest boundary change is below 1e-12;
* quadrature is not specified: composite Gauss-Legendre in fp64 for the cell mass,
  and the closed form -(1 - y^2)^(m+1) / (2(m+1)) for the first moment;
* the table is stored as fp32, rounded to nearest from the fp64 fixed point.

Only the positive half is iterated; the negative half is its mirror image, and the
middle boundary is exactly 0 for an even number of levels.
"""

from __future__ import annotations

import numpy as np

_GL_NODES, _GL_WEIGHTS = np.polynomial.legendre.leggauss(48)


def m_beta(dim: int) -> float:
    """Exponent m of (1 - y^2)^m for the Beta(d/2, d/2) law of [Spec] Step 1/2."""
    return dim / 2.0 - 1.0


def m_sphere(dim: int) -> float:
    """Exponent of the exact marginal of one coordinate of a uniform unit vector."""
    return (dim - 3) / 2.0


def _mass(a: np.ndarray, b: np.ndarray, m: float, panels: int = 32) -> np.ndarray:
    """Integral of (1 - y^2)^m over [a, b], elementwise, by composite Gauss-Legendre."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    edges = a[..., None] + (b - a)[..., None] * np.linspace(0.0, 1.0, panels + 1)
    lo, hi = edges[..., :-1], edges[..., 1:]
    half = 0.5 * (hi - lo)
    mid = 0.5 * (hi + lo)
    y = mid[..., None] + half[..., None] * _GL_NODES
    f = np.clip(1.0 - y * y, 0.0, None) ** m
    return np.sum(np.sum(f * _GL_WEIGHTS, axis=-1) * half, axis=-1)


def _first_moment(a: np.ndarray, b: np.ndarray, m: float) -> np.ndarray:
    """Integral of y (1 - y^2)^m over [a, b] (closed form)."""
    fa = np.clip(1.0 - np.asarray(a, np.float64) ** 2, 0.0, None) ** (m + 1.0)
    fb = np.clip(1.0 - np.asarray(b, np.float64) ** 2, 0.0, None) ** (m + 1.0)
    return (fa - fb) / (2.0 * (m + 1.0))


def _second_moment_about(a, b, c, m: float, panels: int = 32) -> np.ndarray:
    """Integral of (y - c)^2 (1 - y^2)^m over [a, b] by composite Gauss-Legendre."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    edges = a[..., None] + (b - a)[..., None] * np.linspace(0.0, 1.0, panels + 1)
    lo, hi = edges[..., :-1], edges[..., 1:]
    half = 0.5 * (hi - lo)
    mid = 0.5 * (hi + lo)
    y = mid[..., None] + half[..., None] * _GL_NODES
    f = np.clip(1.0 - y * y, 0.0, None) ** m * (y - c[..., None, None]) ** 2
    return np.sum(np.sum(f * _GL_WEIGHTS, axis=-1) * half, axis=-1)


def lloyd_max_fp64(bits: int, dim: int = 128, m: float | None = None,
                   tol: float = 1e-12, max_iter: int = 100000,
                   init: np.ndarray | None = None):
    """Lloyd-Max fixed point in fp64 for density proportional to (1 - y^2)^m on [-1, 1].

    Returns (boundaries[L-1], centroids[L], iterations).  ``init`` optionally gives
    the positive boundaries (L/2 - 1 values, ascending, in (0, 1)) to start from;
    by default the start is the uniform grid y_k = 2k/L - 1 of [Spec]
    "Codebook Generation" (uniform in u = (y + 1)/2).
    """
    if m is None:
        m = m_beta(dim)
    L = 1 << bits
    half = L // 2
    if init is None:
        pos = np.array([2.0 * k / L - 1.0 for k in range(half + 1, L)], dtype=np.float64)
    else:
        pos = np.array(init, dtype=np.float64)
    it = 0
    for it in range(1, max_iter + 1):
        edges = np.concatenate(([0.0], pos, [1.0]))
        a, b = edges[:-1], edges[1:]
        cent = _first_moment(a, b, m) / _mass(a, b, m)
        new_pos = 0.5 * (cent[:-1] + cent[1:])
        delta = np.max(np.abs(new_pos - pos)) if pos.size else 0.0
        pos = new_pos
        if delta < tol:
            break
    edges = np.concatenate(([0.0], pos, [1.0]))
    cent = _first_moment(edges[:-1], edges[1:], m) / _mass(edges[:-1], edges[1:], m)
    boundaries = np.concatenate((-pos[::-1], [0.0], pos))
    centroids = np.concatenate((-cent[::-1], cent))
    return boundaries, centroids, it


def codebook(bits: int, dim: int = 128):
    """fp32 table (boundaries[L-1], centroids[L]) as the kernels consume it."""
    b, c, _ = lloyd_max_fp64(bits, dim)
    return b.astype(np.float32), c.astype(np.float32)


def distortion(boundaries, centroids, m: float) -> float:
    """Mean squared error per coordinate, E (y - Q(y))^2, under density prop. to (1-y^2)^m."""
    b = np.asarray(boundaries, np.float64)
    c = np.asarray(centroids, np.float64)
    edges = np.concatenate(([-1.0], b, [1.0]))
    num = np.sum(_second_moment_about(edges[:-1], edges[1:], c, m))
    den = np.sum(_mass(edges[:-1], edges[1:], m))
    return float(num / den)
