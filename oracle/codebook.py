"""Lloyd-Max codebook for one coordinate of a randomly rotated unit vector (oracle).

Method (TurboQuant vLLM guide, kwkr.cn, section 2 step 2; TurboQuant-MLX page,
core technique item 2): after the random rotation each coordinate of a unit
vector follows a fixed distribution, and the scalar quantiser is the
MSE-optimal (Lloyd-Max) one for that distribution, with 2^b levels.

The exact density of one coordinate X of a uniform unit vector in R^d is
    f_d(x) = C_d (1 - x^2)^((d-3)/2),  x in [-1, 1],
    C_d    = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)),
i.e. (X+1)/2 ~ Beta((d-1)/2, (d-1)/2).  (The pages call it a Beta distribution;
the Gaussian description on the MLX page is its large-d limit.)

Lloyd-Max fixed point: thresholds are midpoints of adjacent centroids, and each
centroid is the conditional mean of X over its cell.  The cell mass uses the
regularised incomplete beta function; the first moment has the closed form
    int_a^b x f_d(x) dx = C_d / (d-1) * [(1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2)].
"""
from __future__ import annotations

import numpy as np
from scipy import special


def _log_cd(d: int) -> float:
    return special.gammaln(d / 2.0) - 0.5 * np.log(np.pi) - special.gammaln((d - 1) / 2.0)


def coord_pdf(x, d: int):
    x = np.asarray(x, dtype=np.float64)
    return np.exp(_log_cd(d) + (d - 3) / 2.0 * np.log1p(-x * x))


def coord_cdf(t, d: int):
    a = (d - 1) / 2.0
    return special.betainc(a, a, (1.0 + np.asarray(t, dtype=np.float64)) / 2.0)


def cell_mass(lo: float, hi: float, d: int) -> float:
    """P(lo < X <= hi), evaluated on the side of zero that avoids cancellation."""
    a = (d - 1) / 2.0
    if lo >= 0.0:   # both in the right tail: use the mirror image 1 - F(t) = F(-t)
        return float(special.betainc(a, a, (1.0 - lo) / 2.0) - special.betainc(a, a, (1.0 - hi) / 2.0))
    return float(special.betainc(a, a, (1.0 + hi) / 2.0) - special.betainc(a, a, (1.0 + lo) / 2.0))


def cell_first_moment(lo: float, hi: float, d: int) -> float:
    e = (d - 1) / 2.0
    c = np.exp(_log_cd(d)) / (d - 1)
    return float(c * ((1.0 - lo * lo) ** e - (1.0 - hi * hi) ** e))


def lloyd_max(d: int, bits: int, tol: float = 4e-15, max_iter: int = 100000):
    """Return (centroids, thresholds) in float64, ascending, symmetric about 0.

    Iterates the two Lloyd-Max conditions until the largest centroid update is at the
    float64 noise floor (below ``tol``, or no longer shrinking for 50 sweeps).
    """
    L = 1 << bits
    a = (d - 1) / 2.0
    # start from the quantiles of the (i + 1/2)/L levels
    c = 2.0 * special.betaincinv(a, a, (np.arange(L) + 0.5) / L) - 1.0
    best, stall = np.inf, 0
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([-1.0], t, [1.0]))
        new = np.array([cell_first_moment(edges[i], edges[i + 1], d) / cell_mass(edges[i], edges[i + 1], d)
                        for i in range(L)])
        new = 0.5 * (new - new[::-1])          # the density is even: c_i = -c_{L-1-i}
        delta = np.max(np.abs(new - c))
        c = new
        if delta < best:
            best, stall = delta, 0
        else:
            stall += 1
        if delta <= tol or (best < 1e-13 and stall >= 50):
            break
    else:
        raise RuntimeError(f"Lloyd-Max did not converge for d={d}, bits={bits}")
    t = 0.5 * (c[:-1] + c[1:])
    return c, t


def distortion(c: np.ndarray, d: int) -> float:
    """Per-coordinate MSE E[(X - Q(X))^2] of a Lloyd-Max codebook (centroids = cell means).

    With c_i the conditional means, E[(X-Q)^2] = E[X^2] - sum_i P_i c_i^2 and E[X^2] = 1/d.
    """
    t = 0.5 * (c[:-1] + c[1:])
    edges = np.concatenate(([-1.0], t, [1.0]))
    p = np.array([cell_mass(edges[i], edges[i + 1], d) for i in range(len(c))])
    return float(1.0 / d - np.sum(p * c * c))


def codebook_f32(d: int, bits: int):
    """The stored codebook: float32 centroids and float32 thresholds (midpoints taken in float64)."""
    c, t = lloyd_max(d, bits)
    return c.astype(np.float32), t.astype(np.float32)
