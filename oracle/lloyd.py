"""Lloyd-Max magnitude levels for ParisKV's 3-bit coordinate magnitudes, float64.

Test infrastructure (see the package docstring).

Source: ParisKV close-reading, section 2.4 (paper Proposition 4.1, Eqs.
(11)-(12), Appendix B.1): each coordinate of a unit subspace direction gets
1 sign bit + 3 magnitude bits; the eight magnitude reconstruction values come
from offline Lloyd-Max scalar quantisation under the prior
(u_b)_j^2 ~ Beta(1/2, (m-1)/2), so they depend on m only.

Reading (the page gives no numbers): y = |u_j| has density proportional to
(1 - y^2)^((m-3)/2) on [0, 1]; Lloyd-Max for squared error alternates
"thresholds = midpoints of adjacent levels" and "level = conditional mean of
its cell" until a fixed point; |u| >= threshold goes to the upper cell.  The
cell masses use the regularised incomplete beta function
(integral_0^t (1-y^2)^a dy = B(1/2, a+1) I_{t^2}(1/2, a+1) / 2) and the cell
first moments the closed form (1 - t^2)^(a+1) / (2(a+1)).
"""
from __future__ import annotations

import numpy as np
from scipy.special import beta as beta_fn
from scipy.special import betainc


def _cells(m: int):
    a = (m - 3) / 2.0
    c = 0.5 * beta_fn(0.5, a + 1.0)

    def mass(t1, t2):
        return c * (betainc(0.5, a + 1.0, t2 * t2) - betainc(0.5, a + 1.0, t1 * t1))

    def moment(t1, t2):
        return ((1.0 - t1 * t1) ** (a + 1.0) - (1.0 - t2 * t2) ** (a + 1.0)) / (2.0 * (a + 1.0))

    return mass, moment


def lloyd_max_abs_coord(m: int, n_levels: int = 8, tol: float = 1e-15, max_iter: int = 20000):
    """Float64 Lloyd-Max fixed point: (levels[n_levels], thresholds[n_levels-1])."""
    mass, moment = _cells(m)
    levels = (np.arange(n_levels) + 0.5) / n_levels
    for _ in range(max_iter):
        th = 0.5 * (levels[:-1] + levels[1:])
        edges = np.concatenate([[0.0], th, [1.0]])
        new = moment(edges[:-1], edges[1:]) / mass(edges[:-1], edges[1:])
        if np.max(np.abs(new - levels)) <= tol:
            levels = new
            break
        levels = new
    th = 0.5 * (levels[:-1] + levels[1:])
    return levels, th


def codebook_f32(m: int, n_levels: int = 8):
    """The frozen fp32 codebook: fp32(levels), fp32(midpoints in float64)."""
    lv, th = lloyd_max_abs_coord(m, n_levels)
    return lv.astype(np.float32), th.astype(np.float32)
