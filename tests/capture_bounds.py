"""Which keep decisions of pattern capture a small error in the maps can change (test helper).

Capture thresholds continuous values twice: t >= tau per cell, then hits / length >= mu per
pattern.  Maps computed another way (fp32 on the GPU) carry a small error, which can flip a
decision lying close to a threshold.  Given reference maps A and a bound
|A' - A| <= rel * A + abs, `certain_patterns` marks the patterns whose keep decision is the
same for every A' within the bound.  It uses interval bounds on the normalised value
t = (y - ymin) / (ymax - ymin), y = (sqrt(A + eps) - 1) / 0.5, min and max over the causal
row: t grows with y and falls as ymin or ymax grow, so the extremes of t come from the
extremes of y, ymin and ymax taken separately (a superset of what any A' can reach).
"""
import numpy as np


def _y(x, eps):
    return (np.sqrt(x + eps) - 1.0) / 0.5


def certain_patterns(A, rel, ab, eps=1e-8, tau=0.3, mu=0.8):
    """A: maps [n, L, L] (rows j <= i used).  Returns (certain_diag, certain_vert), bool [n, L]."""
    A = np.asarray(A, dtype=np.float64)
    n, L, _ = A.shape
    tri = np.tri(L, dtype=bool)
    cd = np.zeros((n, L), bool)
    cv = np.zeros((n, L), bool)
    i_idx, j_idx = np.nonzero(tri)
    r_idx = i_idx - j_idx
    length = (L - np.arange(L)).astype(np.float64)
    for m in range(n):
        a = A[m]
        ylo = _y(np.maximum(a * (1.0 - rel) - ab, 0.0), eps)
        yhi = _y(a * (1.0 + rel) + ab, eps)
        ymin_lo = np.where(tri, ylo, np.inf).min(axis=1)[:, None]
        ymin_hi = np.where(tri, yhi, np.inf).min(axis=1)[:, None]
        ymax_lo = np.where(tri, ylo, -np.inf).max(axis=1)[:, None]
        ymax_hi = np.where(tri, yhi, -np.inf).max(axis=1)[:, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            tmax = (yhi - ymin_lo) / (ymax_lo - ymin_lo)
            tmin = (ylo - ymin_hi) / (ymax_hi - ymin_hi)
        sure_in = tri & (tmin >= tau)
        sure_out = tri & (tmax < tau)
        shaky = (ymax_lo - ymin_hi <= 0.0)[:, 0]    # rows whose range may vanish: nothing is sure
        sure_in[shaky] = False
        sure_out[shaky] = False
        if tau <= 1.0:                              # row 0 has one cell: t = 1 for every A'
            sure_in[0, 0], sure_out[0, 0] = True, False
        si = sure_in[i_idx, j_idx].astype(np.float64)
        maybe = (~sure_out[i_idx, j_idx]).astype(np.float64)
        for idx, out in ((r_idx, cd), (j_idx, cv)):
            lo = np.bincount(idx, weights=si, minlength=L)
            hi = np.bincount(idx, weights=maybe, minlength=L)
            out[m] = (lo / length >= mu) | (hi / length < mu)
    return cd, cv


def certain_selection(x, rel, ab, alpha, rows, band=0):
    """Scores x (float64 [n, S], mass units) and a bound |x' - x| <= rel * x + ab on another computation
    of them: per pattern, whether sa_select_patterns decides it the same way for every such x'.

    With U = T_all - ceil(alpha * T_all) (the mass allowed to stay uncovered; T_all = rows), a
    pattern is dropped exactly when the mass of all patterns scoring at or below it, itself
    included, fits in U (and always when its score is 0).  The interval bounds of that sum decide
    which patterns are sure either way.  Patterns x < band are kept for every x'."""
    x = np.asarray(x, dtype=np.float64)
    n, S = x.shape
    t_all = float(rows)
    U = t_all - np.ceil(alpha * t_all * 4294967296.0) / 4294967296.0
    sure = np.zeros((n, S), bool)
    for h in range(n):
        v = x[h]
        lo = np.maximum(v * (1 - rel) - ab, 0.0)
        hi = v * (1 + rel) + ab
        # largest possible bottom sum of p: every y whose low end can be <= p's high end, at its high end
        o_lo = np.sort(lo)
        c_hi = np.concatenate([[0.0], np.cumsum(hi[np.argsort(lo)])])
        bmax = c_hi[np.searchsorted(o_lo, hi, side="right")]
        # smallest possible bottom sum: p itself plus every y whose high end is <= p's low end, at its low end
        o_hi = np.sort(hi)
        c_lo = np.concatenate([[0.0], np.cumsum(lo[np.argsort(hi)])])
        bmin = c_lo[np.searchsorted(o_hi, lo, side="right")]
        bmin = np.maximum(bmin, lo)   # p's own low end is always in its bottom sum
        zero = hi <= 0.0
        sure[h] = zero | (bmax <= U) | ((bmin > U) & (lo > 0.0))
        sure[h, :band] = True
    return sure
