"""Brute-force steps at 50 significant digits with explicit loops (mpmath).

Test infrastructure: a second, independent statement of each step on tiny 2-D
and 1-D inputs, written element by element from the definitions (row and column
means as loops, the factored estimate entry by entry), used to pin the vectorised
fp64 oracle. It imports nothing from the oracle or the library.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import mpmath as mp

mp.mp.dps = 50

Mat = List[List[mp.mpf]]


def _to_mat(a) -> Mat:
    """2-D numpy array or nested list -> list of rows of mpf (exact binary64 values)."""
    return [[mp.mpf(float(v)) for v in row] for row in a]


def _rms(m: Mat) -> mp.mpf:
    n = sum(len(r) for r in m)
    return mp.sqrt(mp.fsum(v * v for r in m for v in r) / n)


def _row_means(m: Mat) -> List[mp.mpf]:
    return [mp.fsum(r) / len(r) for r in m]


def _col_means(m: Mat) -> List[mp.mpf]:
    h, w = len(m), len(m[0])
    return [mp.fsum(m[i][j] for i in range(h)) / h for j in range(w)]


def _estimate(row: List[mp.mpf], col: List[mp.mpf]) -> Mat:
    mean_row = mp.fsum(row) / len(row)
    return [[row[i] * col[j] / mean_row for j in range(len(col))] for i in range(len(row))]


def adafactor(x, g, st: Dict, t: int, *, factored: bool, eps=(1e-30, 1e-3), d=1.0,
              decay=-0.8, beta1: Optional[float] = None, wd=0.0, scale=True, lr=None,
              warmup=False):
    """x, g: 2-D (for 1-D pass one row and factored=False). st holds mpf lists."""
    X, G = _to_mat(x), _to_mat(g)
    h, w = len(X), len(X[0])
    e1, e2 = mp.mpf(eps[0]), mp.mpf(eps[1])
    if lr is None:
        cap = mp.mpf("1e-6") * t if warmup else mp.mpf("0.01")
        rho = min(cap, 1 / mp.sqrt(t))
    else:
        rho = mp.mpf(lr)
    alpha = rho * (max(e2, _rms(X)) if scale else 1)
    b2 = 1 - mp.power(t, mp.mpf(decay))
    Q = [[G[i][j] ** 2 + e1 for j in range(w)] for i in range(h)]
    new = {}
    if factored:
        rm, cm = _row_means(Q), _col_means(Q)
        row = [b2 * st["row"][i] + (1 - b2) * rm[i] for i in range(h)]
        col = [b2 * st["col"][j] + (1 - b2) * cm[j] for j in range(w)]
        new["row"], new["col"] = row, col
        V = _estimate(row, col)
    else:
        V = [[b2 * st["v"][0][j] + (1 - b2) * Q[0][j] for j in range(w)]]
        new["v"] = V
    U = [[G[i][j] / mp.sqrt(V[i][j]) for j in range(w)] for i in range(h)]
    k = max(mp.mpf(1), _rms(U) / d)
    U = [[alpha * U[i][j] / k for j in range(w)] for i in range(h)]
    if beta1 is not None:
        b1 = mp.mpf(beta1)
        M = [[b1 * st["m"][i][j] + (1 - b1) * U[i][j] for j in range(w)] for i in range(h)]
        new["m"] = M
        D = M
    else:
        D = U
    Xn = [[X[i][j] - mp.mpf(wd) * alpha * X[i][j] - D[i][j] for j in range(w)] for i in range(h)]
    return Xn, new


def came(x, g, st: Dict, t: int, *, factored: bool, lr=2e-4, eps=(1e-30, 1e-16), d=1.0,
         betas=(0.9, 0.999, 0.9999), wd=0.0):
    X, G = _to_mat(x), _to_mat(g)
    h, w = len(X), len(X[0])
    e1, e2 = mp.mpf(eps[0]), mp.mpf(eps[1])
    b1, b2, b3 = (mp.mpf(b) for b in betas)
    Q = [[G[i][j] ** 2 + e1 for j in range(w)] for i in range(h)]
    new = {}
    if factored:
        rm, cm = _row_means(Q), _col_means(Q)
        row = [b2 * st["row"][i] + (1 - b2) * rm[i] for i in range(h)]
        col = [b2 * st["col"][j] + (1 - b2) * cm[j] for j in range(w)]
        new["row"], new["col"] = row, col
        V = _estimate(row, col)
    else:
        V = [[b2 * st["v"][0][j] + (1 - b2) * Q[0][j] for j in range(w)]]
        new["v"] = V
    U = [[G[i][j] / mp.sqrt(V[i][j]) for j in range(w)] for i in range(h)]
    k = max(mp.mpf(1), _rms(U) / d)
    U = [[U[i][j] / k for j in range(w)] for i in range(h)]
    M = [[b1 * st["m"][i][j] + (1 - b1) * U[i][j] for j in range(w)] for i in range(h)]
    new["m"] = M
    if factored:
        E = [[(U[i][j] - M[i][j]) ** 2 + e2 for j in range(w)] for i in range(h)]
        rm, cm = _row_means(E), _col_means(E)
        rrow = [b3 * st["rrow"][i] + (1 - b3) * rm[i] for i in range(h)]
        rcol = [b3 * st["rcol"][j] + (1 - b3) * cm[j] for j in range(w)]
        new["rrow"], new["rcol"] = rrow, rcol
        S = _estimate(rrow, rcol)
        D = [[M[i][j] / mp.sqrt(S[i][j]) for j in range(w)] for i in range(h)]
    else:
        D = M
    lr_ = mp.mpf(lr)
    Xn = [[X[i][j] - lr_ * mp.mpf(wd) * X[i][j] - lr_ * D[i][j] for j in range(w)]
          for i in range(h)]
    return Xn, new


def lamb(x, g, st: Dict, t: int, *, lr=1e-3, betas=(0.9, 0.999), eps=1e-6, wd=0.01, bc=True):
    X, G = _to_mat(x), _to_mat(g)
    h, w = len(X), len(X[0])
    b1, b2 = mp.mpf(betas[0]), mp.mpf(betas[1])
    M = [[b1 * st["m"][i][j] + (1 - b1) * G[i][j] for j in range(w)] for i in range(h)]
    V = [[b2 * st["v"][i][j] + (1 - b2) * G[i][j] ** 2 for j in range(w)] for i in range(h)]
    c1 = (1 - b1 ** t) if bc else mp.mpf(1)
    c2 = (1 - b2 ** t) if bc else mp.mpf(1)
    D = [[(M[i][j] / c1) / (mp.sqrt(V[i][j] / c2) + mp.mpf(eps)) + mp.mpf(wd) * X[i][j]
          for j in range(w)] for i in range(h)]
    xn = mp.sqrt(mp.fsum(v * v for r in X for v in r))
    dn = mp.sqrt(mp.fsum(v * v for r in D for v in r))
    tr = xn / dn if (xn > 0 and dn > 0) else mp.mpf(1)
    Xn = [[X[i][j] - mp.mpf(lr) * tr * D[i][j] for j in range(w)] for i in range(h)]
    return Xn, {"m": M, "v": V}
