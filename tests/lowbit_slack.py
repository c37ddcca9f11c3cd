"""Flip-aware comparison of a low-bit sparse branch with the oracle's (alpha = 1).

A P code is the nearest grid point of y = P^ / sP.  Two correct implementations that form y in
different precisions (the oracle in float64; a kernel in fp32 with a hardware exp2) round it to
different neighbours where y lies within their difference of a midpoint between grid points,
and each such flip moves its output row by one grid step times sP times |v| over the
denominator.  The bound charges one step to every P entry whose y lies within a relative eps of
a midpoint, plus a relative tol of the row's magnitude sum_n P^_n |v_n| / sum P^ for the
rounding of the scales, the exponentials and the denominator.

eps and tol have a floor (EPS_CODE, TOL_SCALE: a few fp32 ulp of y and of the exponent
argument) and, for e4m3, a term for the fp8 matrix product.  Its fp32 accumulation of 128
code products carries an error of at most (n - 1) u sum_k |q_k k_k| with u = 2^-23 (any
summation order, round to nearest or toward zero), i.e. 2^-16 T with T = sum_k |q_k k_k| /
sqrt(d) / ln 2 in log2 units.  An entry's exponent S - m moves by at most that for its own
score plus its row's maximum, and its tile scale by that of the tile maximum, so
eps = EPS_CODE + ln 2 * 2^-16 (T_n + T_row + T_tile) and tol = TOL_SCALE + 3 ln 2 * 2^-16 max T.
int8 products are exact integers (no term).

Another reading of the P step (a per-row or per-query-block scale, a dequantised denominator,
a running maximum) changes codes far from any midpoint and breaks the bound on many elements,
which the acceptance bar on the relative L2 error cannot see (the readings lie 1.3e-3 to 3e-2
apart there, while fp32 flips alone reach about 1e-3).
"""

from __future__ import annotations

import numpy as np

EPS_CODE = 6e-5
TOL_SCALE = 5e-5
ACC_FP8 = 2.0 ** -16  # fp32 accumulation of 128 e4m3 products, relative to sum |q_k k_k|


def grid_step(y: np.ndarray, fmt: str) -> np.ndarray:
    """Spacing of the code grid around non-negative y: 1 for int8; for e4m3 2^(e - 3) in the
    binade [2^e, 2^(e+1)) of a normal value and 2^-9 below 2^-6 (subnormals)."""
    if fmt == "int8":
        return np.ones_like(y)
    _, ex = np.frexp(np.maximum(y, 2.0 ** -6))  # y = m 2^ex, m in [0.5, 1): binade ex - 1
    return np.where(y < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, ex - 4))


def near_midpoint(y: np.ndarray, fmt: str, eps=EPS_CODE):
    """(mask of entries within a relative eps (a scalar or an array like y) of a rounding
    midpoint, grid step)."""
    step = grid_step(y, fmt)
    r = y / step
    return np.abs((r - np.floor(r)) - 0.5) * step <= eps * y, step


def slack_rows(trace, Vd, starts, ends, q_blocks, fmt: str, Qd=None, Kd=None):
    """Per query block in q_blocks: (slack [r_i, d], tolerance [r_i, d]) from the oracle's trace
    of (query block, key block, P^ tile, sP), the dequantised V of the head and, for e4m3, the
    dequantised Q and K (for the accumulation term)."""
    by_block = {}
    for i, j, p, sP in trace:
        by_block.setdefault(i, []).append((j, p, sP))
    acc = ACC_FP8 if fmt == "fp8" else 0.0
    out = []
    for i in q_blocks:
        tiles = by_block.get(i, [])
        r = ends[i] - starts[i]
        slack = np.zeros((r, Vd.shape[1]))
        mag = np.zeros((r, Vd.shape[1]))
        den = np.zeros((r, 1))
        T = []
        for j, p, sP in tiles:
            if acc:
                d = Qd.shape[1]
                T.append((np.abs(Qd[starts[i]:ends[i]]) @ np.abs(Kd[starts[j]:ends[j]]).T) / np.sqrt(d) / np.log(2.0))
            else:
                T.append(np.zeros_like(p))
        t_row = np.max([t.max(axis=1) for t in T], axis=0)[:, None] if tiles else np.zeros((r, 1))
        t_all = max([float(t.max()) for t in T], default=0.0)
        for (j, p, sP), t in zip(tiles, T):
            av = np.abs(Vd[starts[j]:ends[j]])
            den += p.sum(axis=1, keepdims=True)
            mag += p @ av
            if sP > 0:
                eps = EPS_CODE + np.log(2.0) * acc * (t + t_row + t.max())
                amb, step = near_midpoint(p / sP, fmt, eps)
                slack += (amb * step * sP) @ av
        if tiles:
            slack /= den
            mag /= den
        out.append((slack, (TOL_SCALE + 3.0 * np.log(2.0) * acc * t_all) * mag))
    return out


def check_within_slack(got: np.ndarray, ref: np.ndarray, slack: np.ndarray, tol: np.ndarray) -> dict:
    """Largest excess of |got - ref| over slack + tol (<= 0 when inside the bound), and how many
    elements carry a flip allowance."""
    excess = np.abs(got - ref) - (slack + tol)
    return {"excess": float(excess.max()) if excess.size else 0.0,
            "violations": int((excess > 0).sum()),
            "flip_elems": int((slack > 0).sum()),
            "elems": int(excess.size)}
