"""Test inputs: seeded draws from ``gen`` plus the router score-gap guarantee.

The HardTop-k mask is compared bit for bit, which is only meaningful when the k-th and
(k+1)-th block scores of every row are separated by more than the GPU's fp32 rounding.  The
inputs therefore promise a gap of at least ``GAP`` between them, measured on the oracle's
float64 pre-softmax scores of the stored (rounded) inputs.  Rows that miss it get their query
block's noise redrawn until they pass.  Only the rows' own query blocks change (a score-map row
depends on its query block and on every key block, and keys are never touched).
"""

from __future__ import annotations

import numpy as np

import gen
import oracle

GAP = 1e-3
MAX_TRIES = 10_000


def _row_gaps(s: np.ndarray, k: int) -> np.ndarray:
    """s [n_b, n_b] -> gap between the k-th and (k+1)-th largest entry of each row."""
    if k <= 0 or k >= s.shape[-1]:
        return np.full(s.shape[0], np.inf)
    part = -np.partition(-s, (k - 1, k), axis=-1)
    return part[:, k - 1] - part[:, k]


def enforce_gap(inputs: dict, gap: float = GAP) -> dict:
    """Redraw failing query blocks in place; returns statistics {'rows_redrawn', 'tries'}."""
    wl = inputs["workload"]
    Wq = inputs["Wq"].double().numpy()
    Wk = inputs["Wk"].double().numpy()
    k = wl.topk
    stats = {"rows_redrawn": 0, "tries": 0, "min_gap": np.inf}
    blk = wl.block
    for b in range(wl.B):
        for h in range(wl.H):
            kt = oracle.pool_blocks(inputs["K"][b, h], blk) @ Wk
            s = (oracle.pool_blocks(inputs["Q"][b, h], blk) @ Wq @ kt.T) / np.sqrt(wl.d)
            g = _row_gaps(s, k)
            bad = np.nonzero(g < gap)[0]
            stats["rows_redrawn"] += len(bad)
            attempt = 0
            while len(bad):
                attempt += 1
                stats["tries"] += len(bad)
                if attempt > MAX_TRIES:
                    raise RuntimeError(f"score gap not reached for head ({b},{h}) rows {bad[:8]}")
                gen.redraw_query_blocks(inputs, b, h, bad, attempt)
                rows = np.stack(
                    [oracle.pool_blocks(inputs["Q"][b, h, i * blk : (i + 1) * blk], blk)[0] for i in bad]
                )
                s[bad] = (rows @ Wq @ kt.T) / np.sqrt(wl.d)
                g[bad] = _row_gaps(s[bad], k)
                bad = bad[g[bad] < gap]
            stats["min_gap"] = min(stats["min_gap"], float(g.min()))
    return stats


def make_case(name_or_wl, seed: int = 0, gap: bool = True, **overrides) -> dict:
    wl = gen.workload(name_or_wl, **overrides) if isinstance(name_or_wl, str) else name_or_wl
    inputs = gen.draw(wl, seed)
    inputs["gap_stats"] = enforce_gap(inputs) if gap else None
    return inputs
