"""Test inputs: seeded draws from ``gen`` plus the router score-gap guarantee.

The HardTop-k mask is compared bit for bit, which is only meaningful when the k-th and
(k+1)-th block scores of every row are separated by more than the GPU's fp32 rounding.  The
inputs therefore promise a gap of at least ``GAP`` between them, measured on the oracle's
float64 pre-softmax scores of the stored (rounded) inputs.  Rows that miss it get their query
block's noise redrawn until they pass.  Only the rows' own query blocks change (a score-map row
depends on its query block and on every key block, and keys are never touched).
"""

from __future__ import annotations

import concurrent.futures

import numpy as np
import torch

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


def enforce_gap(inputs: dict, gap: float = GAP, ks=None) -> dict:
    """Redraw failing query blocks in place until every row's k-th/(k+1)-th score gap is at
    least `gap` for every k in `ks` (default: the workload's topk).  Returns statistics."""
    wl = inputs["workload"]
    Wq = inputs["Wq"].double().numpy()
    Wk = inputs["Wk"].double().numpy()
    ks = [wl.topk] if ks is None else list(ks)
    blk = wl.block

    def row_gaps(s):
        return np.min([_row_gaps(s, k) for k in ks], axis=0)

    def one_head(bh):
        b, h = divmod(bh, wl.H)
        kt = oracle.pool_blocks(inputs["K"][b, h], blk) @ Wk
        s = (oracle.pool_blocks(inputs["Q"][b, h], blk) @ Wq @ kt.T) / np.sqrt(wl.d)
        g = row_gaps(s)
        bad = np.nonzero(g < gap)[0]
        redrawn, tries, attempt = len(bad), 0, 0
        while len(bad):
            attempt += 1
            tries += len(bad)
            if attempt > MAX_TRIES:
                raise RuntimeError(f"score gap not reached for head ({b},{h}) rows {bad[:8]}")
            gen.redraw_query_blocks(inputs, b, h, bad, attempt)
            # the failing blocks' rows back to back (only the last block can be short, and it
            # comes last), so pooling them in 64-row groups gives each block's mean
            qrows = torch.cat([inputs["Q"][b, h, i * blk : (i + 1) * blk] for i in bad])
            s[bad] = (oracle.pool_blocks(qrows, blk) @ Wq @ kt.T) / np.sqrt(wl.d)
            g[bad] = row_gaps(s[bad])
            bad = bad[g[bad] < gap]
        return redrawn, tries, float(g.min())

    with concurrent.futures.ThreadPoolExecutor(max_workers=gen.workers()) as ex:
        res = list(ex.map(one_head, range(wl.B * wl.H)))
    return {
        "rows_redrawn": sum(r[0] for r in res),
        "tries": sum(r[1] for r in res),
        "min_gap": min(r[2] for r in res),
    }


def make_case(name_or_wl, seed: int = 0, gap: bool = True, ks=None, **overrides) -> dict:
    wl = gen.workload(name_or_wl, **overrides) if isinstance(name_or_wl, str) else name_or_wl
    inputs = gen.draw(wl, seed)
    inputs["gap_stats"] = enforce_gap(inputs, ks=ks) if gap else None
    return inputs
