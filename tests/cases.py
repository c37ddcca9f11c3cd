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
import threadpoolctl
import torch

import gen
import oracle

GAP = 1e-3
MAX_ROUNDS = 200
CHUNK = 64  # failing blocks screened together
SCREEN = 1.02  # screening margin on the candidate mean (rounding moves scores by ~1e-5)


def _row_gaps(s: np.ndarray, k: int) -> np.ndarray:
    """s [n_b, n_b] -> gap between the k-th and (k+1)-th largest entry of each row."""
    if k <= 0 or k >= s.shape[-1]:
        return np.full(s.shape[0], np.inf)
    part = -np.partition(-s, (k - 1, k), axis=-1)
    return part[:, k - 1] - part[:, k]


def enforce_gap(inputs: dict, gap: float = GAP, ks=None, log=None) -> dict:
    """Redraw failing query blocks in place until every row's k-th/(k+1)-th score gap is at
    least `gap` for every k in `ks` (default: the workload's topk).

    A block's score row depends on its tokens only through their mean, so candidates are
    screened on their noise mean (the centre part plus noise_std times the candidate mean,
    screen margin SCREEN x gap); the first passing candidate is realised as tokens and accepted
    only if the oracle's exact float64 scores of the rounded tokens meet the gap.
    Returns statistics."""
    wl = inputs["workload"]
    Wq = inputs["Wq"].double().numpy()
    Wk = inputs["Wk"].double().numpy()
    ks = [wl.topk] if ks is None else list(ks)
    blk = wl.block
    sd = gen.noise_std(wl)

    def row_gaps(s):
        return np.min([_row_gaps(s, k) for k in ks], axis=0)

    def one_head(bh):
        b, h = divmod(bh, wl.H)
        kt = oracle.pool_blocks(inputs["K"][b, h], blk) @ Wk
        s = (oracle.pool_blocks(inputs["Q"][b, h], blk) @ Wq @ kt.T) / np.sqrt(wl.d)
        A = (Wq @ kt.T) / np.sqrt(wl.d)  # a candidate mean's score row is qbar @ A
        g = row_gaps(s)
        bad = np.nonzero(g < gap)[0]
        redrawn, tries, attempt = len(bad), 0, 0
        centre = {}
        while len(bad):
            attempt += 1
            if attempt > MAX_ROUNDS:
                raise RuntimeError(f"score gap not reached for head ({b},{h}) rows {bad[:8]}")
            count = min(16 * 2 ** attempt, 256)
            still = []
            for c0 in range(0, len(bad), CHUNK):
                rows = bad[c0 : c0 + CHUNK]
                for i in rows:
                    if i not in centre:
                        centre[i] = oracle.pool_blocks(gen.query_block_centres(inputs, b, h, int(i)), blk)[0]
                m = gen.query_noise_means(inputs, b, h, rows, attempt, count, c0 // CHUNK)
                cs = np.stack([centre[i] for i in rows]) @ A  # [rows, n_b]
                sc = cs[:, None, :] + sd * (m.reshape(-1, wl.d).astype(np.float64) @ A).reshape(len(rows), count, -1)
                gc = row_gaps(sc.reshape(-1, sc.shape[-1])).reshape(len(rows), count)
                chosen, means = [], []
                for n, i in enumerate(rows):
                    ok = np.nonzero(gc[n] >= SCREEN * gap)[0]
                    tries += count if len(ok) == 0 else int(ok[0]) + 1
                    if len(ok) == 0:
                        still.append(i)
                    else:
                        chosen.append(i)
                        means.append(m[n, ok[0]])
                if not chosen:
                    continue
                chosen = np.asarray(chosen, dtype=np.int64)
                gen.realize_query_blocks(inputs, b, h, chosen, np.stack(means), attempt, c0 // CHUNK)
                # exact check on the rounded tokens: the chosen blocks back to back (only the
                # last block can be short and it comes last), pooled in 64-row groups
                q = torch.cat([inputs["Q"][b, h, i * blk : (i + 1) * blk] for i in chosen])
                sn = (oracle.pool_blocks(q, blk) @ Wq @ kt.T) / np.sqrt(wl.d)
                gn = row_gaps(sn)
                s[chosen], g[chosen] = sn, gn
                still.extend(chosen[gn < gap].tolist())
            bad = np.asarray(still, dtype=np.int64)
        return redrawn, tries, float(g.min())

    # heads run in parallel threads, each with single-threaded BLAS
    with threadpoolctl.threadpool_limits(1), concurrent.futures.ThreadPoolExecutor(max_workers=gen.workers()) as ex:
        res = []
        for n, r in enumerate(ex.map(one_head, range(wl.B * wl.H))):
            res.append(r)
            if log and (n + 1) % 8 == 0:
                log(f"gap repair: {n + 1}/{wl.B * wl.H} heads done")
    return {
        "rows_redrawn": sum(r[0] for r in res),
        "tries": sum(r[1] for r in res),
        "min_gap": min(r[2] for r in res),
    }


def make_case(name_or_wl, seed: int = 0, gap: bool = True, ks=None, log=None, **overrides) -> dict:
    wl = gen.workload(name_or_wl, **overrides) if isinstance(name_or_wl, str) else name_or_wl
    inputs = gen.draw(wl, seed)
    if log:
        log(f"drawn {wl.name}")
    inputs["gap_stats"] = enforce_gap(inputs, ks=ks, log=log) if gap else None
    if log:
        log(f"gap stats {inputs['gap_stats']}")
    return inputs
