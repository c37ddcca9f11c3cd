"""PISA (piecewise sparse attention) inference forward, written out in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): tests, smoke() and bench.py's cpu_baseline
leg may use it; the HIP library never does.

Source: "PISA - Piecewise Sparse Attention per Efficient Diffusion Transformers", Italian technical
summary (gist.science/it/paper/2602.01077), section 2 (Metodologia): the core algorithm with its
numerator formula, the covariance-aware top-k, and the three-phase kernel outline.

The method, per head and per query block i with kept KV blocks S_i and the rest U_i, per query
row t (logits x = q k^T / sqrt(d)):
  * exact terms over S_i: sum_n e^{x_tn} v_n in the numerator, sum_n e^{x_tn} in the denominator;
  * a zero-order term per unselected block from its key centroid kbar_j and value sum:
    alpha_tj = e^{q_t kbar_j^T / sqrt(d)}, numerator alpha_tj * sum_n v_n;
  * one global first-order correction: (q_t / sqrt(d)) Hbar * sum_{j in U_i} alpha_tj, where Hbar
    is the mean over all blocks of the per-block first-order matrices H_j;
  * o_t = N_t / D_t.

Readings where the page is silent (each listed with its reason in the design notes):
  * the page's formula carries no softmax scale; q_t there stands for q_t / sqrt(d), the scale of
    ordinary attention, in every term (exact, alpha and the first-order correction);
  * H_j is the first-order Taylor term of block j around its centroid,
    H_j = sum_n (k_n - kbar_j)^T v_n  [d_k x d_v], kbar_j the mean of the block's valid keys;
  * D_t follows from the same expansion: exact terms over S_i plus sum_{j in U_i} r_j alpha_tj
    (r_j = the block's token count); its first-order term sum_n (k_n - kbar_j) is identically 0;
  * the max subtraction of a practical softmax rescales N_t and D_t alike and cancels;
  * M_j = ||H_j - Hbar|| is the Frobenius norm (the 2-norm of the matrix's entries); it bounds the
    operator 2-norm from above, so ||q (H_j - Hbar)|| <= ||q|| M_j still holds;
  * the covariance-aware score of block j for query block i is the first-order error bound of
    approximating block j, e^{s_ij} M_j with s_ij = qbar_i . kbar_j / sqrt(d) (qbar_i the mean
    query of block i), ranked as s_ij + ln M_j; the row-constant factor ||qbar_i|| / sqrt(d) drops
    out of a per-row ranking.  HardTop-k as in the SLA2 router (ties to the lower index, ascending
    indices).
"""

from __future__ import annotations

import numpy as np

from .sla import _f64, block_ranges, hard_topk, pool_blocks

__all__ = ["pisa_block_stats", "pisa_cov_norms", "pisa_route", "pisa_forward_head", "pisa_forward"]


def pisa_block_stats(K, V, block: int) -> dict:
    """Per-block statistics of one head's keys and values (the pre-computation phase).

    PISA (Italian summary) section 2, hardware implementation step 1: block centroids, value sums
    and the global statistic Hbar; core algorithm: Hbar is the mean over all blocks of the
    per-block first-order matrices.  K [N, d_k], V [N, d_v].

    Returns {'centroid' [n_b, d_k], 'vsum' [n_b, d_v], 'count' [n_b], 'H' [n_b, d_k, d_v],
    'Hbar' [d_k, d_v]} in float64.
    """
    K = _f64(K)
    V = _f64(V)
    starts, ends, counts = block_ranges(K.shape[0], block)
    n_b = len(starts)
    centroid = np.empty((n_b, K.shape[1]))
    vsum = np.empty((n_b, V.shape[1]))
    H = np.empty((n_b, K.shape[1], V.shape[1]))
    for j, (a, b) in enumerate(zip(starts, ends)):
        centroid[j] = K[a:b].mean(axis=0)
        vsum[j] = V[a:b].sum(axis=0)
        H[j] = (K[a:b] - centroid[j]).T @ V[a:b]
    return {"centroid": centroid, "vsum": vsum, "count": counts.astype(np.float64), "H": H,
            "Hbar": H.mean(axis=0)}


def pisa_cov_norms(H, Hbar) -> np.ndarray:
    """M_j = ||H_j - Hbar|| (Frobenius), the covariance norm of each block.

    PISA (Italian summary) section 2, covariance-aware routing.  H [n_b, d_k, d_v].
    """
    D = _f64(H) - _f64(Hbar)[None]
    return np.sqrt((D * D).sum(axis=(1, 2)))


def pisa_route(Q, K, V, topk: int, block: int = 64, covariance: bool = True) -> dict:
    """Covariance-aware HardTop-k for one head.

    PISA (Italian summary) section 2, covariance-aware routing: the selection score of a block
    combines its attention score with its covariance norm; blocks whose zero-order approximation
    with the global first-order correction would be worst are computed exactly.  Scores:
    s_ij = qbar_i . kbar_j / sqrt(d); selection score s_ij + ln M_j (covariance=True) or s_ij.

    Returns {'idx' int32 [n_b, k], 'mask' uint8 [n_b, n_b], 'scores' s, 'select' the ranked
    score, 'M' [n_b], 'stats' (pisa_block_stats)}.
    """
    Q = _f64(Q)
    st = pisa_block_stats(K, V, block)
    qbar = pool_blocks(Q, block)
    s = (qbar @ st["centroid"].T) / np.sqrt(Q.shape[1])
    M = pisa_cov_norms(st["H"], st["Hbar"])
    if covariance:
        with np.errstate(divide="ignore"):
            sel = s + np.log(M)[None, :]
    else:
        sel = s
    idx, mask = hard_topk(sel, topk)
    return {"idx": idx, "mask": mask, "scores": s, "select": sel, "M": M, "stats": st}


def pisa_forward_head(Q, K, V, idx, block: int = 64, q_blocks=None, stats=None):
    """PISA output rows of one head for the listed query blocks.

    PISA (Italian summary) section 2, core algorithm: o_t = N_t / D_t with exact terms over the
    kept blocks, the per-block zero-order term over the others, and the global first-order
    correction with Hbar (numerator formula of that section; the denominator by the same
    expansion, see the module docstring).  Q, K, V [N, d]; idx [n_b, k].

    Returns a list of [r_i, d_v] float64 arrays in the order of q_blocks (default: all).
    """
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    idx = np.asarray(idx)
    N, d = Q.shape
    starts, ends, _ = block_ranges(N, block)
    n_b = len(starts)
    st = stats if stats is not None else pisa_block_stats(K, V, block)
    kbar, vsum, cnt, Hbar = st["centroid"], st["vsum"], st["count"], st["Hbar"]
    scale = 1.0 / np.sqrt(d)
    if q_blocks is None:
        q_blocks = range(n_b)
    outs = []
    for i in q_blocks:
        a, b = starts[i], ends[i]
        q = Q[a:b] * scale  # the softmax scale folded into q
        sel = np.asarray(idx[i], dtype=np.int64)
        keep = np.zeros(n_b, dtype=bool)
        keep[sel] = True
        uns = np.flatnonzero(~keep)
        tok = np.concatenate([np.arange(starts[j], ends[j]) for j in sel]) if len(sel) else np.zeros(0, np.int64)
        x = q @ K[tok].T  # exact logits over the kept tokens
        y = q @ kbar[uns].T  # centroid logits of the unselected blocks
        m = np.full(b - a, -np.inf)
        if x.size:
            m = np.maximum(m, x.max(axis=1))
        if y.size:
            m = np.maximum(m, y.max(axis=1))
        e = np.exp(x - m[:, None])
        al = np.exp(y - m[:, None])  # alpha_tj, shifted by the same m
        num = e @ V[tok] + al @ vsum[uns] + (q @ Hbar) * al.sum(axis=1, keepdims=True)
        den = e.sum(axis=1) + al @ cnt[uns]
        outs.append(num / den[:, None])
    return outs


def pisa_forward(Q, K, V, idx, block: int = 64):
    """PISA forward over [B, H, N, d] inputs with idx [B, H, n_b, k]; returns O [B, H, N, d_v]."""
    Qa = _f64(Q)
    Ka = _f64(K)
    Va = _f64(V)
    idx = np.asarray(idx)
    B, H, N, _ = Qa.shape
    O = np.empty((B, H, N, Va.shape[-1]))
    for b in range(B):
        for h in range(H):
            O[b, h] = np.concatenate(pisa_forward_head(Qa[b, h], Ka[b, h], Va[b, h], idx[b, h], block), axis=0)
    return O
