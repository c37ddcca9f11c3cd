"""SLA2 inference forward, written out in float64 from its definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): tests, smoke() and bench.py's cpu_baseline
leg may use it; the HIP library never does.

Notation (shared with the pages): a head's tokens are split into blocks of ``block`` adjacent
tokens; block t holds tokens [t*block, min((t+1)*block, N)) and r_t of them.  sel(i) is the set
of KV blocks the router keeps for query block i, U(i) the rest.  phi(x) = max(x, 0).

Readings where the pages are silent (each is listed with its reason in the design notes):
  * blocks are contiguous in the given token order, the same blocking for queries and keys,
    and the last block may be short (its mean is over its valid tokens only);
  * the projections act as y = x @ W with W[d_in][d_out], no bias, one W shared by all heads;
  * block scores are s_ij = q~_i . k~_j / sqrt(d); HardTop-k keeps the k largest per row, ties
    broken towards the lower block index, and the kept indices are listed in ascending order;
  * the sparse branch is softmax(q k^T / sqrt(d)) renormalised over the kept tokens;
  * the linear branch uses phi = ReLU on the raw q and k (the SALAD kernel function), the same
    Q, K, V as the sparse branch, and is normalised over U(i) with no epsilon; an empty U(i) or a
    zero denominator gives 0;
  * alpha is one value per (batch, head, query token).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "block_ranges",
    "pool_blocks",
    "router_scores",
    "hard_topk",
    "route",
    "block_states",
    "forward_head",
    "forward",
    "branch_drops",
    "forward_dropped",
    "dense_P",
]


def _f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or a CPU torch tensor (bf16, fp32, ...) to float64."""
    if hasattr(x, "detach"):  # torch tensor: bf16 has no numpy dtype, go through fp32 (exact)
        import torch

        x = x.detach().to("cpu")
        if x.dtype in (torch.bfloat16, torch.float16):
            x = x.to(torch.float32)
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def block_ranges(N: int, block: int):
    """Token ranges of the blocks of adjacent tokens.

    SLA2 (Italian summary) section 2.B and SLA2 (Arabic summary) section 2.ba: Q and K are
    mean-pooled over blocks of adjacent tokens before routing.  Returns (starts, ends, counts)
    as int64 arrays of length n_b = ceil(N / block); the last block may hold fewer tokens.
    """
    if N < 1 or block < 1:
        raise ValueError("N and block must be positive")
    n_b = -(-N // block)
    starts = np.arange(n_b, dtype=np.int64) * block
    ends = np.minimum(starts + block, N)
    return starts, ends, ends - starts


def pool_blocks(X, block: int) -> np.ndarray:
    """Mean of each block's valid rows: X [..., N, d] -> [..., n_b, d] (float64).

    SLA2 (Italian summary) section 2.B: mean pooling of Q and K over adjacent-token blocks.
    """
    X = _f64(X)
    N = X.shape[-2]
    starts, ends, counts = block_ranges(N, block)
    out = np.empty(X.shape[:-2] + (len(starts), X.shape[-1]), dtype=np.float64)
    for t, (a, b) in enumerate(zip(starts, ends)):
        out[..., t, :] = X[..., a:b, :].sum(axis=-2) / float(b - a)
    return out


def router_scores(Q, K, Wq, Wk, block: int) -> np.ndarray:
    """Compressed block-score map s [..., n_b, n_b] before the row softmax.

    SLA2 (Italian summary) section 2.B and (Arabic summary) section 2.ba: pooled Q and K go
    through the learnable projections proj_q and proj_k, which produce a compressed attention
    score map.  Reading: q~ = mean(Q_i) @ Wq, k~ = mean(K_j) @ Wk, s_ij = q~_i . k~_j / sqrt(d).
    """
    Wq = _f64(Wq)
    Wk = _f64(Wk)
    qt = pool_blocks(Q, block) @ Wq
    kt = pool_blocks(K, block) @ Wk
    d = qt.shape[-1]
    return (qt @ np.swapaxes(kt, -1, -2)) / np.sqrt(d)


def hard_topk(s: np.ndarray, k: int):
    """Inference-time HardTop-k over the last axis of s.

    SLA2 (Italian summary) section 2.B and (Arabic summary) section 2.dal: training uses a
    differentiable SoftTop-k, inference a hard top-k; the router's output is the mask M.
    Reading: per row keep the k largest entries, prefer the lower index among equal scores, and
    list the kept indices in ascending order.  Returns (idx int32 [..., n_b, k],
    mask uint8 [..., n_b, n_b]).
    """
    n = s.shape[-1]
    if not 0 <= k <= n:
        raise ValueError(f"top-k {k} outside [0, {n}]")
    # a stable sort of -s keeps equal scores in index order, so the lower index wins a tie
    order = np.argsort(-s, axis=-1, kind="stable")[..., :k]
    idx = np.sort(order, axis=-1).astype(np.int32)
    mask = np.zeros(s.shape, dtype=np.uint8)
    np.put_along_axis(mask, idx.astype(np.int64), 1, axis=-1)
    return idx, mask


def route(Q, K, Wq, Wk, topk: int, block: int = 64) -> dict:
    """The router: pool -> project -> score map -> row softmax -> HardTop-k.

    SLA2 (Italian summary) section 2.B; (Arabic summary) section 2.ba.  The router reads Q and K
    only, never V.  Returns a dict with 'idx', 'mask', 'scores' (pre-softmax s) and 'probs'
    (the row softmax of s, the compressed attention map).
    """
    s = router_scores(Q, K, Wq, Wk, block)
    idx, mask = hard_topk(s, topk)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    probs = e / e.sum(axis=-1, keepdims=True)
    return {"idx": idx, "mask": mask, "scores": s, "probs": probs}


def block_states(K, V, block: int):
    """Per-KV-block linear-attention states of one head.

    SALAD section 2: linear attention with a ReLU kernel function phi.  For block j:
    h_j = phi(K_j)^T V_j [d x d] and z_j = phi(K_j)^T 1 [d].  K, V: [N, d].
    Returns h [n_b, d, d], z [n_b, d].
    """
    K = _f64(K)
    V = _f64(V)
    starts, ends, _ = block_ranges(K.shape[0], block)
    d_k, d_v = K.shape[1], V.shape[1]
    h = np.empty((len(starts), d_k, d_v))
    z = np.empty((len(starts), d_k))
    for j, (a, b) in enumerate(zip(starts, ends)):
        pk = np.maximum(K[a:b], 0.0)
        h[j] = pk.T @ V[a:b]
        z[j] = pk.sum(axis=0)
    return h, z


def forward_head(Q, K, V, idx, alpha, block: int = 64, q_blocks=None, states=None):
    """SLA2 output rows of one head for the listed query blocks.

    Q, K, V [N, d]; idx [n_b, k] kept KV blocks per query block; alpha [N].
    Returns (O, O_s, O_l), each a list of [r_i, d] float64 arrays in the order of q_blocks
    (default: every query block).

    * Sparse branch (SLA2 Italian summary sections 1 and 2.A; Arabic summary sections 1 and
      2.alef): exact softmax attention over the tokens of the kept blocks only, renormalised over
      that set; O_s = 0 when nothing is kept.
    * Linear branch (SALAD section 2 for phi = ReLU; SLA2 section 1 for "the rest"): the sum runs
      directly over the unselected blocks U(i): A_i = sum_{j in U(i)} h_j,
      zeta_i = sum_{j in U(i)} z_j, O_l(q) = phi(q) A_i / (phi(q) . zeta_i); 0 when U(i) is
      empty or the denominator is exactly 0 (the output stays row-normalised, Arabic summary
      section 2.alef).
    * Combine (SLA2 Italian summary section 2.A, Arabic summary section 2.alef):
      O = alpha * O_s + (1 - alpha) * O_l.
    """
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    alpha = _f64(alpha)
    idx = np.asarray(idx)
    N, d = Q.shape
    starts, ends, _ = block_ranges(N, block)
    n_b = len(starts)
    if q_blocks is None:
        q_blocks = range(n_b)
    h, z = states if states is not None else block_states(K, V, block)
    h_flat = h.reshape(n_b, -1)
    scale = 1.0 / np.sqrt(d)
    outs, outs_s, outs_l = [], [], []
    for i in q_blocks:
        a, b = starts[i], ends[i]
        q = Q[a:b]
        sel = np.asarray(idx[i], dtype=np.int64)
        keep = np.zeros(n_b, dtype=bool)
        keep[sel] = True
        # sparse branch: softmax over the tokens of the kept blocks
        if len(sel):
            tok = np.concatenate([np.arange(starts[j], ends[j]) for j in sel])
            logits = (q @ K[tok].T) * scale
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            o_s = (p @ V[tok]) / p.sum(axis=1, keepdims=True)
        else:
            o_s = np.zeros((b - a, V.shape[1]))
        # linear branch: states summed over the unselected blocks directly
        unsel = (~keep).astype(np.float64)
        if unsel.any():
            A = (unsel @ h_flat).reshape(h.shape[1], h.shape[2])
            zeta = unsel @ z
            pq = np.maximum(q, 0.0)
            num = pq @ A
            den = pq @ zeta
            o_l = np.zeros_like(num)
            nz = den != 0.0
            o_l[nz] = num[nz] / den[nz, None]
        else:
            o_l = np.zeros((b - a, V.shape[1]))
        al = alpha[a:b, None]
        outs.append(al * o_s + (1.0 - al) * o_l)
        outs_s.append(o_s)
        outs_l.append(o_l)
    return outs, outs_s, outs_l


def forward(Q, K, V, idx, alpha, block: int = 64):
    """Whole SLA2 forward over [B, H, N, d] inputs (every query block of every head).

    Returns (O, O_s, O_l) as float64 arrays of shape [B, H, N, d].  See forward_head for the
    definition and its sources.
    """
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    alpha = _f64(alpha)
    idx = np.asarray(idx)
    B, H, N, d = Q.shape
    shape = (B, H, N, V.shape[-1])
    O = np.empty(shape)
    Os = np.empty(shape)
    Ol = np.empty(shape)
    for bb in range(B):
        for hh in range(H):
            o, os_, ol = forward_head(
                Q[bb, hh], K[bb, hh], V[bb, hh], idx[bb, hh], alpha[bb, hh], block
            )
            O[bb, hh] = np.concatenate(o)
            Os[bb, hh] = np.concatenate(os_)
            Ol[bb, hh] = np.concatenate(ol)
    return O, Os, Ol


def branch_drops(alpha, tau: float):
    """Which branches a head drops (SALAD section 2, Post-Tuning Branch Dropping: a linear
    branch whose scale is very low is removed at inference).

    In SLA2 the linear branch of query token t is weighted by 1 - alpha_t and the sparse branch
    by alpha_t (SLA2 Italian summary section 2.A).  Reading: per (batch, head), the linear branch
    is dropped when max_t (1 - alpha_t) <= tau and the sparse branch when max_t alpha_t <= tau,
    0 <= tau < 0.5 (so at most one branch of a head is dropped); tau = 0 drops only branches
    whose weight is exactly 0 everywhere.  The threshold is taken as float32, the precision the
    GPU compares in; 1 - alpha is exact in both precisions wherever it can reach tau.
    alpha [B, H, N] -> (drop_linear [B, H] bool, drop_sparse [B, H] bool).
    """
    a = _f64(alpha)
    t = float(np.float32(tau))
    if not 0.0 <= t < 0.5:
        raise ValueError("tau must lie in [0, 0.5)")
    return (1.0 - a).max(axis=-1) <= t, a.max(axis=-1) <= t


def forward_dropped(Q, K, V, idx, alpha, tau: float, block: int = 64):
    """SLA2 forward with branch dropping (see branch_drops): a dropped branch contributes
    nothing, the kept one keeps its weight, O = [alpha O_s] + [(1 - alpha) O_l].
    Returns (O, drop_linear, drop_sparse)."""
    _, Os, Ol = forward(Q, K, V, idx, alpha, block)
    dl, ds = branch_drops(alpha, tau)
    a = _f64(alpha)[..., None]
    O = np.where(ds[..., None, None], 0.0, a * Os) + np.where(dl[..., None, None], 0.0, (1.0 - a) * Ol)
    return O, dl, ds


def dense_P(Q, K, idx, alpha, block: int = 64):
    """Dense token-level mixing matrices of one head, for tiny inputs only.

    SLA2 (Italian summary) section 2.A: the combine matches the decomposition
    P ~ alpha * P_s + (1 - alpha) * P_l.  Built entry by entry from the token-level mask
    (query token q in block i sees key token n in block j through P_s when j is kept, through
    P_l otherwise).  Returns (P, P_s, P_l), each [N, N]; O = P @ V.
    """
    Q = _f64(Q)
    K = _f64(K)
    alpha = _f64(alpha)
    N, d = Q.shape
    starts, ends, _ = block_ranges(N, block)
    blk = np.repeat(np.arange(len(starts)), ends - starts)
    kept = np.zeros((N, N), dtype=bool)
    for q in range(N):
        kept[q] = np.isin(blk, np.asarray(idx[blk[q]]))
    logits = (Q @ K.T) / np.sqrt(d)
    e = np.where(kept, np.exp(logits - np.where(kept, logits, -np.inf).max(axis=1, keepdims=True)), 0.0)
    es = e.sum(axis=1, keepdims=True)
    P_s = np.divide(e, es, out=np.zeros_like(e), where=es > 0)
    w = np.where(kept, 0.0, np.maximum(Q, 0.0) @ np.maximum(K, 0.0).T)
    ws = w.sum(axis=1, keepdims=True)
    P_l = np.divide(w, ws, out=np.zeros_like(w), where=ws > 0)
    a = alpha[:, None]
    return a * P_s + (1.0 - a) * P_l, P_s, P_l
