"""SVOO online bidirectional Q-K co-clustering ahead of blocking, written out in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): tests, smoke() and bench.py's cpu_baseline
leg may use it; the HIP library never does.

Source: "Training-Free Sparse Attention for Fast Video Generation via Offline Layer-Wise Sparsity
Profiling and Online Bidirectional Co-Clustering" (SVOO), Italian summary
(gist.science/it/paper/2603.18636), section 2.B: queries and keys are partitioned jointly by an
alternating procedure - keys go to the cluster whose current query centroid they have the
highest affinity with, then queries go to the cluster whose updated key centroid they have the
highest affinity with - so that tokens sharing a block share attention preferences; the result
is reused over several diffusion steps.

Readings where the page is silent (each listed with its reason in the design notes):
  * C = n_b clusters (one per 64-token block of the original order), so that cutting the
    cluster-sorted sequence into 64-token blocks keeps the block count of the unpermuted path;
  * the initial centroids are the block means of Q and K in the original order (the router's
    pooling); the key centroids of that start are used only by clusters that receive no key in
    the first pass;
  * affinity is the inner product (the attention logit without the 1/sqrt(d) factor, which does
    not change an argmax); among equal affinities the lower cluster index wins;
  * one iteration is the key step followed by the query step, each recomputing its centroids
    as the plain mean of the members; a cluster left empty keeps its previous centroid; the
    number of iterations is a parameter;
  * the permutation is the stable sort of the tokens by cluster index (clusters in index order,
    original order inside a cluster); Q and alpha follow the query permutation, K and V the key
    permutation; the path then runs unchanged on the permuted tensors and its output rows are
    scattered back to the original query order.
"""

from __future__ import annotations

import numpy as np

from .sla import _f64, forward, pool_blocks, route

__all__ = ["svoo_assign", "svoo_centroids", "svoo_cocluster_head", "svoo_cocluster", "svoo_order",
           "svoo_forward"]


def svoo_assign(X, cent):
    """Nearest cluster of every row of X by inner-product affinity (SVOO section 2.B).

    X [N, d], cent [C, d].  Returns (assign int64 [N], margin float64 [N]): the index of the
    largest x . c (the lower index among equals) and its lead over the second largest (+inf
    when C == 1).
    """
    X = _f64(X)
    cent = _f64(cent)
    aff = X @ cent.T
    assign = np.argmax(aff, axis=1)  # the first maximum: the lower index among equals
    if cent.shape[0] == 1:
        return assign, np.full(X.shape[0], np.inf)
    top2 = -np.partition(-aff, 1, axis=1)[:, :2]
    return assign, top2[:, 0] - top2[:, 1]


def svoo_centroids(X, assign, prev):
    """Mean of each cluster's member rows; an empty cluster keeps its row of prev."""
    X = _f64(X)
    out = np.array(_f64(prev), copy=True)
    for c in range(out.shape[0]):
        members = X[assign == c]
        if len(members):
            out[c] = members.sum(axis=0) / len(members)
    return out


def svoo_cocluster_head(Q, K, iters: int, block: int = 64, trace=None):
    """Alternating co-clustering of one head's queries and keys (SVOO section 2.B).

    Q, K [N, d].  Returns (q_assign, k_assign) int64 [N] with C = n_b clusters.  If trace is a
    list, one dict per iteration is appended: the centroids each step used, the assignments and
    the margins (lead of the best affinity over the second).
    """
    if iters < 1:
        raise ValueError("at least one iteration")
    Q = _f64(Q)
    K = _f64(K)
    q_cent = pool_blocks(Q, block)
    k_cent = pool_blocks(K, block)
    for _ in range(iters):
        k_assign, k_margin = svoo_assign(K, q_cent)  # keys by the current query centroids
        k_used = q_cent
        k_cent = svoo_centroids(K, k_assign, k_cent)
        q_assign, q_margin = svoo_assign(Q, k_cent)  # queries by the updated key centroids
        q_used = k_cent
        q_cent = svoo_centroids(Q, q_assign, q_cent)
        if trace is not None:
            trace.append({"k_assign": k_assign, "k_margin": k_margin, "k_used": k_used,
                          "q_assign": q_assign, "q_margin": q_margin, "q_used": q_used})
    return q_assign, k_assign


def svoo_cocluster(Q, K, iters: int, block: int = 64):
    """Co-clustering over [B, H, N, d]; returns (q_assign, k_assign) int64 [B, H, N]."""
    Q = _f64(Q)
    K = _f64(K)
    B, H, N, _ = Q.shape
    qa = np.empty((B, H, N), dtype=np.int64)
    ka = np.empty((B, H, N), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            qa[b, h], ka[b, h] = svoo_cocluster_head(Q[b, h], K[b, h], iters, block)
    return qa, ka


def svoo_order(assign):
    """The permutation of a cluster assignment: position -> original token, the stable sort of
    the tokens by cluster index (over the last axis)."""
    return np.argsort(np.asarray(assign), axis=-1, kind="stable")


def svoo_forward(Q, K, V, Wq, Wk, alpha, topk: int, perm_q, perm_k, block: int = 64):
    """The SLA2 forward on co-clustered blocks: gather Q and alpha by perm_q and K, V by perm_k,
    route and run the forward on the permuted sequence, scatter the output rows back.

    Inputs [B, H, N, d] (alpha [B, H, N]); perm_q, perm_k [B, H, N] position -> token.
    Returns (O [B, H, N, d] in the original query order, idx of the permuted blocks).
    """
    Q, K, V, alpha = (_f64(x) for x in (Q, K, V, alpha))
    pq = np.asarray(perm_q, dtype=np.int64)
    pk = np.asarray(perm_k, dtype=np.int64)
    Qp = np.take_along_axis(Q, pq[..., None], axis=2)
    Kp = np.take_along_axis(K, pk[..., None], axis=2)
    Vp = np.take_along_axis(V, pk[..., None], axis=2)
    ap = np.take_along_axis(alpha, pq, axis=2)
    idx = route(Qp, Kp, Wq, Wk, topk, block)["idx"]
    Op = forward(Qp, Kp, Vp, idx, ap, block)[0]
    O = np.empty_like(Op)
    np.put_along_axis(O, pq[..., None], Op, axis=2)  # row p of the permuted output is token pq[p]
    return O, idx
