"""SoftTop-k router and the stage-1 fit of the SLA2 training path, written out in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

SLA2 (Italian summary) section 2.B and (Arabic summary) section 2.ba: during training the router
uses a differentiable SoftTop-k to build the mask M, so that gradients reach proj_q and proj_k;
inference switches to HardTop-k.  (Arabic summary) section 2.dal: stage 1 trains the router R
and the mixing ratio alpha with an MSE loss against full-attention outputs, SoftTop-k letting
the gradient flow; stage 2 fine-tunes end to end with HardTop-k.

The pages do not define SoftTop-k.  Reading used here: the logistic relaxation of the per-row
top-k threshold, M_ij = sigmoid((s_ij - tau_i) / T), with tau_i chosen so that sum_j M_ij = k
(a continuous top-k whose mask keeps the row's budget of k blocks; as T -> 0 it tends to the
HardTop-k mask).  Its gradient follows by implicit differentiation of the budget constraint:
with sigma'_ij = M_ij (1 - M_ij),
    ds_ij = (sigma'_ij / T) (dM_ij - sum_l dM_il sigma'_il / sum_l sigma'_il).
k = 0 gives M = 0 and k = n_b gives M = 1 (no gradient).

The soft mask enters the forward the way the hard mask does, as a per-(query block, key block)
weight: the sparse branch weighs each key of block j by M_ij and the linear branch by 1 - M_ij,
    O_s(q) = sum_n M_{i,b(n)} e^{x_qn} v_n / sum_n M_{i,b(n)} e^{x_qn},  x_qn = q . k_n / sqrt(d),
    O_l(q) = phi(q) sum_j (1 - M_ij) h_j / phi(q) . sum_j (1 - M_ij) z_j,
    O = alpha O_s + (1 - alpha) O_l,
which is the HardTop-k forward when M is 0/1 (O_s := 0 when its weights sum to 0; O_l := 0 when
its denominator is 0, as in the hard forward).

Stage 1 (this module's stage1_grads): loss L = mean over (b, h, token, channel) of (O - O_full)^2
with O_full = softmax(Q K^T / sqrt(d)) V, minimised over proj_q, proj_k and alpha.  Router
scores as in the hard router: s_ij = (Qbar_i Wq) . (Kbar_j Wk) / sqrt(d).
"""

from __future__ import annotations

import numpy as np

from .sla import _f64, block_ranges, pool_blocks

__all__ = [
    "soft_topk",
    "soft_topk_backward",
    "soft_route",
    "forward_soft_head",
    "forward_soft",
    "backward_soft_head",
    "backward_soft",
    "router_backward",
    "full_attention",
    "stage1_loss",
    "stage1_grads",
]


def _sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def soft_topk(s, k: int, T: float) -> np.ndarray:
    """M = sigmoid((s - tau) / T) along the last axis, tau per row with sum_j M_j = k (bisection
    in float64 to the last bit of tau).  s [..., n]; returns M with the shape of s."""
    s = _f64(s)
    n = s.shape[-1]
    if k <= 0:
        return np.zeros_like(s)
    if k >= n:
        return np.ones_like(s)
    lo = s.min(axis=-1, keepdims=True) - 60.0 * T  # sum M = n - tiny  > k
    hi = s.max(axis=-1, keepdims=True) + 60.0 * T  # sum M = tiny      < k
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        tot = _sigmoid((s - mid) / T).sum(axis=-1, keepdims=True)
        above = tot > k  # the threshold is too low: raise it
        lo = np.where(above, mid, lo)
        hi = np.where(above, hi, mid)
    return _sigmoid((s - 0.5 * (lo + hi)) / T)


def soft_topk_backward(M, dM, T: float, k: int) -> np.ndarray:
    """ds for dM through soft_topk (implicit gradient of the budget constraint); 0 for the
    degenerate k = 0 and k = n (constant masks)."""
    M = _f64(M)
    dM = _f64(dM)
    n = M.shape[-1]
    if k <= 0 or k >= n:
        return np.zeros_like(M)
    sp = M * (1.0 - M)
    tot = sp.sum(axis=-1, keepdims=True)
    corr = np.where(tot > 0, (dM * sp).sum(axis=-1, keepdims=True) / np.where(tot > 0, tot, 1.0), 0.0)
    return (sp / T) * (dM - corr)


def soft_route(Q, K, Wq, Wk, topk: int, T: float, block: int = 64) -> dict:
    """Pooled projections, scores and the SoftTop-k mask over [B, H, N, d]."""
    qbar = pool_blocks(Q, block)
    kbar = pool_blocks(K, block)
    qt = qbar @ _f64(Wq)
    kt = kbar @ _f64(Wk)
    d = qt.shape[-1]
    s = (qt @ np.swapaxes(kt, -1, -2)) / np.sqrt(d)
    return {"qbar": qbar, "kbar": kbar, "qt": qt, "kt": kt, "s": s, "M": soft_topk(s, topk, T)}


def forward_soft_head(Q, K, V, M, alpha, block: int = 64):
    """Soft-mask forward of one head: Q, K, V [N, d], M [n_b, n_b], alpha [N].  Returns
    (O, O_s, O_l, L_s, den) with the row normalisers L_s = sum_n w_n e^{x_qn - m_q} (m_q the row's
    maximum) and den = phi(q) . zeta_i, for the backward."""
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    M = _f64(M)
    alpha = _f64(alpha)
    N, d = Q.shape
    starts, ends, _ = block_ranges(N, block)
    bid = np.arange(N) // block  # block of every token
    n_b = len(starts)
    pK = np.maximum(K, 0.0)
    h = np.stack([pK[a:b].T @ V[a:b] for a, b in zip(starts, ends)])  # [n_b, d, dv]
    z = np.stack([pK[a:b].sum(axis=0) for a, b in zip(starts, ends)])  # [n_b, d]
    O = np.zeros((N, V.shape[1]))
    Os = np.zeros_like(O)
    Ol = np.zeros_like(O)
    Ls = np.zeros(N)
    den = np.zeros(N)
    for i in range(n_b):
        a, b = starts[i], ends[i]
        q = Q[a:b]
        w = M[i][bid]  # weight of every key
        x = (q @ K.T) / np.sqrt(d)
        m = x.max(axis=1, keepdims=True)
        e = w[None, :] * np.exp(x - m)
        tot = e.sum(axis=1, keepdims=True)
        os_ = np.where(tot > 0, (e @ V) / np.where(tot > 0, tot, 1.0), 0.0)
        A = np.tensordot(1.0 - M[i], h, axes=(0, 0))  # [d, dv]
        zeta = (1.0 - M[i]) @ z  # [d]
        pq = np.maximum(q, 0.0)
        dn = pq @ zeta
        nz = dn != 0
        ol = np.zeros((b - a, V.shape[1]))
        ol[nz] = (pq[nz] @ A) / dn[nz, None]
        al = alpha[a:b, None]
        O[a:b] = al * os_ + (1.0 - al) * ol
        Os[a:b] = os_
        Ol[a:b] = ol
        Ls[a:b] = tot[:, 0]
        den[a:b] = dn
    return O, Os, Ol, Ls, den


def forward_soft(Q, K, V, M, alpha, block: int = 64):
    """Soft-mask forward over [B, H, N, d] with M [B, H, n_b, n_b]; returns (O, O_s, O_l)."""
    Q = _f64(Q)
    B, H, N, _ = Q.shape
    out = [np.empty((B, H, N, V.shape[-1])) for _ in range(3)]
    for bb in range(B):
        for hh in range(H):
            o, os_, ol, _, _ = forward_soft_head(Q[bb, hh], K[bb, hh], V[bb, hh], M[bb, hh], _f64(alpha)[bb, hh], block)
            out[0][bb, hh], out[1][bb, hh], out[2][bb, hh] = o, os_, ol
    return tuple(out)


def backward_soft_head(Q, K, V, M, alpha, dO, block: int = 64):
    """dM [n_b, n_b] and dalpha [N] of one head (Q, K, V are inputs of the fit, not trained).

    With g = dO, O_s = sum_n w_n e^{x_n} v_n / L_s:
      dM_ij (sparse) = sum_{q in i, n in j} alpha_q e^{x_qn} (g_q . v_n - g_q . O_s,q) / L_s,q;
    with O_l = phi(q) T_i / den, T_i = sum_j (1 - M_ij) h_j, zeta_i = sum_j (1 - M_ij) z_j:
      dT_i = sum_q phi(q)^T (1 - alpha_q) g_q / den_q,
      dzeta_i = -sum_q phi(q) (1 - alpha_q) (g_q . O_l,q) / den_q,
      dM_ij (linear) = -(<dT_i, h_j> + dzeta_i . z_j);
    dalpha_q = g_q . (O_s,q - O_l,q).  Rows with a zero linear denominator pass nothing through
    the linear branch (it is defined as 0 there)."""
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    M = _f64(M)
    alpha = _f64(alpha)
    dO = _f64(dO)
    N, d = Q.shape
    starts, ends, _ = block_ranges(N, block)
    bid = np.arange(N) // block  # block of every token
    n_b = len(starts)
    _, Os, Ol, Ls, den = forward_soft_head(Q, K, V, M, alpha, block)
    pK = np.maximum(K, 0.0)
    h = np.stack([pK[a:b].T @ V[a:b] for a, b in zip(starts, ends)])
    z = np.stack([pK[a:b].sum(axis=0) for a, b in zip(starts, ends)])
    dM = np.zeros((n_b, n_b))
    dalpha = (dO * (Os - Ol)).sum(axis=1)
    for i in range(n_b):
        a, b = starts[i], ends[i]
        q = Q[a:b]
        g = dO[a:b]
        al = alpha[a:b]
        x = (q @ K.T) / np.sqrt(d)
        m = x.max(axis=1, keepdims=True)
        ex = np.exp(x - m)  # unweighted
        ok = Ls[a:b] > 0
        gv = g @ V.T  # g_q . v_n
        D = (g * Os[a:b]).sum(axis=1)
        coef = np.where(ok, al / np.where(ok, Ls[a:b], 1.0), 0.0)
        contrib = (ex * (gv - D[:, None])) * coef[:, None]  # [r, N]
        dM[i] += np.array([contrib[:, s_:e_].sum() for s_, e_ in zip(starts, ends)])
        dn = den[a:b]
        nz = dn != 0
        pq = np.maximum(q, 0.0)
        gl = np.zeros_like(g)
        gl[nz] = ((1.0 - al[nz])[:, None] * g[nz]) / dn[nz, None]
        dT = pq.T @ gl  # [d, dv]
        dzeta = -(pq * (gl * Ol[a:b]).sum(axis=1)[:, None]).sum(axis=0)
        dM[i] -= np.tensordot(h, dT, axes=([1, 2], [0, 1])) + z @ dzeta
    return dM, dalpha


def backward_soft(Q, K, V, M, alpha, dO, block: int = 64):
    """dM [B, H, n_b, n_b] and dalpha [B, H, N] over [B, H, N, d]."""
    Q = _f64(Q)
    B, H, N, _ = Q.shape
    nb = -(-N // block)
    dM = np.empty((B, H, nb, nb))
    dal = np.empty((B, H, N))
    for bb in range(B):
        for hh in range(H):
            dM[bb, hh], dal[bb, hh] = backward_soft_head(Q[bb, hh], K[bb, hh], V[bb, hh], _f64(M)[bb, hh],
                                                         _f64(alpha)[bb, hh], _f64(dO)[bb, hh], block)
    return dM, dal


def router_backward(qbar, kbar, qt, kt, ds):
    """dWq, dWk [d, d] for ds [B, H, n_b, n_b] through s = (qbar Wq)(kbar Wk)^T / sqrt(d), summed
    over every (b, h) (one projection is shared by all heads)."""
    d = qt.shape[-1]
    dqt = (ds @ kt) / np.sqrt(d)
    dkt = (np.swapaxes(ds, -1, -2) @ qt) / np.sqrt(d)
    dWq = np.einsum("bhic,bhie->ce", qbar, dqt)
    dWk = np.einsum("bhjc,bhje->ce", kbar, dkt)
    return dWq, dWk


def full_attention(Q, K, V):
    """softmax(Q K^T / sqrt(d)) V over [B, H, N, d], float64."""
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    x = (Q @ np.swapaxes(K, -1, -2)) / np.sqrt(Q.shape[-1])
    p = np.exp(x - x.max(axis=-1, keepdims=True))
    return (p / p.sum(axis=-1, keepdims=True)) @ V


def stage1_loss(Q, K, V, Wq, Wk, alpha, topk: int, T: float, O_full, block: int = 64) -> float:
    """The stage-1 MSE of the soft-mask forward against O_full."""
    r = soft_route(Q, K, Wq, Wk, topk, T, block)
    O, _, _ = forward_soft(Q, K, V, r["M"], alpha, block)
    return float(np.mean((O - _f64(O_full)) ** 2))


def stage1_grads(Q, K, V, Wq, Wk, alpha, topk: int, T: float, O_full, block: int = 64) -> dict:
    """Loss and its gradients with respect to proj_q, proj_k and alpha (stage 1): the soft
    router, the soft-mask forward, dO = 2 (O - O_full) / count, the soft backward, SoftTop-k's
    implicit gradient, the router's projection gradient."""
    r = soft_route(Q, K, Wq, Wk, topk, T, block)
    O, _, _ = forward_soft(Q, K, V, r["M"], alpha, block)
    diff = O - _f64(O_full)
    dO = 2.0 * diff / diff.size
    dM, dalpha = backward_soft(Q, K, V, r["M"], alpha, dO, block)
    ds = soft_topk_backward(r["M"], dM, T, topk)
    dWq, dWk = router_backward(r["qbar"], r["kbar"], r["qt"], r["kt"], ds)
    return {"loss": float(np.mean(diff ** 2)), "dWq": dWq, "dWk": dWk, "dalpha": dalpha, "dM": dM,
            "ds": ds, "M": r["M"], "O": O}
