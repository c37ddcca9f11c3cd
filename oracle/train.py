"""Backward of the SLA2 attention forward (the training path), written out in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

SLA2 (Italian summary) section 2 and (Arabic summary) section 2: the model is fine-tuned with the
sparse-linear attention in place, so the attention needs gradients with respect to Q, K, V and
the mixing vector alpha.  The router's HardTop-k has no gradient and its differentiable training
form (SoftTop-k) is not specified by the pages, so the kept sets are an input here; the QAT
reading (SLA2 Arabic summary section 2.jim: low-bit forward, backward on the unquantised values)
makes the backward that of the unquantised forward.

Forward (sla.forward_head): per query row t of block i with kept set S_i and the rest U_i,
  sparse  p_tn = exp(q_t k_n / sqrt(d) - L_t) over the tokens n of S_i, O_s = sum_n p_tn v_n;
  linear  A_i = sum_{U_i} phi(K_j)^T V_j, zeta_i = sum_{U_i} phi(K_j)^T 1, phi = ReLU,
          O_l = phi(q_t) A_i / (phi(q_t) . zeta_i)   (0 when U_i is empty or the denominator is 0);
  O = alpha_t O_s + (1 - alpha_t) O_l.

Backward, given dO (the chain rule written out; readings: the derivative of ReLU at 0 is 0, and a
row whose linear branch is defined as 0 (empty U_i or zero denominator) passes no gradient
through it):
  dalpha_t = dO_t . (O_s,t - O_l,t);  dO_s = alpha dO;  dO_l = (1 - alpha) dO
  sparse  dv_n += p_tn dO_s,t;  dp_tn = dO_s,t . v_n;  D_t = dO_s,t . O_s,t;
          ds_tn = p_tn (dp_tn - D_t);  dq_t += sum_n ds_tn k_n / sqrt(d);  dk_n += ds_tn q_t / sqrt(d)
  linear  g_t = dO_l,t / den_t;  e_t = -g_t . O_l,t  (the gradient of the denominator);
          dphi(q_t) = g_t A_i^T + e_t zeta_i;  dq_t += dphi(q_t) [q_t > 0];
          dA_i = sum_{t in i} phi(q_t)^T g_t;  dzeta_i = sum_{t in i} e_t phi(q_t);
          dh_j = sum_{i: j in U_i} dA_i;  dz_j = sum_{i: j in U_i} dzeta_i;
          dv_n += phi(k_n) dh_j;  dk_n += (dh_j v_n + dz_j) [k_n > 0]   (n in block j).
"""

from __future__ import annotations

import numpy as np

from .sla import _f64, block_ranges

__all__ = ["backward_head", "backward"]


def backward_head(Q, K, V, idx, alpha, dO, block: int = 64):
    """Gradients of one head: returns (dQ, dK, dV [N, d], dalpha [N]) in float64.

    Q, K, V, dO [N, d]; idx [n_b, k] kept blocks per query block (ascending); alpha [N].
    """
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    dO = _f64(dO)
    alpha = _f64(alpha)
    idx = np.asarray(idx)
    N, d = Q.shape
    starts, ends, _ = block_ranges(N, block)
    n_b = len(starts)
    scale = 1.0 / np.sqrt(d)
    pK = np.maximum(K, 0.0)
    pQ = np.maximum(Q, 0.0)
    h = np.stack([pK[a:b].T @ V[a:b] for a, b in zip(starts, ends)])  # [n_b, d, d]
    z = np.stack([pK[a:b].sum(axis=0) for a, b in zip(starts, ends)])  # [n_b, d]
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    dalpha = np.zeros(N)
    dh = np.zeros_like(h)
    dz = np.zeros_like(z)
    for i in range(n_b):
        a, b = starts[i], ends[i]
        q, g_o, al = Q[a:b], dO[a:b], alpha[a:b, None]
        sel = np.asarray(idx[i], dtype=np.int64)
        keep = np.zeros(n_b, dtype=bool)
        keep[sel] = True
        uns = np.flatnonzero(~keep)
        # sparse branch
        if len(sel):
            tok = np.concatenate([np.arange(starts[j], ends[j]) for j in sel])
            x = (q @ K[tok].T) * scale
            p = np.exp(x - x.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o_s = p @ V[tok]
            dos = al * g_o
            dV[tok] += p.T @ dos
            dp = dos @ V[tok].T
            D = (dos * o_s).sum(axis=1, keepdims=True)
            ds = p * (dp - D)
            dQ[a:b] += (ds @ K[tok]) * scale
            dK[tok] += (ds.T @ q) * scale
        else:
            o_s = np.zeros_like(q)
        # linear branch
        o_l = np.zeros_like(q)
        if len(uns):
            A = h[uns].sum(axis=0)
            zeta = z[uns].sum(axis=0)
            pq = pQ[a:b]
            num = pq @ A
            den = pq @ zeta
            live = den != 0.0
            o_l[live] = num[live] / den[live, None]
            g = np.zeros_like(q)
            g[live] = ((1.0 - al) * g_o)[live] / den[live, None]
            e = -(g * o_l).sum(axis=1)
            dphi = g @ A.T + e[:, None] * zeta[None, :]
            dQ[a:b] += dphi * (q > 0.0)
            dA = pq.T @ g
            dzeta = pq.T @ e
            dh[uns] += dA[None]
            dz[uns] += dzeta[None]
        dalpha[a:b] = (g_o * (o_s - o_l)).sum(axis=1)
    for j, (a, b) in enumerate(zip(starts, ends)):
        dV[a:b] += pK[a:b] @ dh[j]
        dK[a:b] += (V[a:b] @ dh[j].T + dz[j][None, :]) * (K[a:b] > 0.0)
    return dQ, dK, dV, dalpha


def backward(Q, K, V, idx, alpha, dO, block: int = 64):
    """Gradients over [B, H, N, d] inputs; returns (dQ, dK, dV [B, H, N, d], dalpha [B, H, N])."""
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    dO = _f64(dO)
    alpha = _f64(alpha)
    idx = np.asarray(idx)
    B, H, N, d = Q.shape
    dQ, dK, dV = (np.empty((B, H, N, d)) for _ in range(3))
    da = np.empty((B, H, N))
    for bb in range(B):
        for hh in range(H):
            dQ[bb, hh], dK[bb, hh], dV[bb, hh], da[bb, hh] = backward_head(
                Q[bb, hh], K[bb, hh], V[bb, hh], idx[bb, hh], alpha[bb, hh], dO[bb, hh], block)
    return dQ, dK, dV, da
